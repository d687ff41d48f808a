"""Seeded synthetic inputs for the MoE layer; no layer arithmetic lives here."""
from .workloads import ALL, BY_NAME, DEFAULT_SEED, Workload  # noqa: F401
from .gen import LayerInputs, ExpertWeights, encode_bf16, substream  # noqa: F401
