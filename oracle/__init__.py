"""CPU oracle of the MoE layer forward (float64 NumPy).

TEST INFRASTRUCTURE: only the tests, the smoke check and the bench's CPU
baseline import this package.  The HIP product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .adapters import workload_spec, decoded_inputs, margin_acceptor  # noqa: F401
