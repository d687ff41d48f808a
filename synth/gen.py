"""Seeded synthetic inputs for the MoE layer (shared by the tests and the bench).

Every tensor comes from its own counter-free substream
``numpy.random.SeedSequence([seed, TAG, index...])`` so any expert's weights,
or any redrawn token row, can be regenerated alone and in any order.

Recipe (all draws are float32 standard normals):
  * x[t, :]            ~ N(0, 1), then stored in the activation dtype
  * router weight      ~ N(0, 1) / sqrt(d), stored [E][d] (out x in)
  * W1_e, W3_e         ~ N(0, 1) / sqrt(d), stored [f][d] (out x in)
  * W2_e               ~ N(0, 1) / sqrt(f), stored [d][f] (out x in)
  * shared W1s/W3s/W2s   likewise with f_shared
  * e4m3 experts: per output channel (row) s = amax / 448 (1 when amax is 0),
    codes = round-to-nearest-even(w / s) in OCP E4M3, saturated to +-448
  * router bias b_e = -c * ln(rank_e), rank_e = 1 + pi(e), pi a seeded
    permutation of the experts (c = 0: no bias)
  * optional margin redraw: rows that a caller-supplied ``accept`` callback
    rejects are redrawn from substream (seed, X_REDRAW, t, attempt), at most
    64 attempts.

Storage encodings produced here: bf16 as uint16 bit patterns (round to nearest
even from float32), fp32 as float32, e4m3 as uint8 codes + float32 scales.
This module holds none of the layer's arithmetic: whatever decides which rows
to redraw is passed in by the caller.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Callable, Optional

import numpy as np

from .workloads import Workload

TAGS = {
    "x": 1, "x_redraw": 2, "w_router": 3, "w1": 4, "w3": 5, "w2": 6,
    "shared_w1": 7, "shared_w3": 8, "shared_w2": 9, "rank": 10,
}
MAX_REDRAW = 64
E4M3_MAX = 448.0


def substream(seed: int, tag: str, *index: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, TAGS[tag], *index])))


def normal32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def encode_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def encode_act(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return encode_bf16(a32)
    raise ValueError(f"unsupported storage dtype {dtype}")


def quantize_e4m3_rows(w32: np.ndarray):
    """Per-row (output channel) e4m3 quantisation -> (uint8 codes, float32 scales)."""
    import torch  # the OCP E4M3 encoder is torch's float8_e4m3fn cast (RNE)

    amax = np.abs(w32).max(axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    v = np.clip(w32 / scale[:, None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.ascontiguousarray(codes), scale


def _weight(seed, tag, index, rows, cols, fan_in, wdt):
    w32 = normal32(substream(seed, tag, *index), (rows, cols)) * np.float32(1.0 / np.sqrt(fan_in))
    if wdt == "e4m3":
        return quantize_e4m3_rows(w32)
    return encode_act(w32, wdt), None


@dataclass
class ExpertWeights:
    w1: np.ndarray                 # [f][d]
    w3: np.ndarray                 # [f][d]
    w2: np.ndarray                 # [d][f]
    s1: Optional[np.ndarray] = None  # [f]   (e4m3 only)
    s3: Optional[np.ndarray] = None  # [f]
    s2: Optional[np.ndarray] = None  # [d]


class LayerInputs:
    """Inputs of one MoE layer; expert weights are generated on demand."""

    def __init__(self, w: Workload, seed: int,
                 accept: Optional[Callable[["LayerInputs", np.ndarray, np.ndarray], np.ndarray]] = None):
        self.w = w
        self.seed = seed
        self.w_router = _weight(seed, "w_router", (), w.E, w.d, w.d, w.act)[0]
        if w.bias_scale != 0.0:
            perm = substream(seed, "rank").permutation(w.E)
            rank = (perm + 1).astype(np.float64)
            self.bias = (-w.bias_scale * np.log(rank)).astype(np.float32)
        else:
            self.bias = None
        self.x = encode_act(normal32(substream(seed, "x"), (w.T, w.d)), w.act)
        self.redrawn = np.zeros(w.T, dtype=np.int32)  # attempts used per row
        if accept is not None:
            self._redraw(accept)

    def _redraw(self, accept):
        rows = np.arange(self.w.T)
        for attempt in range(1, MAX_REDRAW + 1):
            ok = np.asarray(accept(self, rows, self.x[rows]), dtype=bool)
            rows = rows[~ok]
            if rows.size == 0:
                return
            for t in rows:
                self.x[t] = encode_act(normal32(substream(self.seed, "x_redraw", int(t), attempt),
                                                (self.w.d,)), self.w.act)
                self.redrawn[t] = attempt
        ok = np.asarray(accept(self, rows, self.x[rows]), dtype=bool)
        if not ok.all():
            raise RuntimeError(f"{(~ok).sum()} rows still rejected after {MAX_REDRAW} redraws")

    def expert(self, e: int) -> ExpertWeights:
        w = self.w
        w1, s1 = _weight(self.seed, "w1", (e,), w.f, w.d, w.d, w.wdt)
        w3, s3 = _weight(self.seed, "w3", (e,), w.f, w.d, w.d, w.wdt)
        w2, s2 = _weight(self.seed, "w2", (e,), w.d, w.f, w.f, w.wdt)
        return ExpertWeights(w1, w3, w2, s1, s3, s2)

    def shared(self) -> Optional[ExpertWeights]:
        w = self.w
        if w.f_shared == 0:
            return None
        # the shared expert is stored in the activation dtype
        w1 = _weight(self.seed, "shared_w1", (), w.f_shared, w.d, w.d, w.act)[0]
        w3 = _weight(self.seed, "shared_w3", (), w.f_shared, w.d, w.d, w.act)[0]
        w2 = _weight(self.seed, "shared_w2", (), w.d, w.f_shared, w.f_shared, w.act)[0]
        return ExpertWeights(w1, w3, w2)

    def experts(self, threads: Optional[int] = None, experts=None):
        """Yield (e, ExpertWeights) in expert order, generated by a thread pool."""
        ids = list(range(self.w.E)) if experts is None else list(experts)
        n = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max_workers=n) as pool:
            window = 2 * n
            futs = {}
            for i, e in enumerate(ids):
                futs[i] = pool.submit(self.expert, e)
                if i >= window:
                    j = i - window
                    yield ids[j], futs.pop(j).result()
            for j in sorted(futs):
                yield ids[j], futs.pop(j).result()
