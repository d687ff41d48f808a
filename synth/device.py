"""Upload of seeded inputs to the GPU in the library's storage layout.

Shared by the tests and the bench; holds no layer arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from .gen import LayerInputs


def to_torch(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "e4m3":
        t = torch.from_numpy(np.ascontiguousarray(a))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


class DeviceLayer:
    """Inputs of one layer on the GPU, in the library's storage layout."""

    def __init__(self, L: LayerInputs, device="cuda", threads=None):
        w = L.w
        self.L = L
        self.x = to_torch(L.x, w.act, device)
        self.w_router = to_torch(L.w_router, w.act, device)
        self.bias = None if L.bias is None else torch.from_numpy(L.bias).to(device)
        wdt = w.wdt
        tdt = {"bf16": torch.bfloat16, "e4m3": torch.uint8, "f32": torch.float32}[wdt]
        self.w1 = torch.empty((w.E, w.f, w.d), dtype=tdt, device=device)
        self.w3 = torch.empty((w.E, w.f, w.d), dtype=tdt, device=device)
        self.w2 = torch.empty((w.E, w.d, w.f), dtype=tdt, device=device)
        self.s1 = self.s3 = self.s2 = None
        if wdt == "e4m3":
            self.s1 = torch.empty((w.E, w.f), dtype=torch.float32, device=device)
            self.s3 = torch.empty((w.E, w.f), dtype=torch.float32, device=device)
            self.s2 = torch.empty((w.E, w.d), dtype=torch.float32, device=device)
        for e, ew in L.experts(threads=threads):
            self.w1[e].copy_(to_torch(ew.w1, wdt, "cpu"))
            self.w3[e].copy_(to_torch(ew.w3, wdt, "cpu"))
            self.w2[e].copy_(to_torch(ew.w2, wdt, "cpu"))
            if wdt == "e4m3":
                self.s1[e].copy_(torch.from_numpy(ew.s1))
                self.s3[e].copy_(torch.from_numpy(ew.s3))
                self.s2[e].copy_(torch.from_numpy(ew.s2))
        sh = L.shared()
        self.sw1 = self.sw3 = self.sw2 = None
        if sh is not None:
            self.sw1 = to_torch(sh.w1, w.act, device)
            self.sw3 = to_torch(sh.w3, w.act, device)
            self.sw2 = to_torch(sh.w2, w.act, device)
