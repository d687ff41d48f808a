"""Shared test helpers: device upload of seeded inputs, oracle references and
comparisons with the layer's tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from synth import LayerInputs
from synth.device import DeviceLayer, to_torch  # noqa: F401

# Output tolerances: err = max|gpu - oracle| / max|oracle| over a tensor for
# bf16 activations (2e-2) and fp8 weights (6e-2); absolute max error for fp32.
REL_TOL = {"bf16": 2e-2, "e4m3": 6e-2}
ABS_TOL_F32 = 1e-4
# Gates are fp32 in every dtype; logits differ from float64 by ~1e-6.
GATE_TOL = 2e-5


def from_torch(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> float64 values."""
    t = t.detach().cpu()
    if dtype == "bf16":
        return O.bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def oracle_layer(L: LayerInputs, tokens=None) -> O.LayerResult:
    """Full float64 oracle of the layer (on a token subset when given)."""
    x, wr, b = O.decoded_inputs(L)
    if tokens is not None:
        x = x[tokens]
    cache = {}

    def ew(e):
        if e not in cache:
            cache.clear()
            cache[e] = O.adapters.decoded_expert(L, e)
        return cache[e]

    w = L.w
    cap = O.expert_capacity(getattr(w, "capacity_factor", 0), w.T, w.k, w.E)
    assert tokens is None or cap == 0, "a capacity couples the tokens: no subsets"
    return O.layer_forward(x, wr, b, O.workload_spec(w), w.E, ew, w.act,
                           O.adapters.decoded_shared(L), capacity=cap,
                           fp8_dispatch=getattr(w, "dispatch_fp8", False),
                           overflow=getattr(w, "overflow", "drop"))


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    scale = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / scale) if scale > 0 else float(np.max(np.abs(got)))


def assert_values(got: np.ndarray, ref: np.ndarray, w, what: str) -> float:
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    if w.act == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert err <= ABS_TOL_F32, f"{what}: max abs err {err:.3g} > {ABS_TOL_F32}"
        return err
    tol = REL_TOL[w.wdt if w.wdt == "e4m3" else "bf16"]
    err = rel_err(got, ref) if got.size else 0.0
    assert err <= tol, f"{what}: rel err {err:.3g} > {tol}"
    return err


def assert_rows(got: np.ndarray, ref: np.ndarray, w, what: str) -> float:
    """assert_values row by row: each token's output against the largest
    magnitude of its own oracle row (so a wrong low-magnitude row cannot hide
    behind the tensor's maximum).  Returns the largest row error."""
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    if w.act == "f32":
        return assert_values(got, ref, w, what)
    tol = REL_TOL[w.wdt if w.wdt == "e4m3" else "bf16"]
    scale = np.max(np.abs(ref), axis=1)
    diff = np.max(np.abs(got - ref), axis=1)
    err = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)
    t = int(np.argmax(err))
    assert err[t] <= tol, f"{what}: row {t} rel err {err[t]:.3g} > {tol}"
    return float(err[t])


def assert_routing(idx: np.ndarray, gw: np.ndarray, ref: O.LayerResult):
    """Routing indices bit-exact, position by position (the inputs keep every
    adjacent pair of chosen scores apart, so the order is decided); gates
    within GATE_TOL at each position."""
    T, k = ref.topk_idx.shape
    assert idx.shape == (T, k)
    bad = np.nonzero((idx != ref.topk_idx).any(axis=1))[0]
    assert bad.size == 0, [(int(t), idx[t].tolist(), ref.topk_idx[t].tolist()) for t in bad[:5]]
    err = np.abs(gw.astype(np.float64) - ref.topk_w)
    assert err.max(initial=0.0) <= GATE_TOL, f"gate err {err.max():.3g} at token {np.argmax(err) // k}"


def assert_dispatch(idx, counts, offsets, perm_token, inv_pos, ref: O.LayerResult):
    """Bit-exact dispatch: counts, offsets, perm_token and inv_pos (the
    routing indices are already exact)."""
    assert np.array_equal(counts, ref.counts), "counts"
    assert np.array_equal(offsets, ref.offsets), "offsets"
    n = len(ref.perm_token)  # rows kept (all T*k when dropless)
    assert np.array_equal(perm_token[:n], ref.perm_token), "perm_token"
    assert np.array_equal(inv_pos, ref.inv_pos), "inv_pos"
