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
# Adjacent chosen scores closer than this may come out in either order.
ORDER_TIE = 2e-5


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


def assert_routing(idx: np.ndarray, gw: np.ndarray, ref: O.LayerResult, scores: np.ndarray):
    """Selected expert sets bit-exact; order exact except between adjacent
    chosen experts whose oracle scores are within ORDER_TIE; gates within
    GATE_TOL (compared per expert id)."""
    T, k = ref.topk_idx.shape
    assert idx.shape == (T, k)
    for t in range(T):
        r, g = ref.topk_idx[t], idx[t]
        assert sorted(r) == sorted(g), f"token {t}: experts {g} vs oracle {r}"
        if not np.array_equal(r, g):
            s = scores[t, r.astype(np.int64)]
            for j in range(k):
                if g[j] != r[j]:
                    # the swapped entries must be oracle near-ties
                    jj = int(np.nonzero(r == g[j])[0][0])
                    lo, hi = min(j, jj), max(j, jj)
                    assert np.all(np.abs(np.diff(s[lo:hi + 1])) < ORDER_TIE), \
                        f"token {t}: order {g} vs {r} (scores {s})"
        ref_by_e = dict(zip(r.tolist(), ref.topk_w[t].tolist()))
        for j in range(k):
            assert abs(gw[t, j] - ref_by_e[int(g[j])]) <= GATE_TOL, \
                f"token {t}: gate {gw[t, j]} vs {ref_by_e[int(g[j])]}"


def assert_dispatch(idx, counts, offsets, perm_token, inv_pos, ref: O.LayerResult):
    """Bit-exact dispatch.  Given the same expert sets, counts, offsets and
    perm_token are unique; inv_pos is compared per (token, expert) pair so a
    tolerated order swap within a token's k experts maps consistently."""
    assert np.array_equal(counts, ref.counts), "counts"
    assert np.array_equal(offsets, ref.offsets), "offsets"
    n = len(ref.perm_token)  # rows kept (all T*k when dropless)
    assert np.array_equal(perm_token[:n], ref.perm_token), "perm_token"
    T, k = ref.topk_idx.shape
    got = inv_pos.reshape(T, k)
    want = ref.inv_pos.reshape(T, k)
    og = np.argsort(idx, axis=1, kind="stable")
    orf = np.argsort(ref.topk_idx, axis=1, kind="stable")
    assert np.array_equal(np.take_along_axis(got, og, 1), np.take_along_axis(want, orf, 1)), "inv_pos"
