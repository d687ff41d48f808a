"""Dispatch around its size switch.

Up to 4096 assignments the index work (histogram, scan, stable scatter) runs
in one single-block kernel; above that, as three kernels over chunks of 256
assignments, of 512 above 16384 and of 1024 above 32768 (up to 128 chunks at
131072).  All must give the oracle's layout exactly.  Expert ids are drawn per token
without replacement from a skewed distribution (Gumbel top-k), so some
experts overflow a capacity; the cases sit on both sides of the switch and
at the small edges, dropless and with a capacity.  The gathered rows are
checked bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_36_amd as moe
import oracle as O
from synth.workloads import MIXTRAL_PREFILL

pytestmark = pytest.mark.gpu

E, D = 64, 256
# (T, k): T*k assignments
SIZES = [(1, 1), (32, 2), (4095, 1), (512, 8), (4097, 1), (1024, 8), (700, 6), (2500, 8), (5000, 8),
         (9001, 8), (16384, 8)]


def _topk(T, k, seed):
    rng = np.random.default_rng(seed)
    logp = -1.2 * np.log(1.0 + rng.permutation(E))  # Zipf-like expert popularity
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


@pytest.mark.parametrize("cf", [0.0, 1.0], ids=["dropless", "cap1.0"])
@pytest.mark.parametrize("T,k", SIZES, ids=[f"{t * k}" for t, k in SIZES])
def test_dispatch_matches_oracle_around_size_switch(T, k, cf):
    w = MIXTRAL_PREFILL.scaled(T=T, d=D, f=256, E=E, k=k, capacity_factor=cf)
    desc = moe.Desc.from_attrs(w)
    idx = _topk(T, k, seed=T * 16 + k)
    cap = O.expert_capacity(cf, T, k, E)
    ref_counts, ref_off, ref_perm, ref_inv = O.dispatch(idx, E, capacity=cap)
    x = torch.randn(T, D, device="cuda").to(torch.bfloat16)
    A = T * k
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((A,), -7, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    x_perm = torch.zeros((A, D), dtype=torch.bfloat16, device="cuda")
    moe.dispatch(desc, torch.from_numpy(idx).cuda(), x, counts, offsets, perm, inv, x_perm,
                 moe.workspace(desc, moe.STAGE_DISPATCH))
    torch.cuda.synchronize()
    n = int(ref_off[-1])
    assert np.array_equal(counts.cpu().numpy(), ref_counts)
    assert np.array_equal(offsets.cpu().numpy(), ref_off)
    assert np.array_equal(inv.cpu().numpy(), ref_inv)
    assert np.array_equal(perm.cpu().numpy()[:n], ref_perm)
    assert torch.equal(x_perm[:n], x[torch.from_numpy(ref_perm).long().cuda()])
    if cf > 0:
        assert (ref_inv < 0).any() or ref_counts.max() <= cap  # the capacity case drops when it must
