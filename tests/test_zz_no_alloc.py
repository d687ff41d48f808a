"""moe_dispatch_noalloc (the library's static scratch instead of a caller
workspace) against moe_dispatch with a workspace, through the C ABI: bit for
bit on every output, on calls in a row -- large, then smaller, then with a
capacity and with the fp8 payload -- so the second call runs over the first
call's leftovers in the shared scratch."""
import numpy as np
import pytest
import torch

import mixture_experts_layer_36_amd as moe
from synth.workloads import DSV3_PREFILL_SKEW, QWEN_FP8_SKEW

pytestmark = pytest.mark.gpu


def _topk(T, k, E, seed):
    rng = np.random.default_rng(seed)
    logp = -1.2 * np.log(1.0 + rng.permutation(E))  # skewed expert popularity
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    return torch.from_numpy(np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)).cuda()


def _outputs(w, A):
    counts = torch.full((w.E,), -5, dtype=torch.int32, device="cuda")
    offsets = torch.full((w.E + 1,), -5, dtype=torch.int32, device="cuda")
    perm = torch.full((A,), -5, dtype=torch.int32, device="cuda")
    inv = torch.full((A,), -5, dtype=torch.int32, device="cuda")
    if w.dispatch_fp8:
        xp = torch.zeros(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        xp = torch.zeros((A, w.d), dtype=torch.bfloat16, device="cuda")
    return counts, offsets, perm, inv, xp


# (workload, T, k): 131072 assignments in 1024-chunks (512 KB of scratch),
# then 12000 in 256-chunks, then a capacity, then the fp8 payload; the
# last is below the single-block size (no scratch at all)
CALLS = [(DSV3_PREFILL_SKEW, 16384, 8, 0.0, False), (DSV3_PREFILL_SKEW, 3000, 4, 0.0, False),
         (DSV3_PREFILL_SKEW, 5000, 8, 1.0, False), (QWEN_FP8_SKEW, 2500, 8, 0.0, True),
         (QWEN_FP8_SKEW, 300, 8, 0.0, False)]


def test_noalloc_dispatch_matches_workspace_dispatch():
    for n, (base, T, k, cf, f8) in enumerate(CALLS):
        w = base.scaled(T=T, d=512, k=k, capacity_factor=cf, dispatch_fp8=f8)
        desc = moe.Desc.from_attrs(w)
        A = T * k
        print(f"[noalloc] call {n}: T={T} k={k} E={w.E} cf={cf} fp8={f8}", flush=True)
        idx = _topk(T, k, w.E, seed=100 + n)
        x = torch.randn(T, w.d, device="cuda").to(torch.bfloat16)
        ref = _outputs(w, A)
        moe.dispatch(desc, idx, x, *ref, moe.workspace(desc, moe.STAGE_DISPATCH))
        got = _outputs(w, A)
        moe.dispatch_noalloc(desc, idx, x, *got)
        torch.cuda.synchronize()
        for name, u, v in zip(("counts", "offsets", "perm_token", "inv_pos", "x_perm"), ref, got):
            assert torch.equal(u, v), (n, name)
        assert int(ref[1][-1]) == (A if cf == 0 else int(ref[1][-1]))
        assert int(ref[0].sum()) == A


def test_noalloc_dispatch_rejects_oversize():
    w = DSV3_PREFILL_SKEW.scaled(T=(1 << 20) // 8 + 256, d=512, E=256)  # > 4 MiB of chunk counts
    desc = moe.Desc.from_attrs(w)
    # real (tiny) buffers: the size check returns before anything is enqueued
    b = [torch.zeros(64, dtype=torch.int32, device="cuda") for _ in range(7)]
    with pytest.raises(moe.MoeError) as err:
        moe.dispatch_noalloc(desc, *b)
    assert err.value.status == moe.MOE_ERR_WORKSPACE
    torch.cuda.synchronize()
