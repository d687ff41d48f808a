"""Grouped-FFN parity on hand-built expert segment sizes.

The prefill-shaped GEMM runs 256-row tiles; an expert's last tile runs in a
full, half (at most 128 rows) or quarter (at most 64 rows) layout, whole or
as split-K pieces added by a fixup pass.  Routing decides the segment sizes
in the other parity tests, so which layouts they reach is left to chance.
Here each token's single expert is assigned directly, so the segments have
tails on both sides of every layout boundary (1, 63, 64, 65, 127, 128, 129
rows, and the same past whole tiles), and dispatch + grouped FFN run through
the C ABI against the float64 oracle on the same rows.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import mixture_experts_layer_36_amd as moe
import oracle as O
from synth import LayerInputs
from synth.workloads import MIXTRAL_PREFILL, QWEN_FP8_SKEW
from tests.helpers import DeviceLayer, assert_values, from_torch

pytestmark = pytest.mark.gpu

# rows per expert: tails of 1, 63, 64, 65, 127, 128, 129, 0 (whole tiles) rows
COUNTS = np.array([1, 63, 64, 65, 256 + 127, 128, 256 + 129, 512, 256 + 64, 256 + 1])
T = int(COUNTS.sum())  # 2178 tokens, one expert each

# (base workload, d, f, extra): d = 256 keeps every tile whole (8 k-stages, too
# few to split); d = 1024 splits the tiles of the single wave into K-pieces.
SHAPES = {
    "bf16_whole": (MIXTRAL_PREFILL, 256, 384, {}),
    "bf16_split": (MIXTRAL_PREFILL, 1024, 512, {}),
    "fp8w_whole": (QWEN_FP8_SKEW, 256, 384, {}),
    "fp8w_split": (QWEN_FP8_SKEW, 1024, 512, {}),
    "f8d_whole": (QWEN_FP8_SKEW, 512, 384, {"dispatch_fp8": True}),
    "f8d_split": (QWEN_FP8_SKEW, 1024, 512, {"dispatch_fp8": True}),
}


def _case(name, seed=5):
    base, d, f, extra = SHAPES[name]
    E = len(COUNTS)
    w = base.scaled(T=T, d=d, f=f, E=E, k=1, n_group=0, topk_group=0, f_shared=0, **extra)
    L = LayerInputs(w, seed)
    rng = np.random.default_rng(seed)
    idx = rng.permutation(np.repeat(np.arange(E, dtype=np.int32), COUNTS))  # tokens in random expert order
    return w, L, idx


@pytest.mark.parametrize("kblocked", [False, True], ids=["rowmajor", "kblocked"])
@pytest.mark.parametrize("name", list(SHAPES))
def test_grouped_ffn_segment_tails(name, kblocked):
    w, L, idx = _case(name)
    dev = DeviceLayer(L)
    desc = moe.Desc.from_attrs(w)
    w1, w3, w2 = dev.w1, dev.w3, dev.w2
    if kblocked:
        desc.w_layout = moe.W_KBLOCKED
        w1, w3, w2 = moe.pack_weights(w1), moe.pack_weights(w3), moe.pack_weights(w2)
    A = w.T
    topk = torch.from_numpy(idx.reshape(T, 1)).cuda()
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    if w.dispatch_fp8:
        x_perm = torch.empty(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.dispatch(desc, topk, dev.x, counts, offsets, perm, inv, x_perm, moe.workspace(desc, moe.STAGE_DISPATCH))
    h = torch.empty((A, w.f), dtype=dev.x.dtype, device="cuda")
    y = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.grouped_ffn(desc, x_perm, offsets, w1, w3, w2, dev.s1, dev.s3, dev.s2, h, y,
                    moe.workspace(desc, moe.STAGE_FFN))
    torch.cuda.synchronize()

    # the layout the segments were built for (integer work: exact)
    ref_perm = np.argsort(idx, kind="stable").astype(np.int32)
    ref_off = np.concatenate([[0], np.cumsum(COUNTS)]).astype(np.int32)
    assert np.array_equal(counts.cpu().numpy(), COUNTS)
    assert np.array_equal(offsets.cpu().numpy(), ref_off)
    assert np.array_equal(perm.cpu().numpy(), ref_perm)

    x, _, _ = O.decoded_inputs(L)
    if w.dispatch_fp8:
        x = O.dequantize_fp8_blocks(*O.quantize_fp8_blocks(x))
    ref_h, ref_y = O.grouped_ffn(O.gather_rows(x, ref_perm), ref_off, lambda e: O.adapters.decoded_expert(L, e),
                                 w.act)
    assert_values(from_torch(h, w.act), ref_h, w, "h")
    assert_values(from_torch(y, w.act), ref_y, w, "y_perm")
    # each segment on its own rows: a layout mix-up in one tail shows there
    # even when the tensor-wide error is dominated by larger segments
    for e in range(w.E):
        lo, hi = ref_off[e], ref_off[e + 1]
        assert_values(from_torch(y[lo:hi], w.act), ref_y[lo:hi], w, f"y_perm expert {e} ({hi - lo} rows)")
