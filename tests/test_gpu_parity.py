"""GPU parity of the HIP path against the float64 oracle, through the C ABI.

Sizes here are ones the oracle finishes in seconds while still spanning
several GEMM tiles, ragged segment tails and empty experts.  Routing indices,
counts, offsets and the permutation must be bit-exact; values must be within
the tolerances in tests/helpers.py.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_36_amd as moe
import oracle as O
from synth import LayerInputs
from synth.workloads import (DSV3_DECODE, DSV3_PREFILL_SKEW, MIXTRAL_PREFILL, QWEN_FP8_SKEW,
                             TINY_F32)
from tests.helpers import (GATE_TOL, DeviceLayer, assert_dispatch, assert_routing, assert_values,
                           from_torch, oracle_layer, to_torch)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_f32": TINY_F32,
    "tiny_f32_ragged": TINY_F32.scaled(T=77, d=256, f=384, E=5, k=3),
    "mixtral_small": MIXTRAL_PREFILL.scaled(T=300, d=256, f=384),
    "mixtral_tiles": MIXTRAL_PREFILL.scaled(T=700, d=512, f=640),
    # 256-row direct-to-LDS kernel: ragged tails, K = 3 * 128, N not a multiple of 256
    "mixtral_big_tiles": MIXTRAL_PREFILL.scaled(T=1500, d=384, f=384, E=6),
    "mixtral_big_k128": MIXTRAL_PREFILL.scaled(T=600, d=128, f=128, E=4),
    # 48 tiles per GEMM on 256 compute units: every tile is split along K (4
    # pieces in the gate-up GEMM, 2 in the down GEMM) and summed by the fixup
    "mixtral_big_split": MIXTRAL_PREFILL.scaled(T=1200, d=1024, f=512, E=4),
    # weight-streaming decode kernel (at most 32 rows per expert on average):
    # shared segment over several 32-row token blocks, K below the pipeline depth,
    # shared width different from the routed width
    "dsv3_decode_small": DSV3_DECODE.scaled(T=40, d=512, f=256, E=64, f_shared=256),
    "decode_k128": DSV3_DECODE.scaled(T=24, d=128, f=128, E=16, f_shared=128),
    "decode_shared_wide": DSV3_DECODE.scaled(T=70, d=256, f=128, E=32, f_shared=384),
    # the down projection's slices go four to a block: three slices (a
    # partial group), and experts with more than one 32-row token block
    "decode_d384": DSV3_DECODE.scaled(T=40, d=384, f=256, E=64, f_shared=256),
    "decode_hot": DSV3_DECODE.scaled(T=200, d=512, f=256, E=64, f_shared=128),
    "dsv3_skew_small": DSV3_PREFILL_SKEW.scaled(T=300, d=384, f=256, E=64, f_shared=128),
    "qwen_fp8_small": QWEN_FP8_SKEW.scaled(T=260, d=256, f=384, E=32),
    # fp8 weights in the 256-row kernel: skewed tails (half tiles), K-split
    # gate-up tiles, and a 128-wide down-projection tile (d = 384)
    "qwen_fp8_big": QWEN_FP8_SKEW.scaled(T=800, d=512, f=384, E=16, k=4),
    "qwen_fp8_big_n128": QWEN_FP8_SKEW.scaled(T=600, d=384, f=256, E=8, k=4),
    # expert capacity (overflow dropped): every GEMM path and the shared expert
    "mixtral_cap": MIXTRAL_PREFILL.scaled(T=300, d=256, f=384, capacity_factor=1.0),
    "mixtral_big_cap": MIXTRAL_PREFILL.scaled(T=1500, d=384, f=384, E=6, capacity_factor=1.0),
    "dsv3_skew_cap": DSV3_PREFILL_SKEW.scaled(T=300, d=384, f=256, E=64, f_shared=128,
                                             capacity_factor=1.0),
    "decode_cap": DSV3_DECODE.scaled(T=40, d=512, f=256, E=64, f_shared=256, capacity_factor=1.0),
    "qwen_fp8_cap": QWEN_FP8_SKEW.scaled(T=260, d=256, f=384, E=32, capacity_factor=1.25),
    "tiny_f32_cap": TINY_F32.scaled(T=77, d=256, f=384, E=5, k=3, capacity_factor=0.75),
    # block-scaled E4M3 dispatch payload.  fp8 x fp8 gate-up GEMM: skewed
    # tails (half tiles), K-split tiles (pieces of 8-stage scale chunks), K
    # not a multiple of 512 (padded scale rows), a capacity
    "qwen_f8d_big": QWEN_FP8_SKEW.scaled(T=800, d=512, f=384, E=16, k=4, dispatch_fp8=True),
    "qwen_f8d_split": QWEN_FP8_SKEW.scaled(T=1200, d=1024, f=512, E=4, k=2, dispatch_fp8=True),
    "qwen_f8d_n128": QWEN_FP8_SKEW.scaled(T=600, d=384, f=256, E=8, k=4, dispatch_fp8=True),
    "qwen_f8d_cap": QWEN_FP8_SKEW.scaled(T=800, d=512, f=384, E=16, k=4, capacity_factor=1.25,
                                         dispatch_fp8=True),
    # payload values as bf16 rows: fp8 weights below the fp8 x fp8 shapes, bf16
    # weights on the 128-row, 256-row and decode kernels (with the shared expert)
    "qwen_f8d_small": QWEN_FP8_SKEW.scaled(T=260, d=256, f=384, E=32, dispatch_fp8=True),
    "mixtral_f8d": MIXTRAL_PREFILL.scaled(T=300, d=256, f=384, dispatch_fp8=True),
    "mixtral_big_f8d": MIXTRAL_PREFILL.scaled(T=1500, d=384, f=384, E=6, dispatch_fp8=True),
    "decode_f8d": DSV3_DECODE.scaled(T=40, d=512, f=256, E=64, f_shared=256, dispatch_fp8=True),
    # capacity overflow rerouted to the next-best expert: every GEMM path, the
    # group limit and the shared expert, the fp8 payload, and a case where
    # some tokens have fewer candidates than overflows (E = 5, k = 3)
    "mixtral_cap_rr": MIXTRAL_PREFILL.scaled(T=300, d=256, f=384, capacity_factor=1.0, overflow="reroute"),
    "mixtral_big_cap_rr": MIXTRAL_PREFILL.scaled(T=1500, d=384, f=384, E=6, capacity_factor=1.0,
                                                 overflow="reroute"),
    "dsv3_skew_cap_rr": DSV3_PREFILL_SKEW.scaled(T=300, d=384, f=256, E=64, f_shared=128, capacity_factor=1.0,
                                                 overflow="reroute"),
    "qwen_fp8_cap_rr": QWEN_FP8_SKEW.scaled(T=260, d=256, f=384, E=32, capacity_factor=1.25, overflow="reroute"),
    "qwen_f8d_cap_rr": QWEN_FP8_SKEW.scaled(T=800, d=512, f=384, E=16, k=4, capacity_factor=1.25,
                                            dispatch_fp8=True, overflow="reroute"),
    "decode_cap_rr": DSV3_DECODE.scaled(T=40, d=512, f=256, E=64, f_shared=256, capacity_factor=1.0,
                                        overflow="reroute"),
    "tiny_f32_cap_rr": TINY_F32.scaled(T=77, d=256, f=384, E=5, k=3, capacity_factor=1.0, overflow="reroute"),
    # the shared expert as an extra segment of the 256-row kernel, wider than
    # the routed experts and with a half-tile tail: x and h (routed and shared)
    # in K-blocked planes, also with the payload values written blocked
    # f >= 4096 on the 256-row kernel: the layer gathers x_perm into K-blocked
    # planes (ragged expert tails; with a capacity the gather stops early)
    "mixtral_wide_f": MIXTRAL_PREFILL.scaled(T=1100, d=256, f=4096, E=4),
    "mixtral_wide_f_cap": MIXTRAL_PREFILL.scaled(T=1100, d=256, f=4096, E=4, capacity_factor=1.0),
    "mixtral_wide_f_rr": MIXTRAL_PREFILL.scaled(T=1100, d=256, f=4096, E=4, capacity_factor=1.0,
                                                overflow="reroute"),
    # ... with fp8 weights, and beside a fused shared expert (which keeps
    # reading x row-major while the routed rows come K-blocked)
    "qwen_wide_f": QWEN_FP8_SKEW.scaled(T=1100, d=256, f=4096, E=4, k=2),
    "dsv3_wide_f_shared": DSV3_PREFILL_SKEW.scaled(T=1100, d=256, f=4096, E=8, k=2, n_group=4, topk_group=2,
                                                   f_shared=256),
    # router logits on the 256-row kernel (T >= 1024, E >= 128): one 128-wide
    # column tile (E = 128) and three (E = 384), K split across the GPU
    "router_big_e128": QWEN_FP8_SKEW.scaled(T=1100, d=512, f=128, E=128, k=2),
    "router_big_e384": QWEN_FP8_SKEW.scaled(T=1100, d=384, f=128, E=384, k=4),
    "dsv3_big_shared": DSV3_PREFILL_SKEW.scaled(T=1100, d=384, f=256, E=16, k=4, f_shared=384),
    "dsv3_big_shared_f8d": DSV3_PREFILL_SKEW.scaled(T=1100, d=384, f=256, E=16, k=4, f_shared=384,
                                                    dispatch_fp8=True),
    # router tiles ending in a quarter-height tail (1050 = 4 * 256 + 26 rows;
    # 1040: 16 rows, with the group limit and a shared expert)
    "router_big_e256_qtail": QWEN_FP8_SKEW.scaled(T=1050, d=512, f=128, E=256, k=4),
    "router_big_dsv3_qtail": DSV3_PREFILL_SKEW.scaled(T=1040, d=512, f=128, E=256, f_shared=128),
    # the token-order K-blocked copy of x (64-column planes, read two stages
    # per load) at d = 1024: the last wave's tiles split along K into pieces
    # of whole stage pairs
    "xblk_wide_split": DSV3_PREFILL_SKEW.scaled(T=1100, d=1024, f=256, E=16, k=4, f_shared=0),
    # group limits in the selection kernel: groups of 64 and of 2 (64 groups)
    # ranked in registers, groups of 48 (not a power of two) through LDS
    "group_g64": DSV3_PREFILL_SKEW.scaled(T=64, d=256, f=256, E=256, n_group=4, topk_group=2, f_shared=0),
    "group_g2": DSV3_PREFILL_SKEW.scaled(T=64, d=256, f=256, E=128, k=4, n_group=64, topk_group=8, f_shared=0),
    "group_g48": DSV3_PREFILL_SKEW.scaled(T=64, d=256, f=256, E=192, n_group=4, topk_group=2, f_shared=0),
}

_CACHE = {}


def _setup(name, seed=1):
    key = (name, seed)
    if key not in _CACHE:
        w = CASES[name]
        L = LayerInputs(w, seed, accept=O.margin_acceptor())
        _CACHE[key] = (w, L, DeviceLayer(L), oracle_layer(L))
    return _CACHE[key]


def _scores(L):
    x, wr, b = O.decoded_inputs(L)
    return O.expert_scores(O.router_logits(x, wr, b), L.w.score)


def _run_layer(w, dev, desc=None, weights=None):
    desc = desc or moe.Desc.from_attrs(w)
    w1, w3, w2 = weights or (dev.w1, dev.w3, dev.w2)
    T = w.T
    out = torch.empty((T, w.d), dtype=dev.x.dtype, device="cuda")
    idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    ws = moe.workspace(desc)
    moe.layer_forward(desc, dev.x, dev.w_router, dev.bias, w1, w3, w2, dev.s1, dev.s3,
                      dev.s2, dev.sw1, dev.sw3, dev.sw2, out, idx, gw, counts, ws)
    torch.cuda.synchronize()
    return out, idx, gw, counts


@pytest.mark.parametrize("name", list(CASES))
def test_layer_forward(name):
    w, L, dev, ref = _setup(name)
    out, idx, gw, counts = _run_layer(w, dev)
    idx_h = idx.cpu().numpy()
    assert_routing(idx_h, gw.cpu().numpy(), ref)
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    err = assert_values(from_torch(out, w.act), ref.out, w, "out")
    print(f"{name}: out err {err:.3g}")


@pytest.mark.parametrize("name", list(CASES))
def test_stages_chain(name):
    """route -> dispatch -> grouped_ffn -> combine, each output checked."""
    w, L, dev, ref = _setup(name)
    desc = moe.Desc.from_attrs(w)
    T, A = w.T, w.T * w.k
    idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    moe.route(desc, dev.x, dev.w_router, dev.bias, idx, gw, moe.workspace(desc, moe.STAGE_ROUTE))
    torch.cuda.synchronize()
    assert_routing(idx.cpu().numpy(), gw.cpu().numpy(), ref)

    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    if w.overflow == "reroute":
        # the router stage returns no candidates: the stage API refuses
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
        with pytest.raises(moe.MoeError) as err:
            moe.dispatch(desc, idx, dev.x, counts, offsets, perm, inv, x_perm,
                         moe.workspace(desc, moe.STAGE_DISPATCH))
        assert err.value.status == moe.MOE_ERR_UNSUPPORTED
        return
    if w.dispatch_fp8:
        x_perm = torch.empty(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.dispatch(desc, idx, dev.x, counts, offsets, perm, inv, x_perm,
                 moe.workspace(desc, moe.STAGE_DISPATCH))
    torch.cuda.synchronize()
    assert_dispatch(idx.cpu().numpy(), counts.cpu().numpy(), offsets.cpu().numpy(),
                    perm.cpu().numpy(), inv.cpu().numpy(), ref)
    n = int(offsets[-1])  # rows laid out: T*k, or fewer with a capacity
    if w.dispatch_fp8:  # the payload of the gathered rows, byte for byte
        codes, scales = moe.fp8_payload_views(x_perm, A, w.d)
        rc, rs = O.quantize_fp8_blocks(O.decoded_inputs(L)[0][perm[:n].cpu().numpy()])
        assert np.array_equal(codes[:n].cpu().numpy(), rc)
        assert np.array_equal(scales[:n].cpu().numpy(), rs)
    else:
        assert torch.equal(x_perm[:n], dev.x[perm[:n].long()])  # bitwise row copies

    h = torch.empty((A, w.f), dtype=dev.x.dtype, device="cuda")
    y = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.grouped_ffn(desc, x_perm, offsets, dev.w1, dev.w3, dev.w2, dev.s1, dev.s3, dev.s2, h, y,
                    moe.workspace(desc, moe.STAGE_FFN))
    torch.cuda.synchronize()
    eh = assert_values(from_torch(h[:n], w.act), ref.h, w, "h")
    ey = assert_values(from_torch(y[:n], w.act), ref.y_perm, w, "y_perm")

    out = torch.empty((T, w.d), dtype=dev.x.dtype, device="cuda")
    moe.combine(desc, y, inv, gw, None, out)
    torch.cuda.synchronize()
    # combine alone: compare with the oracle combine of the GPU's own y_perm
    ref_c = O.combine(from_torch(y, w.act), inv.cpu().numpy(), gw.cpu().numpy().astype(np.float64),
                      w.act)
    ec = assert_values(from_torch(out, w.act), ref_c, w, "combine")
    print(f"{name}: h {eh:.3g} y {ey:.3g} combine {ec:.3g}")


@pytest.mark.parametrize("name", ["mixtral_small", "qwen_fp8_small", "tiny_f32_ragged", "dsv3_skew_small",
                                  "mixtral_big_tiles", "dsv3_decode_small", "mixtral_big_split",
                                  "qwen_fp8_big"])
def test_grouped_ffn_from_oracle_inputs(name):
    """The FFN stage fed the oracle's own x_perm and offsets."""
    w, L, dev, ref = _setup(name)
    desc = moe.Desc.from_attrs(w)
    A = w.T * w.k
    if w.act == "bf16":
        xp = to_torch(O_encode_bf16(ref.x_perm), "bf16")
    else:
        xp = to_torch(ref.x_perm.astype(np.float32), "f32")
    offsets = torch.from_numpy(ref.offsets).cuda()
    h = torch.empty((A, w.f), dtype=xp.dtype, device="cuda")
    y = torch.empty((A, w.d), dtype=xp.dtype, device="cuda")
    moe.grouped_ffn(desc, xp, offsets, dev.w1, dev.w3, dev.w2, dev.s1, dev.s3, dev.s2, h, y,
                    moe.workspace(desc, moe.STAGE_FFN))
    torch.cuda.synchronize()
    assert_values(from_torch(h, w.act), ref.h, w, "h")
    assert_values(from_torch(y, w.act), ref.y_perm, w, "y_perm")


def O_encode_bf16(a):
    """float64 values that are exactly bf16 -> bf16 bit patterns."""
    f = a.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), a)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_shared_expert_and_combine_from_oracle_inputs():
    w, L, dev, ref = _setup("dsv3_decode_small")
    desc = moe.Desc.from_attrs(w)
    y = to_torch(O_encode_bf16(ref.y_perm), "bf16")
    ys = to_torch(O_encode_bf16(ref.shared_y), "bf16")
    inv = torch.from_numpy(ref.inv_pos).cuda()
    gw = torch.from_numpy(ref.topk_w.astype(np.float32)).cuda()
    out = torch.empty((w.T, w.d), dtype=torch.bfloat16, device="cuda")
    moe.combine(desc, y, inv, gw, ys, out)
    torch.cuda.synchronize()
    ref_out = O.combine(ref.y_perm, ref.inv_pos, gw.cpu().numpy().astype(np.float64), "bf16",
                        ref.shared_y)
    # same inputs, fp32 vs fp64 accumulation: at most one bf16 rounding apart
    got = from_torch(out, "bf16")
    assert np.max(np.abs(got - ref_out)) <= 2.0 ** -7 * np.max(np.abs(ref_out))


@pytest.mark.parametrize("name", ["mixtral_tiles", "dsv3_skew_small", "qwen_fp8_small", "mixtral_big_tiles",
                                  "decode_shared_wide", "mixtral_big_split", "qwen_fp8_big", "dsv3_skew_cap",
                                  "qwen_f8d_split", "decode_f8d", "dsv3_skew_cap_rr", "qwen_f8d_cap_rr",
                                  "mixtral_wide_f", "dsv3_big_shared"])
def test_deterministic(name):
    w, L, dev, ref = _setup(name)
    a = _run_layer(w, dev)
    b = _run_layer(w, dev)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("name", ["mixtral_big_tiles", "mixtral_big_k128", "mixtral_big_split", "qwen_fp8_big",
                                  "qwen_fp8_big_n128", "mixtral_big_f8d", "qwen_f8d_split", "mixtral_big_cap",
                                  "mixtral_wide_f", "mixtral_wide_f_cap", "qwen_wide_f"])
def test_layer_matches_stage_chain_bitwise(name):
    """On the 256-row kernel the layer keeps h (and for f >= 4096 x_perm) in
    K-blocked planes, or reads x through the row map; the stage entry points
    use row-major x_perm and h.  Same products in the same order: identical
    outputs."""
    w, L, dev, ref = _setup(name)
    out_l, idx, gw, counts = _run_layer(w, dev)
    desc = moe.Desc.from_attrs(w)
    T, A = w.T, w.T * w.k
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    counts2 = torch.empty(w.E, dtype=torch.int32, device="cuda")
    if w.dispatch_fp8:
        x_perm = torch.empty(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.dispatch(desc, idx, dev.x, counts2, offsets, perm, inv, x_perm, moe.workspace(desc, moe.STAGE_DISPATCH))
    h = torch.empty((A, w.f), dtype=dev.x.dtype, device="cuda")
    y = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.grouped_ffn(desc, x_perm, offsets, dev.w1, dev.w3, dev.w2, dev.s1, dev.s3, dev.s2, h, y,
                    moe.workspace(desc, moe.STAGE_FFN))
    out_c = torch.empty((T, w.d), dtype=dev.x.dtype, device="cuda")
    moe.combine(desc, y, inv, gw, None, out_c)
    torch.cuda.synchronize()
    assert torch.equal(counts, counts2)
    assert torch.equal(out_l, out_c)


@pytest.mark.parametrize("name", ["mixtral_cap_rr", "mixtral_big_cap_rr", "dsv3_skew_cap_rr", "qwen_fp8_cap_rr",
                                  "qwen_f8d_cap_rr", "decode_cap_rr", "tiny_f32_cap_rr", "mixtral_wide_f_rr"])
def test_stages_chain_reroute(name):
    """Rerouting as stages: moe_route_candidates -> moe_dispatch_reroute ->
    moe_grouped_ffn -> moe_combine with the serving gates, each output checked
    against the oracle, and the result equal to the whole layer's."""
    w, L, dev, ref = _setup(name)
    desc = moe.Desc.from_attrs(w)
    T, A, k = w.T, w.T * w.k, w.k
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    cidx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    cw = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.route_candidates(desc, dev.x, dev.w_router, dev.bias, idx, gw, cidx, cw, moe.workspace(desc, moe.STAGE_ROUTE))
    torch.cuda.synchronize()
    s = _scores(L)
    assert_routing(idx.cpu().numpy(), gw.cpu().numpy(), ref)
    # candidates: the oracle's from the same scores (indices exactly -- the
    # inputs keep ranks up to 2k apart -- and gates to the gate tolerance)
    ref_ci, ref_cw = O.reroute_candidates(s, O.workload_spec(w))
    assert np.array_equal(cidx.cpu().numpy(), ref_ci)
    have = ref_ci >= 0
    np.testing.assert_allclose(cw.cpu().numpy()[have], ref_cw[have], rtol=0, atol=GATE_TOL)

    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    gates = torch.empty(A, dtype=torch.float32, device="cuda")
    if w.dispatch_fp8:
        x_perm = torch.empty(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.dispatch_reroute(desc, idx, gw, cidx, cw, dev.x, counts, offsets, perm, inv, gates, x_perm,
                         moe.workspace(desc, moe.STAGE_DISPATCH))
    torch.cuda.synchronize()
    # the permutation and serving gates against the oracle's two passes, run
    # on the GPU's own routing outputs
    r_counts, r_off, r_perm, r_inv, r_gates, _ = O.dispatch_reroute(
        idx.cpu().numpy(), gw.cpu().numpy().astype(np.float64), cidx.cpu().numpy(),
        cw.cpu().numpy().astype(np.float64), w.E, desc.capacity)
    assert np.array_equal(counts.cpu().numpy(), r_counts)
    assert np.array_equal(offsets.cpu().numpy(), r_off)
    n = int(r_off[-1])
    assert np.array_equal(perm[:n].cpu().numpy(), r_perm)
    inv_h = inv.cpu().numpy()
    assert np.array_equal(inv_h, r_inv)
    kept = inv_h >= 0
    assert np.array_equal(gates.cpu().numpy()[kept], r_gates.reshape(-1)[kept].astype(np.float32))

    h = torch.empty((A, w.f), dtype=dev.x.dtype, device="cuda")
    y = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.grouped_ffn(desc, x_perm, offsets, dev.w1, dev.w3, dev.w2, dev.s1, dev.s3, dev.s2, h, y,
                    moe.workspace(desc, moe.STAGE_FFN))
    out = torch.empty((T, w.d), dtype=dev.x.dtype, device="cuda")
    shared_y = None
    if w.f_shared:  # the shared expert as its own 1-segment FFN over all tokens, in order
        sh_desc = moe.Desc.make(T, w.d, w.f_shared, 1, 1, act=w.act, wdtype=w.act)
        sh_off = torch.tensor([0, T], dtype=torch.int32, device="cuda")
        sh_h = torch.empty((T, w.f_shared), dtype=dev.x.dtype, device="cuda")
        shared_y = torch.empty((T, w.d), dtype=dev.x.dtype, device="cuda")
        moe.grouped_ffn(sh_desc, dev.x, sh_off, dev.sw1.unsqueeze(0).contiguous(), dev.sw3.unsqueeze(0).contiguous(),
                        dev.sw2.unsqueeze(0).contiguous(), None, None, None, sh_h, shared_y,
                        moe.workspace(sh_desc, moe.STAGE_FFN))
    moe.combine(desc, y, inv, gates, shared_y, out)
    torch.cuda.synchronize()
    assert_values(from_torch(out, w.act), ref.out, w, "out (stages)")
    if not w.f_shared:  # the layer runs the same products in the same order
        out_l, _, _, _ = _run_layer(w, dev)
        assert torch.equal(out, out_l)


# ------------------------------------------------- K-blocked expert weights

@pytest.mark.parametrize("shape,dtype", [((3, 384, 256), torch.bfloat16), ((2, 128, 96), torch.uint8),
                                         ((1, 1, 32), torch.bfloat16), ((5, 7, 64), torch.uint8)])
def test_pack_weights_layout(shape, dtype):
    """moe_pack_weights against the layout's definition: element (n, c) of a
    matrix at (c / 32) * N * 32 + n * 32 + c % 32."""
    g = torch.Generator().manual_seed(5)
    w = torch.randint(0, 256, shape, generator=g, dtype=torch.int32).to(torch.uint8)
    if dtype == torch.bfloat16:
        w = torch.randint(-2 ** 15, 2 ** 15, shape, generator=g, dtype=torch.int32).to(torch.int16).view(dtype)
    wd = w.cuda()
    packed = moe.pack_weights(wd)
    torch.cuda.synchronize()
    M, N, K = shape
    expect = w.view(M, N, K // 32, 32).permute(0, 2, 1, 3).contiguous().view(shape)
    bits = torch.uint8 if dtype == torch.uint8 else torch.int16  # random patterns include NaNs
    assert torch.equal(packed.cpu().view(bits), expect.view(bits))


def _packed(dev):
    return moe.pack_weights(dev.w1), moe.pack_weights(dev.w3), moe.pack_weights(dev.w2)


KBLOCKED_CASES = [
    # weight-streaming decode kernel (with the shared segment)
    "dsv3_decode_small", "decode_k128", "decode_shared_wide", "decode_f8d", "decode_cap",
    # 128-row kernel: bf16 and fp8 weights, shared expert
    "mixtral_small", "mixtral_tiles", "qwen_fp8_small", "dsv3_skew_small", "qwen_f8d_small",
    # 256-row kernel: half tiles, K-split tiles, K = 128, N = 128 tiles, fp8
    # weights, wide f (blocked x_perm), shared segment, payload values
    "mixtral_big_tiles", "mixtral_big_split", "mixtral_big_k128", "qwen_fp8_big", "qwen_fp8_big_n128",
    "mixtral_wide_f", "qwen_wide_f", "dsv3_wide_f_shared", "dsv3_big_shared", "mixtral_big_f8d",
    # fp8 x fp8 gate-up kernel
    "qwen_f8d_big", "qwen_f8d_split", "qwen_f8d_n128",
    # capacity: dropped and rerouted rows
    "mixtral_big_cap", "qwen_f8d_cap_rr", "dsv3_skew_cap_rr", "mixtral_wide_f_rr",
]


@pytest.mark.parametrize("name", KBLOCKED_CASES)
def test_layer_kblocked_weights_bitwise(name):
    """Routed weights packed K-blocked: every kernel multiplies the same
    values in the same order, so the layer's outputs are those of the
    row-major weights bit for bit (which the oracle checks elsewhere)."""
    w, L, dev, ref = _setup(name)
    a = _run_layer(w, dev)
    desc = moe.Desc.from_attrs(w)
    desc.w_layout = moe.W_KBLOCKED
    b = _run_layer(w, dev, desc, _packed(dev))
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("name", ["mixtral_big_split", "qwen_f8d_split", "dsv3_decode_small", "qwen_fp8_small",
                                  "qwen_fp8_big"])
def test_grouped_ffn_kblocked_weights_bitwise(name):
    w, L, dev, ref = _setup(name)
    desc = moe.Desc.from_attrs(w)
    T, A = w.T, w.T * w.k
    idx = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    moe.route(desc, dev.x, dev.w_router, dev.bias, idx, gw, moe.workspace(desc, moe.STAGE_ROUTE))
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(A, dtype=torch.int32, device="cuda")
    inv = torch.empty(A, dtype=torch.int32, device="cuda")
    if w.dispatch_fp8:
        x_perm = torch.empty(moe.fp8_payload_bytes(A, w.d), dtype=torch.uint8, device="cuda")
    else:
        x_perm = torch.empty((A, w.d), dtype=dev.x.dtype, device="cuda")
    moe.dispatch(desc, idx, dev.x, counts, offsets, perm, inv, x_perm, moe.workspace(desc, moe.STAGE_DISPATCH))
    outs = []
    for layout, (w1, w3, w2) in ((moe.W_ROWMAJOR, (dev.w1, dev.w3, dev.w2)), (moe.W_KBLOCKED, _packed(dev))):
        desc.w_layout = layout
        h = torch.zeros((A, w.f), dtype=dev.x.dtype, device="cuda")
        y = torch.zeros((A, w.d), dtype=dev.x.dtype, device="cuda")
        moe.grouped_ffn(desc, x_perm, offsets, w1, w3, w2, dev.s1, dev.s3, dev.s2, h, y,
                        moe.workspace(desc, moe.STAGE_FFN))
        torch.cuda.synchronize()
        outs.append((h, y))
    n = int(offsets[-1])
    assert torch.equal(outs[0][0][:n], outs[1][0][:n])
    assert torch.equal(outs[0][1][:n], outs[1][1][:n])


# ----------------------------------------------------------------- edge cases

def _bf16_edge_rows(d=256, seed=11):
    """bf16 rows that reach every branch of the payload quantiser: an all-zero
    row; random bit patterns over the whole finite range (subnormal inputs,
    blocks whose scale clamps at 2^-127, huge blocks); blocks spanning 2^-20
    of their amax (subnormal E4M3 codes and values that round to zero, of both
    signs); amax exactly 448 * 2^s and one bf16 step above it (the two scale
    choices); every E4M3 tie point at several scales; -0.0 entries."""
    rng = np.random.default_rng(seed)
    rows = [np.zeros(d, np.uint16)]
    for _ in range(6):  # random finite bf16 bit patterns
        r = rng.integers(0, 1 << 16, d, dtype=np.uint32).astype(np.uint16)
        r[(r & 0x7f80) == 0x7f80] &= 0xbfff  # no Inf / NaN: clear an exponent bit
        rows.append(r)
    for lo, hi in ((-20, 0), (-130, 0), (-140, -118)):  # wide ranges, bf16 subnormals, clamped scales
        e = rng.integers(lo, hi, d)
        m = rng.integers(0, 128, d)
        sign = rng.integers(0, 2, d)
        v = np.ldexp(1.0 + m / 128.0, e) * np.where(sign, -1.0, 1.0)
        rows.append(O_round_to_bf16_bits(v))
    f = np.zeros(d)
    for b in range(d // 32):  # amax = 448 * 2^s exactly / one bf16 step above
        s = b - 4
        blk = rng.standard_normal(32) * 2.0 ** s
        blk[b % 32] = (448.0 if b % 2 == 0 else 456.0) * 2.0 ** s
        f[b * 32:(b + 1) * 32] = blk
    rows.append(O_round_to_bf16_bits(f))
    ties = []  # midpoints between neighbouring E4M3 magnitudes, scale 2^0
    codes = np.arange(0, 127)
    vals = O.e4m3_to_f64(codes.astype(np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2
    mids = mids[mids == O.round_bf16(mids)]  # exactly representable in bf16
    for k in range(2):
        t = np.resize(mids, d) * np.where(np.arange(d) % 2, -1.0, 1.0) * 2.0 ** (3 * k)
        t[::32] = 448.0 * 2.0 ** (3 * k)  # pins each block's scale
        rows.append(O_round_to_bf16_bits(t))
    negz = rng.standard_normal(d)
    negz[::3] = -0.0
    rows.append(O_round_to_bf16_bits(negz))
    return np.stack(rows)


def O_round_to_bf16_bits(v):
    """float64 -> nearest bf16 bit patterns (via the oracle's rounding)."""
    r = O.round_bf16(np.asarray(v, dtype=np.float64)).astype(np.float32)
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def test_fp8_payload_bytes_edge_values():
    """The dispatch payload of crafted rows, byte for byte against the
    oracle's quantiser (one expert, k = 1: rows in order)."""
    xb = _bf16_edge_rows()
    T, d = xb.shape
    w = MIXTRAL_PREFILL.scaled(T=T, d=d, f=128, E=1, k=1, dispatch_fp8=True)
    desc = moe.Desc.from_attrs(w)
    x = to_torch(xb, "bf16")
    idx = torch.zeros((T, 1), dtype=torch.int32, device="cuda")
    counts = torch.empty(1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(2, dtype=torch.int32, device="cuda")
    perm = torch.empty(T, dtype=torch.int32, device="cuda")
    inv = torch.empty(T, dtype=torch.int32, device="cuda")
    buf = torch.empty(moe.fp8_payload_bytes(T, d), dtype=torch.uint8, device="cuda")
    moe.dispatch(desc, idx, x, counts, offsets, perm, inv, buf, moe.workspace(desc, moe.STAGE_DISPATCH))
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), np.arange(T))
    codes, scales = moe.fp8_payload_views(buf, T, d)
    rc, rs = O.quantize_fp8_blocks(O.bf16_to_f64(xb))
    sc = scales.cpu().numpy()
    assert np.array_equal(sc, rs), np.argwhere(sc != rs)[:5]
    cc = codes.cpu().numpy()
    bad = np.argwhere(cc != rc)
    assert bad.size == 0, [(tuple(i), hex(xb[tuple(i)]), cc[tuple(i)], rc[tuple(i)]) for i in bad[:5]]
    # the scale choices the rows were built to reach
    assert (rs == 0).any() and (rs == 127).any()
    assert (((rc & 0x78) == 0) & ((rc & 7) != 0)).any() and (rc == 0).any()  # subnormal codes, zeros



def _custom(w, seed=3, bias=None, wr=None, accept=True):
    L = LayerInputs(w, seed)
    if bias is not None:
        L.bias = np.asarray(bias, dtype=np.float32)
    if wr is not None:
        L.w_router = wr
    if accept:
        L._redraw(O.margin_acceptor())
    return L


def _check_custom(L, exact_order=False):
    w = L.w
    dev = DeviceLayer(L)
    ref = oracle_layer(L)
    out, idx, gw, counts = _run_layer(w, dev)
    idx_h = idx.cpu().numpy()
    if exact_order:
        assert np.array_equal(idx_h, ref.topk_idx)
        assert np.allclose(gw.cpu().numpy(), ref.topk_w, rtol=0, atol=1e-6)
    else:
        assert_routing(idx_h, gw.cpu().numpy(), ref)
    assert np.array_equal(counts.cpu().numpy(), ref.counts)
    assert_values(from_torch(out, w.act), ref.out, w, "out")
    return ref


@pytest.mark.parametrize("T", [1, 2, 129])
def test_token_counts(T):
    _check_custom(_custom(MIXTRAL_PREFILL.scaled(T=T, d=256, f=256)))


@pytest.mark.parametrize("T", [1, 2, 129])
def test_token_counts_fp8_payload(T):
    _check_custom(_custom(QWEN_FP8_SKEW.scaled(T=T, d=256, f=256, E=16, k=4, dispatch_fp8=True)))


@pytest.mark.parametrize("T,cf", [(1, 1.0), (2, 0.5), (129, 1.0)])
def test_token_counts_reroute(T, cf):
    # cf 0.5 at T = 2: one slot per expert, so the second token's repeated
    # choices overflow onto its candidates
    ref = _check_custom(_custom(DSV3_DECODE.scaled(T=T, d=256, f=256, E=16, k=4, f_shared=128,
                                                   capacity_factor=cf, overflow="reroute")))
    assert ref.served is not None


def test_reroute_k_equals_e_has_no_candidates():
    # every expert is chosen, so an overflow has no next-best expert: dropped
    ref = _check_custom(_custom(MIXTRAL_PREFILL.scaled(T=64, d=256, f=256, E=4, k=4, capacity_factor=0.5,
                                                       overflow="reroute")))
    assert (ref.served < 0).any()
    assert np.array_equal(ref.served >= 0, ref.inv_pos.reshape(ref.served.shape) >= 0)


def test_zero_tokens():
    w = MIXTRAL_PREFILL.scaled(T=0, d=256, f=256)
    desc = moe.Desc.from_attrs(w)
    counts = torch.full((w.E,), 7, dtype=torch.int32, device="cuda")
    e = torch.empty(0, device="cuda")
    moe.layer_forward(desc, e, e, None, e, e, e, None, None, None, None, None, None, e, e, e,
                      counts, None)
    torch.cuda.synchronize()
    assert (counts.cpu() == 0).all()


def test_single_expert_dense():
    _check_custom(_custom(MIXTRAL_PREFILL.scaled(T=100, d=256, f=256, E=1, k=1)))


def test_k_equals_e():
    _check_custom(_custom(MIXTRAL_PREFILL.scaled(T=64, d=256, f=256, E=8, k=8)))


def test_all_tokens_one_expert():
    # sigmoid scores: the other experts keep usable margins beside the +100 one
    w = DSV3_DECODE.scaled(T=200, d=256, f=256, E=16, k=2, f_shared=0)
    b = np.zeros(16, dtype=np.float32)
    b[11] = 100.0
    ref = _check_custom(_custom(w, bias=b))
    assert ref.counts[11] == 200


def test_empty_experts():
    w = DSV3_PREFILL_SKEW.scaled(T=8, d=256, f=256, E=128, n_group=8, topk_group=4, f_shared=0)
    ref = _check_custom(_custom(w))
    assert (ref.counts == 0).sum() > 0


def test_ties_zero_router():
    w = MIXTRAL_PREFILL.scaled(T=50, d=256, f=256, E=8, k=3)
    L = _custom(w, wr=np.zeros((8, 256), dtype=np.uint16), accept=False)
    ref = _check_custom(L, exact_order=True)
    assert (ref.topk_idx == np.arange(3)).all()


def test_ties_duplicate_router_rows():
    w = MIXTRAL_PREFILL.scaled(T=64, d=256, f=256, E=8, k=2)
    L = LayerInputs(w, 5)
    wr = L.w_router.copy()
    wr[5] = wr[2]
    bias = np.full(8, -10.0, dtype=np.float32)
    bias[2] = bias[5] = 10.0
    L = _custom(w, seed=5, bias=bias, wr=wr, accept=False)
    ref = _check_custom(L, exact_order=True)
    assert (ref.topk_idx == np.array([2, 5])).all()


def test_sigmoid_no_renorm():
    w = DSV3_DECODE.scaled(T=64, d=256, f=256, E=32, f_shared=0, renorm=False)
    _check_custom(_custom(w))


def test_softmax_no_renorm_group_limit():
    w = QWEN_FP8_SKEW.scaled(T=96, d=256, f=256, E=32, renorm=False, n_group=4, topk_group=2,
                             wdt="bf16")
    _check_custom(_custom(w))
