"""Seeded input generator: reproducibility, encodings, margin redraw."""
import numpy as np
import torch

import oracle as O
from synth import LayerInputs, encode_bf16
from synth.workloads import ALL, DSV3_PREFILL_SKEW, QWEN_FP8_SKEW, TINY_F32


def test_bf16_encoding_matches_torch():
    a = (np.random.default_rng(1).standard_normal(100000) * 7).astype(np.float32)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(encode_bf16(a), ref)


def test_reproducible_and_order_independent():
    w = DSV3_PREFILL_SKEW.scaled(T=32, d=256, f=128, E=16, n_group=4, topk_group=2)
    a = LayerInputs(w, 7)
    b = LayerInputs(w, 7)
    assert a.x.tobytes() == b.x.tobytes()
    assert a.w_router.tobytes() == b.w_router.tobytes()
    assert a.bias.tobytes() == b.bias.tobytes()
    # an expert's weights do not depend on which experts were generated before
    e5 = a.expert(5)
    _ = b.expert(2)
    assert e5.w2.tobytes() == b.expert(5).w2.tobytes()
    got = dict(b.experts(threads=3, experts=[9, 5, 1]))
    assert got[5].w1.tobytes() == e5.w1.tobytes()
    c = LayerInputs(w, 8)
    assert a.x.tobytes() != c.x.tobytes()


def test_bias_is_zipf_permutation():
    L = LayerInputs(QWEN_FP8_SKEW.scaled(T=4, d=128, f=128), 5)
    rank = np.rint(np.exp(-L.bias.astype(np.float64) / 1.5)).astype(int)
    assert sorted(rank) == list(range(1, 129))
    assert LayerInputs(TINY_F32, 1).bias is None


def test_e4m3_quantisation():
    L = LayerInputs(QWEN_FP8_SKEW.scaled(T=4, d=256, f=128), 5)
    ew = L.expert(3)
    # regenerate the float32 weights the codes came from
    from synth.gen import normal32, substream
    w32 = normal32(substream(5, "w1", 3), (128, 256)) * np.float32(1 / np.sqrt(256))
    q = O.e4m3_to_f64(ew.w1)
    assert not np.isnan(q).any() and np.abs(q).max() <= 448
    s = ew.s1.astype(np.float64)
    np.testing.assert_array_equal(s, (np.abs(w32).max(axis=1) / np.float32(448)).astype(np.float32))
    deq = q * s[:, None]
    # |q*s - w| <= half a code spacing (relative 2^-4, absolute s*2^-10 near zero)
    v = w32 / s[:, None]
    spacing = np.where(np.abs(v) >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 1e-30))) - 3), 2.0 ** -9)
    assert (np.abs(deq - w32) <= 0.5 * spacing * s[:, None] * (1 + 1e-6)).all()
    # each row uses the full range (its max element maps to +-448)
    assert (np.abs(q).max(axis=1) == 448).all()


def test_margin_redraw_holds():
    for w in ALL:
        ws = w.scaled(T=min(w.T, 256), d=min(w.d, 512))
        L = LayerInputs(ws, 1, accept=O.margin_acceptor())
        x, wr, b = O.decoded_inputs(L)
        assert O.selection_margin_ok(x, wr, b, O.workload_spec(ws)).all()
        # rows that passed on the first draw are the plain draw
        plain = LayerInputs(ws, 1)
        keep = L.redrawn == 0
        assert np.array_equal(plain.x[keep], L.x[keep])
