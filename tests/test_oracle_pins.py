"""Pins of the CPU oracle against what the pages and mathematics fix.

Each check is written independently of the oracle's own code path: brute
force over all subsets, library routines (scipy, torch) for special cases,
closed forms, invariants, and the worked examples the pages print
(tests/golden/).  ``test_planted_mistakes`` plants plausible bugs in the
oracle and shows each is caught by at least one check.
"""
import itertools
import os

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    rows, kv = [], {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0].isdigit():
                rows.append([int(p) for p in parts])
            else:
                kv[parts[0]] = int(parts[1])
    return rows, kv


def _key_beats(s, a, b):
    """Total order of the router: a beats b iff s[a] > s[b], or equal and a < b."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


# ---------------------------------------------------------------------------
# Checks (each raises AssertionError on failure; reused by the mutation test)
# ---------------------------------------------------------------------------


def check_bf16_round():
    rng = np.random.default_rng(11)
    # every finite bf16 value, as the brute-force candidate table
    codes = np.arange(65536, dtype=np.uint32)
    vals = (codes << 16).view(np.float32).astype(np.float64)
    fin = np.isfinite(vals)
    table, tcodes = vals[fin], codes[fin]
    order = np.argsort(table, kind="stable")
    table, tcodes = table[order], tcodes[order]
    # drop -0 duplicate of +0 (keep +0 code for the tie rule; both are value 0)
    x = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-5, 5, 2000),
                        rng.standard_normal(200) * 1e-39])
    # exact halfway cases between neighbouring bf16 values
    a = table[1000:1100]
    b = table[1001:1101]
    x = np.concatenate([x, (a + b) / 2])
    got = O.round_bf16(x)
    for xi, gi in zip(x, got):
        j = np.searchsorted(table, xi)
        cand = [c for c in (j - 1, j) if 0 <= c < len(table)]
        dist = [abs(table[c] - xi) for c in cand]
        best = min(dist)
        winners = [c for c, dd in zip(cand, dist) if dd == best]
        if len(winners) == 2 and table[winners[0]] != table[winners[1]]:
            # tie: even mantissa (lowest code bit 0) wins
            winners = [c for c in winners if (tcodes[c] & 1) == 0]
        assert gi == table[winners[0]], (xi, gi, table[winners[0]])
    # float32-representable inputs agree with torch's float32 -> bfloat16 cast
    f32 = (rng.standard_normal(10000) * 3).astype(np.float32)
    ref = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_bf16(f32.astype(np.float64)), ref)


def check_decoders():
    u16 = np.random.default_rng(3).integers(0, 65536, 5000).astype(np.uint16)
    ref = torch.from_numpy(u16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = O.bf16_to_f64(u16)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()
    codes = np.arange(256, dtype=np.uint8)
    tref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = O.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(tab), np.isnan(tref))
    fin = ~np.isnan(tab)
    assert np.array_equal(tab[fin], tref[fin])
    # OCP E4M3 facts: max 448, min normal 2^-6, min subnormal 2^-9, 1.0 = 0x38
    assert tab[0x7E] == 448.0 and tab[0x08] == 2.0 ** -6 and tab[0x01] == 2.0 ** -9
    assert tab[0x38] == 1.0 and tab[0xB8] == -1.0 and np.isnan(tab[0x7F]) and np.isnan(tab[0xFF])
    assert np.nanmax(tab) == 448.0


def check_router_logits():
    rng = np.random.default_rng(5)
    T, d, E = 7, 12, 5
    x = rng.standard_normal((T, d))
    sel = np.array([3, 0, 11, 7, 3])
    wr = np.zeros((E, d))
    wr[np.arange(E), sel] = 1.0      # expert e reads hidden unit sel[e]
    b = rng.standard_normal(E)
    z = O.router_logits(x, wr, b)
    assert np.array_equal(z, x[:, sel] + b[None, :])
    z0 = O.router_logits(x, 2.0 * wr, None)
    assert np.array_equal(z0, 2.0 * x[:, sel])


def check_scores():
    z = np.random.default_rng(6).standard_normal((9, 13)) * 4
    assert np.allclose(O.expert_scores(z, "softmax"), scipy.special.softmax(z, axis=1), rtol=1e-14, atol=0)
    assert np.allclose(O.expert_scores(z, "sigmoid"), scipy.special.expit(z), rtol=1e-14, atol=0)


def _brute_topk(s_row, eligible, k):
    cand = [e for e in range(len(s_row)) if eligible[e]]
    winners = []
    for sub in itertools.combinations(cand, k):
        rest = [e for e in cand if e not in sub]
        if all(_key_beats(s_row, a, b) for a in sub for b in rest):
            winners.append(sub)
    assert len(winners) == 1
    sub = list(winners[0])
    # order: position j beats every later position
    ordered = []
    while sub:
        best = [a for a in sub if all(a == b or _key_beats(s_row, a, b) for b in sub)]
        ordered.append(best[0])
        sub.remove(best[0])
    return ordered


def check_topk_bruteforce():
    rng = np.random.default_rng(7)
    for E in range(1, 9):
        for k in range(1, E + 1):
            # coarse values force exact ties
            s = rng.integers(0, 4, size=(6, E)).astype(np.float64) / 4
            idx = O.select_topk(s, O.RouteSpec(k=k))
            for t in range(s.shape[0]):
                assert list(idx[t]) == _brute_topk(s[t], [True] * E, k), (E, k, s[t], idx[t])


def check_k1_argmax():
    s = np.random.default_rng(8).integers(0, 3, size=(50, 6)).astype(np.float64)
    idx = O.select_topk(s, O.RouteSpec(k=1))
    assert np.array_equal(idx[:, 0], np.argmax(s, axis=1))  # argmax returns the first maximum


def check_constructed_ties():
    rng = np.random.default_rng(9)
    T, d, E, k = 16, 8, 6, 3
    x = rng.standard_normal((T, d))
    for score in ("softmax", "sigmoid"):
        idx, w, _ = O.route(x, np.zeros((E, d)), None, O.RouteSpec(k=k, score=score))
        assert (idx == np.arange(k)[None, :]).all()
        assert np.allclose(w, 1.0 / k, rtol=0, atol=1e-15)
    wr = rng.standard_normal((E, d))
    wr[4] = wr[1]                      # experts 1 and 4 always tie
    idx, _, s = O.route(x, wr, None, O.RouteSpec(k=k))
    assert np.array_equal(s[:, 1], s[:, 4])
    for t in range(T):
        row = list(idx[t])
        if 4 in row:
            assert 1 in row and row.index(1) == row.index(4) - 1
        top = _brute_topk(s[t], [True] * E, k)
        assert row == top


def check_group_limit():
    rng = np.random.default_rng(10)
    s = rng.random((40, 16))
    # keeping every group, or one group of all experts, is plain top-k
    plain = O.select_topk(s, O.RouteSpec(k=4))
    assert np.array_equal(O.select_topk(s, O.RouteSpec(k=4, n_group=4, topk_group=4)), plain)
    assert np.array_equal(O.select_topk(s, O.RouteSpec(k=4, n_group=1, topk_group=1)), plain)
    # brute force: E=8 in 4 groups of 2, keep 2 groups, k=2 (with exact ties)
    s = rng.integers(0, 4, size=(60, 8)).astype(np.float64) / 4
    idx = O.select_topk(s, O.RouteSpec(k=2, n_group=4, topk_group=2))
    for t in range(s.shape[0]):
        gs = [max(s[t, 2 * g + a] + s[t, 2 * g + b] for a in range(2) for b in range(2) if a != b)
              for g in range(4)]
        kept = _brute_topk(np.array(gs), [True] * 4, 2)
        elig = [(e // 2) in kept for e in range(8)]
        assert list(idx[t]) == _brute_topk(s[t], elig, 2)
    # groups of 3 (E=9, 3 groups): group score is the best pair sum
    s = rng.random((30, 9))
    idx = O.select_topk(s, O.RouteSpec(k=3, n_group=3, topk_group=1))
    for t in range(30):
        gs = [max(s[t, 3 * g + a] + s[t, 3 * g + b] for a in range(3) for b in range(3) if a != b)
              for g in range(3)]
        g0 = int(np.argmax(gs))
        assert sorted(idx[t]) == [3 * g0, 3 * g0 + 1, 3 * g0 + 2]


def check_gates():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((20, 10))
    wr = rng.standard_normal((7, 10))
    for score in ("softmax", "sigmoid"):
        _, w, s = O.route(x, wr, None, O.RouteSpec(k=3, score=score))
        assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
        idx, w_raw, s = O.route(x, wr, None, O.RouteSpec(k=3, score=score, renorm=False))
        assert np.array_equal(w_raw, np.take_along_axis(s, idx.astype(np.int64), axis=1))
    # k = E with softmax: the gates are the full softmax, in chosen order
    idx, w, _ = O.route(x, wr, None, O.RouteSpec(k=7))
    full = scipy.special.softmax(x @ wr.T, axis=1)
    assert np.allclose(w, np.take_along_axis(full, idx.astype(np.int64), axis=1), rtol=1e-13, atol=0)


def _uniform_router(T, k, E):
    """x one-hot and Wr such that token t picks experts (k*(t mod E) + j) mod E,
    in order j = 0..k-1: a perfectly uniform routing through the real router."""
    x = np.zeros((T, E))
    x[np.arange(T), np.arange(T) % E] = 1.0
    wr = np.zeros((E, E))
    for i in range(E):
        for j in range(k):
            wr[(k * i + j) % E, i] = 1.0 - 0.01 * j
    return x, wr


def check_worked_example_counts():
    _, kv = _golden("worked_example_counts.txt")
    T, k, E = kv["tokens"], kv["k"], kv["experts"]
    x, wr = _uniform_router(T, k, E)
    idx, _, _ = O.route(x, wr, None, O.RouteSpec(k=k))
    counts, offsets, _, _ = O.dispatch(idx, E)
    assert counts.sum() == kv["assignments"] == offsets[-1]
    assert (counts == kv["tokens_per_expert"]).all()
    per_gpu = counts.reshape(-1, kv["experts_per_gpu"]).sum(axis=1)
    assert (per_gpu == kv["token_experts_per_gpu"]).all()


def check_ep_sizing_and_batch():
    rows, kv = _golden("ep_sizing.txt")
    for ep, per_rank, tpe in rows:
        T = ep * per_rank
        x, wr = _uniform_router(T, 8, 256)
        idx, _, _ = O.route(x, wr, None, O.RouteSpec(k=8))
        counts = O.dispatch(idx, 256)[0]
        assert (counts == tpe).all(), (ep, counts[:4])
    assert (256 + 32) // 144 == kv["slots_ep144"]
    rows, _ = _golden("sparsity_batch.txt")
    for batch, tpe in rows:
        x, wr = _uniform_router(batch, 8, 256)
        idx, _, _ = O.route(x, wr, None, O.RouteSpec(k=8))
        assert (O.dispatch(idx, 256)[0] == tpe).all()


def check_dispatch():
    rng = np.random.default_rng(13)
    for T, k, E in ((1, 1, 1), (50, 3, 7), (200, 8, 32), (33, 2, 64)):
        s = rng.random((T, E))
        idx = O.select_topk(s, O.RouteSpec(k=k))
        counts, offsets, perm_token, inv_pos = O.dispatch(idx, E)
        a_exp = idx.reshape(-1)
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[-1] == T * k
        assert np.array_equal(np.sort(inv_pos), np.arange(T * k))          # bijection
        a = np.arange(T * k)
        assert np.array_equal(perm_token[inv_pos], a // k)
        assert ((inv_pos >= offsets[a_exp]) & (inv_pos < offsets[a_exp + 1])).all()
        for e in range(E):                                                   # stable
            seg = perm_token[offsets[e]:offsets[e + 1]]
            assert (np.diff(seg) > 0).all()
        perm = np.argsort(a_exp, kind="stable")                              # library routine
        assert np.array_equal(perm_token, perm // k)
        assert np.array_equal(inv_pos[perm], np.arange(T * k))
        assert np.array_equal(counts, np.bincount(a_exp, minlength=E))


def check_gather():
    x = np.random.default_rng(14).standard_normal((9, 5))
    p = np.array([3, 3, 0, 8, 1])
    g = O.gather_rows(x, p)
    for r, t in enumerate(p):
        assert g[r].tobytes() == x[t].tobytes()


def _torch_swiglu(x, w1, w3, w2):
    xt = torch.from_numpy(x)
    h = F.silu(F.linear(xt, torch.from_numpy(w1))) * F.linear(xt, torch.from_numpy(w3))
    return F.linear(h, torch.from_numpy(w2)).numpy()


def _weights(rng, E, d, f):
    return [(rng.standard_normal((f, d)) / np.sqrt(d), rng.standard_normal((f, d)) / np.sqrt(d),
             rng.standard_normal((d, f)) / np.sqrt(f)) for _ in range(E)]


def check_dense_special_case():
    rng = np.random.default_rng(15)
    T, d, f = 24, 16, 40
    x = rng.standard_normal((T, d))
    ws = _weights(rng, 1, d, f)
    r = O.layer_forward(x, rng.standard_normal((1, d)), None, O.RouteSpec(k=1), 1,
                        lambda e: ws[e], "f32")
    ref = _torch_swiglu(x, *ws[0])
    assert np.allclose(r.out, ref, rtol=2e-6, atol=2e-6)
    # every expert segment equals the dense FFN of its rows
    E = 5
    ws = _weights(rng, E, d, f)
    r = O.layer_forward(x, rng.standard_normal((E, d)), None, O.RouteSpec(k=2), E,
                        lambda e: ws[e], "f32")
    for e in range(E):
        lo, hi = r.offsets[e], r.offsets[e + 1]
        if hi > lo:
            assert np.allclose(r.y_perm[lo:hi], _torch_swiglu(r.x_perm[lo:hi], *ws[e]),
                               rtol=2e-6, atol=2e-6)


def check_identical_experts_closed_form():
    rng = np.random.default_rng(16)
    T, d, f, E = 30, 16, 24, 6
    x = O.round_bf16(rng.standard_normal((T, d)))
    w1, w3, w2 = (O.round_bf16(a) for a in _weights(rng, 1, d, f)[0])
    sw = tuple(O.round_bf16(a) for a in _weights(rng, 1, d, 8)[0])
    wr = rng.standard_normal((E, d))
    for shared in (None, sw):
        r = O.layer_forward(x, wr, None, O.RouteSpec(k=3, score="sigmoid"), E,
                            lambda e: (w1, w3, w2), "bf16", shared)
        ref = _torch_swiglu(x, w1, w3, w2)
        if shared is not None:
            ref = ref + _torch_swiglu(x, *shared)
        # bf16 storage of h, y, out: a few bf16 ulps of the output scale
        assert np.max(np.abs(r.out - ref)) <= 3 * 2.0 ** -8 * np.max(np.abs(ref))


def check_uniform_gates_mean():
    rng = np.random.default_rng(17)
    T, d, f, E = 12, 8, 16, 4
    x = rng.standard_normal((T, d))
    ws = _weights(rng, E, d, f)
    r = O.layer_forward(x, np.zeros((E, d)), None, O.RouteSpec(k=E), E, lambda e: ws[e], "f32")
    ref = np.mean([_torch_swiglu(x, *w) for w in ws], axis=0)
    assert np.allclose(r.out, ref, rtol=1e-5, atol=1e-6)


def check_combine():
    rng = np.random.default_rng(18)
    T, d, E = 20, 6, 5
    idx = O.select_topk(rng.random((T, E)), O.RouteSpec(k=1))
    _, _, perm_token, inv_pos = O.dispatch(idx, E)
    y = rng.standard_normal((T, d))
    out = O.combine(y, inv_pos, np.ones((T, 1)), "f32")
    assert np.array_equal(out, O.round_act(y[inv_pos], "f32"))          # pure un-permute
    # linearity: doubling y doubles out exactly
    k = 3
    idx = O.select_topk(rng.random((T, E)), O.RouteSpec(k=k))
    _, _, _, inv_pos = O.dispatch(idx, E)
    y = O.round_bf16(rng.standard_normal((T * k, d)))
    g = rng.random((T, k))
    assert np.array_equal(O.combine(2 * y, inv_pos, g, "bf16"), 2 * O.combine(y, inv_pos, g, "bf16"))
    # direct sum, written per assignment
    out = O.combine(y, inv_pos, g, "f32")
    for t in range(T):
        ref = sum(g[t, j] * y[inv_pos[t * k + j]] for j in range(k))
        assert np.allclose(out[t], ref, rtol=1e-6, atol=1e-7)


def check_locality():
    rng = np.random.default_rng(19)
    x = rng.standard_normal((64, 12))
    wr = rng.standard_normal((16, 12))
    b = rng.standard_normal(16)
    spec = O.RouteSpec(k=4, score="sigmoid", n_group=4, topk_group=2)
    idx, w, _ = O.route(x, wr, b, spec)
    S = rng.permutation(64)[:17]
    idx2, w2, _ = O.route(x[S], wr, b, spec)
    assert np.array_equal(idx2, idx[S]) and np.array_equal(w2, w[S])


def _margin_row(E, p, gap, rng):
    """Router inputs for one token whose sorted sigmoid scores are 0.05 apart
    except the pair at ranks (p, p+1), which is ``gap`` apart; the scores go
    to a random permutation of the expert ids."""
    gaps = np.full(E - 1, 0.05)
    gaps[p] = gap
    srt = 0.9 - np.concatenate([[0.0], np.cumsum(gaps)])
    s = np.empty(E)
    s[rng.permutation(E)] = srt
    b = np.log(s / (1.0 - s))  # logits whose sigmoid is s
    return np.zeros((1, E)), np.zeros((E, E)), b


def check_margin_rule():
    # every adjacent pair of sorted scores: below the pair's margin the row is
    # rejected, above it accepted; pairs past max(k, ranks) are not checked.
    # k-th vs (k+1)-th by `margin`, every other checked pair by `order_margin`.
    rng = np.random.default_rng(23)
    E, k, margin, om = 10, 3, 1e-3, 2e-5
    spec = O.RouteSpec(k=k, score="sigmoid")
    for ranks in (0, 2 * k):
        top = max(k, ranks)
        for p in range(E - 1):
            need = margin if p == k - 1 else om
            lo = O.selection_margin_ok(*_margin_row(E, p, 0.9 * need, rng), spec, margin, ranks=ranks,
                                       order_margin=om)[0]
            hi = O.selection_margin_ok(*_margin_row(E, p, 1.1 * need, rng), spec, margin, ranks=ranks,
                                       order_margin=om)[0]
            tie = O.selection_margin_ok(*_margin_row(E, p, 0.0, rng), spec, margin, ranks=ranks,
                                        order_margin=om)[0]
            assert hi, (ranks, p)
            assert lo == (p >= top) and tie == (p >= top), (ranks, p, lo, tie)
    # k = E: no k+1-th expert, the chosen order is still checked
    spec = O.RouteSpec(k=4, score="sigmoid")
    assert O.selection_margin_ok(*_margin_row(4, 2, 1.1 * om, rng), spec)[0]
    assert not O.selection_margin_ok(*_margin_row(4, 2, 0.9 * om, rng), spec)[0]
    # group rule: 4 groups of 2, keep 2; groups 1 and 2 tie exactly
    spec = O.RouteSpec(k=2, score="sigmoid", n_group=4, topk_group=2)
    b = np.array([3.0, 3.1, 1.0, 0.0, 1.0, 0.0, -2.0, -2.5])
    assert not O.selection_margin_ok(np.zeros((1, 8)), np.zeros((8, 8)), b, spec)[0]
    b[2] = 1.2  # group 1 now ahead of group 2 by more than the margin
    assert O.selection_margin_ok(np.zeros((1, 8)), np.zeros((8, 8)), b, spec)[0]
    # with a group limit the ranks are those of the eligible experts only:
    # expert 4 (group 2, not kept) scores 1e-5 below the best expert, which
    # does not matter; the same gap between the two chosen experts does
    b = np.array([3.0, 3.1, 1.0, 0.0, 0.0, -9.0, -2.0, -2.5])
    s1 = 1.0 / (1.0 + np.exp(-3.1))
    b[4] = np.log((s1 - 1e-5) / (1.0 - (s1 - 1e-5)))
    assert O.selection_margin_ok(np.zeros((1, 8)), np.zeros((8, 8)), b, spec)[0]
    b[0], b[4] = b[4], 0.0
    assert not O.selection_margin_ok(np.zeros((1, 8)), np.zeros((8, 8)), b, spec)[0]


def check_capacity():
    # slot formula: the page's worked numbers (4096 assignments over 256
    # experts = 16 per expert) at a few factors, rounded up to whole slots
    assert O.expert_capacity(1.0, 512, 8, 256) == 16
    assert O.expert_capacity(1.25, 512, 8, 256) == 20
    assert O.expert_capacity(2.0, 512, 8, 256) == 32
    assert O.expert_capacity(1.1, 512, 8, 256) == 18      # 17.6 -> 18
    assert O.expert_capacity(0.1, 10, 1, 1) == 1          # exact decimal, not 1.0000000000000000555
    assert O.expert_capacity(0, 512, 8, 256) == 0 and O.expert_capacity(-1, 512, 8, 256) == 0
    rng = np.random.default_rng(21)
    for T, k, E, cap in ((40, 2, 4, 7), (100, 3, 8, 20), (64, 8, 16, 25), (30, 1, 3, 1)):
        # skewed scores so some experts overflow
        s = rng.random((T, E)) * np.linspace(1.0, 3.0, E)
        idx = O.select_topk(s, O.RouteSpec(k=k))
        a_exp = idx.reshape(-1)
        counts, offsets, perm_token, inv_pos = O.dispatch(idx, E, cap)
        full = O.dispatch(idx, E)
        # special case: a capacity no expert reaches is the dropless layout
        big = O.dispatch(idx, E, int(full[0].max()))
        for u, v in zip(big, full):
            assert np.array_equal(u, v)
        assert np.array_equal(counts, full[0])             # counts stay the demand
        # brute force: per expert, the first `cap` assignments in increasing a
        kept = np.zeros(T * k, dtype=bool)
        for e in range(E):
            mine = [a for a in range(T * k) if a_exp[a] == e]
            kept[mine[:cap]] = True
        assert np.array_equal(inv_pos >= 0, kept)
        assert np.array_equal(np.diff(offsets), np.minimum(full[0], cap))
        assert offsets[-1] == kept.sum() == len(perm_token)
        for e in range(E):
            rows = [a for a in range(T * k) if a_exp[a] == e and kept[a]]
            assert np.array_equal(inv_pos[rows], offsets[e] + np.arange(len(rows)))
            assert np.array_equal(perm_token[offsets[e]:offsets[e + 1]], np.array(rows, dtype=np.int64) // k)
    # drops only fall as the factor grows, and vanish once every expert fits
    s = rng.random((200, 16)) * np.linspace(1.0, 4.0, 16)
    idx = O.select_topk(s, O.RouteSpec(k=2))
    drops = [int((O.dispatch(idx, 16, O.expert_capacity(cf, 200, 2, 16))[3] < 0).sum())
             for cf in (0.5, 1.0, 1.25, 2.0, 8.0)]
    assert all(a >= b for a, b in zip(drops, drops[1:])) and drops[0] > 0 and drops[-1] == 0
    # layer closed form: the capacity layer's output is the dropless layer's
    # per-assignment terms with the dropped ones removed (gates unchanged)
    T, d, f, E, k = 24, 8, 16, 4, 2
    x = rng.standard_normal((T, d))
    wr = rng.standard_normal((E, d))
    W = _weights(rng, E, d, f)
    spec = O.RouteSpec(k=k)
    ref = O.layer_forward(x, wr, None, spec, E, lambda e: W[e], "f32")
    cap = 5
    got = O.layer_forward(x, wr, None, spec, E, lambda e: W[e], "f32", capacity=cap)
    kept = got.inv_pos >= 0
    assert (~kept).any() and kept.any()
    want = np.zeros((T, d))
    for a in range(T * k):
        if kept[a]:
            want[a // k] += ref.topk_w[a // k, a % k] * ref.y_perm[ref.inv_pos[a]]
    assert np.array_equal(got.out, O.round_act(want, "f32"))  # same j order, same rounding


def check_reroute():
    """Overflow rerouted to the next-best expert: special cases that reduce to
    dispatch(), invariants checked by brute force, and a constructed layer
    whose output is known in closed form."""
    rng = np.random.default_rng(33)
    # candidates: the ranks right after the top-k, by brute force over the order
    s = rng.random((30, 9))
    for spec in (O.RouteSpec(k=2), O.RouteSpec(k=3, renorm=False), O.RouteSpec(k=2, n_group=3, topk_group=2)):
        cand, cw = O.reroute_candidates(s, spec)
        el = O.eligible(s, spec)
        for t in range(30):
            ranked = sorted([e for e in range(9) if el[t, e]], key=lambda e: (-s[t, e], e))
            want = (ranked[spec.k:2 * spec.k] + [-1] * spec.k)[:spec.k]
            assert list(cand[t]) == want, (t, list(cand[t]), want)
            den = sum(s[t, e] for e in ranked[:spec.k]) if spec.renorm else 1.0
            for m, c in enumerate(want):
                assert cw[t, m] == (s[t, c] / den if c >= 0 else 0.0)
    for T, k, E, cap in ((40, 2, 6, 7), (100, 3, 8, 20), (64, 4, 16, 10), (30, 1, 3, 4), (50, 2, 2, 30)):
        s = rng.random((T, E)) * np.linspace(1.0, 3.0, E)
        spec = O.RouteSpec(k=k)
        idx = O.select_topk(s, spec)
        gw = O.gate_weights(s, idx, True)
        cand, cw = O.reroute_candidates(s, spec)
        counts, offsets, perm, inv, gates, served = O.dispatch_reroute(idx, gw, cand, cw, E, cap)
        drop = O.dispatch(idx, E, cap)
        assert np.array_equal(counts, drop[0])
        # a capacity no expert reaches: the dropless layout, every gate its own
        big = O.dispatch_reroute(idx, gw, cand, cw, E, int(drop[0].max()))
        full = O.dispatch(idx, E)
        for u, v in zip(big[:4], full):
            assert np.array_equal(u, v)
        assert np.array_equal(big[4], gw)
        n = T * k
        a_exp = idx.reshape(-1)
        own = (drop[3] >= 0)                      # pass 1 keeps what dropping keeps
        srv = served.reshape(-1)
        assert np.array_equal(srv[own], a_exp[own])
        # brute force of pass 2: offers in increasing a take the slots left
        left = cap - np.minimum(drop[0], cap)
        want_srv = np.where(own, a_exp, -1)
        want_g = np.where(own.reshape(T, k), gw, 0.0)
        # offers ordered by a, one expert at a time
        offers = {}
        for t in range(T):
            over = [j for j in range(k) if not own[t * k + j]]
            for m, j in enumerate(over):
                if cand[t, m] >= 0:
                    offers.setdefault(int(cand[t, m]), []).append((t * k + j, m))
        for c, lst in offers.items():
            for a, m in sorted(lst)[:left[c]]:
                want_srv[a] = c
                want_g[a // k, a % k] = cw[a // k, m]
        assert np.array_equal(srv, want_srv)
        assert np.array_equal(gates, want_g)
        # rows: per expert its own assignments, then the rerouted ones, each by a
        for e in range(E):
            rows = [a for a in range(n) if own[a] and a_exp[a] == e] + \
                   [a for a in range(n) if not own[a] and srv[a] == e]
            assert len(rows) <= cap
            assert np.array_equal(inv[rows], offsets[e] + np.arange(len(rows)))
            assert np.array_equal(perm[offsets[e]:offsets[e + 1]], np.array(rows, dtype=np.int64) // k)
        assert np.array_equal(inv >= 0, srv >= 0)
        assert (inv < 0).sum() <= (drop[3] < 0).sum()
    # E == k: no candidates, so rerouting drops exactly what dropping drops
    s = rng.random((20, 3)) * np.array([1.0, 2.0, 5.0])
    idx = O.select_topk(s, O.RouteSpec(k=3))
    cand, cw = O.reroute_candidates(s, O.RouteSpec(k=3))
    assert (cand == -1).all()
    r = O.dispatch_reroute(idx, O.gate_weights(s, idx, True), cand, cw, 3, 8)
    d = O.dispatch(idx, 3, 8)
    for u, v in zip(r[:4], d):
        assert np.array_equal(u, v)
    # constructed layer (k = 1, one slot per expert): every token's best expert
    # is 0 and token t's second best is t + 1, so token 0 is served by expert
    # 0 with gate 1 and token t > 0 by expert t + 1 with gate s_{t+1} / s_0
    T, d_, f, E = 6, 8, 16, 7
    x = rng.standard_normal((T, d_))
    W = _weights(rng, E, d_, f)
    wr = np.zeros((E, d_))
    bias = np.full(E, -30.0)
    bias[0] = 5.0
    z = np.tile(bias, (T, 1))
    for t in range(T):
        z[t, t + 1] = 1.0 + 0.1 * t
    # express the per-token logits through x: one-hot rows of x pick them
    x_route = np.eye(T)
    wr_route = z.T.copy()
    spec = O.RouteSpec(k=1)
    got = O.layer_forward(np.hstack([x_route, x]), np.hstack([wr_route, np.zeros((E, d_))]), None,
                          spec, E, lambda e: (np.hstack([np.zeros((f, T)), W[e][0]]),
                                              np.hstack([np.zeros((f, T)), W[e][1]]),
                                              np.vstack([np.zeros((T, f)), W[e][2]])),
                          "f32", capacity=1, overflow="reroute")
    sc = O.expert_scores(z, "softmax")
    want = np.zeros((T, T + d_))
    for t in range(T):
        e, g = (0, 1.0) if t == 0 else (t + 1, sc[t, t + 1] / sc[t, 0])
        xt = np.hstack([x_route[t], x[t]])[None, :]
        w1 = np.hstack([np.zeros((f, T)), W[e][0]])
        w3 = np.hstack([np.zeros((f, T)), W[e][1]])
        w2 = np.vstack([np.zeros((T, f)), W[e][2]])
        u, v = xt @ w1.T, xt @ w3.T
        h = O.round_act(u / (1 + np.exp(-u)) * v, "f32")
        want[t] = g * O.round_act(h @ w2.T, "f32")[0]
    assert np.array_equal(got.served.reshape(-1), [0] + [t + 1 for t in range(1, T)])
    np.testing.assert_allclose(got.out, O.round_act(want, "f32"), rtol=0, atol=1e-6)


def _nearest_code_bruteforce(v):
    """Exhaustive nearest E4M3 code of one magnitude, ties to the even mantissa."""
    best = None
    for c in range(0x7F):  # non-negative finite codes
        val = O.E4M3_VALUES[c]
        dist = abs(val - v)
        if best is None or dist < best[0] or (dist == best[0] and (c & 1) == 0):
            best = (dist, c)
    return best[1]


def check_fp8_payload():
    rng = np.random.default_rng(31)
    # magnitudes over the whole range, exact codes, ties and subnormals
    vals = np.concatenate([rng.uniform(0, 448, 300), O.E4M3_VALUES[:0x7F],
                           (O.E4M3_VALUES[1:0x7F] + O.E4M3_VALUES[:0x7E]) / 2,
                           rng.uniform(0, 2.0 ** -6, 60)])
    got = M._rne_e4m3_magnitude(vals)
    for v, c in zip(vals, got):
        assert c == _nearest_code_bruteforce(v), (v, c)
    # rows of blocks at very different scales, with a zero block
    x = O.round_bf16(rng.standard_normal((6, 128)) * np.repeat([1e-4, 3.0, 700.0, 0.0], 32))
    codes, scales = O.quantize_fp8_blocks(x)
    assert codes.shape == x.shape and scales.shape == (6, 4)
    s = scales.astype(np.int64) - 127
    amax = np.abs(x.reshape(6, 4, 32)).max(axis=2)
    nz = amax > 0
    assert (np.ldexp(448.0, s)[nz] >= amax[nz]).all()            # nothing saturates
    assert (np.ldexp(448.0, s - 1)[nz] < amax[nz]).all()         # and s is the smallest such
    assert (scales[~nz] == 127).all() and (codes.reshape(6, 4, 32)[~nz] == 0).all()
    deq = O.dequantize_fp8_blocks(codes, scales)
    # each element is its nearest representable (per-block scale), i.e. within half a step
    v = np.abs(x.reshape(6, 4, 32)) * np.ldexp(1.0, -s)[:, :, None]
    for (r, b, i), vv in np.ndenumerate(v):
        assert codes.reshape(6, 4, 32)[r, b, i] & 0x7F == _nearest_code_bruteforce(vv)
    assert np.array_equal(np.sign(deq), np.sign(x))
    # sign symmetry and exact round trip of representable payloads
    c2, s2 = O.quantize_fp8_blocks(-x)
    assert np.array_equal(s2, scales) and np.array_equal(c2[codes != 0], codes[codes != 0] ^ 0x80)
    # a payload's values are representable, so requantising returns them exactly
    # (the scale may step down when a block's largest element rounded down to
    # 224 * 2^s, so codes need not repeat; values do)
    assert np.array_equal(O.dequantize_fp8_blocks(*O.quantize_fp8_blocks(deq)), deq)
    # layer special case: on a representable payload the fp8 dispatch changes nothing
    T, d, f, E, k = 6, 128, 32, 4, 2
    W = _weights(rng, E, d, f)
    wr = rng.standard_normal((E, d))
    ref = O.layer_forward(deq, wr, None, O.RouteSpec(k=k), E, lambda e: W[e], "f32")
    got = O.layer_forward(deq, wr, None, O.RouteSpec(k=k), E, lambda e: W[e], "f32", fp8_dispatch=True)
    assert np.array_equal(got.out, ref.out)


CHECKS = [check_bf16_round, check_decoders, check_router_logits, check_scores,
          check_topk_bruteforce, check_k1_argmax, check_constructed_ties, check_group_limit,
          check_gates, check_worked_example_counts, check_ep_sizing_and_batch, check_dispatch,
          check_gather, check_dense_special_case, check_identical_experts_closed_form,
          check_uniform_gates_mean, check_combine, check_locality, check_margin_rule,
          check_capacity, check_fp8_payload, check_reroute]


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_pin(check):
    check()


# ---------------------------------------------------------------------------
# Planted mistakes: each must be caught by some check
# ---------------------------------------------------------------------------

M = O.moe_oracle
_DISPATCH = M.dispatch


def _m_silu_dropped(u):
    return u


def _m_softmax_sign(z, score):
    if score == "softmax":
        p = np.exp(-(z - z.max(axis=1, keepdims=True)))
        return p / p.sum(axis=1, keepdims=True)
    return 1.0 / (1.0 + np.exp(-z))


def _m_bias_dropped(x, w_router, bias):
    return x @ w_router.T


def _m_w2_transposed(xr, w1, w3, w2, act):
    u = xr @ w1.T
    v = xr @ w3.T
    h = M.round_act(M.silu(u) * v, act)
    return h, M.round_act(h @ w2.reshape(w2.shape[1], w2.shape[0]), act)


def _m_tie_high_id(values):
    ids = np.broadcast_to(np.arange(values.shape[1]), values.shape)
    return np.lexsort((-ids, -values), axis=-1)


def _m_gate_no_renorm(s, idx, renorm):
    return np.take_along_axis(s, idx.astype(np.int64), axis=1)


def _m_group_top1(s, n_group):
    T, E = s.shape
    return np.sort(s.reshape(T, n_group, E // n_group), axis=2)[:, :, -1]


def _m_dispatch_unstable(topk_idx, E, capacity=0):
    if capacity > 0:
        return _DISPATCH(topk_idx, E, capacity)
    c, o, p, i = _DISPATCH(topk_idx, E)
    p = p.copy()
    i = i.copy()
    for e in range(E):                   # reverse each segment
        lo, hi = o[e], o[e + 1]
        p[lo:hi] = p[lo:hi][::-1]
    for a in range(len(i)):
        e = topk_idx.reshape(-1)[a]
        i[a] = o[e] + o[e + 1] - 1 - i[a]
    return c, o, p, i


def _m_capacity_off_by_one(topk_idx, E, capacity=0):
    return _DISPATCH(topk_idx, E, capacity + 1 if capacity > 0 else 0)


def _m_capacity_keeps_last(topk_idx, E, capacity=0):
    """Fills an expert's slots with its last assignments instead of its first."""
    if capacity <= 0:
        return _DISPATCH(topk_idx, E)
    T, k = topk_idx.shape
    rev = topk_idx.reshape(-1)[::-1].reshape(T, k)
    c, o, p, i = _DISPATCH(rev, E, capacity)
    n = T * k
    i = i[::-1].copy()
    p = np.array([n - 1 - 0 for _ in p])  # rows no longer name the right tokens
    return c, o, p, i


_CANDIDATES = M.reroute_candidates
_REROUTE = M.dispatch_reroute


def _m_candidates_skip_one(s, spec):
    """Offers the rank after the next-best expert."""
    cand, cw = _CANDIDATES(s, spec)
    return np.concatenate([cand[:, 1:], np.full((cand.shape[0], 1), -1, np.int32)], axis=1), \
        np.concatenate([cw[:, 1:], np.zeros((cw.shape[0], 1))], axis=1)


def _m_reroute_ignores_pass1(topk_idx, topk_w, cand_idx, cand_w, E, capacity):
    """Lets the offers use a full capacity on top of the slots pass 1 took."""
    out = _REROUTE(topk_idx, topk_w, cand_idx, cand_w, E, 2 * capacity)
    drop = _DISPATCH(topk_idx, E, capacity)
    return (drop[0],) + out[1:]


def _m_reroute_keeps_gate(topk_idx, topk_w, cand_idx, cand_w, E, capacity):
    """Rerouted copies carry the gate of the expert they were meant for."""
    c, o, p, i, g, sv = _REROUTE(topk_idx, topk_w, cand_idx, cand_w, E, capacity)
    return c, o, p, i, np.where(sv >= 0, topk_w, 0.0), sv


_RNE_E4M3 = M._rne_e4m3_magnitude
_QUANT_FP8 = M.quantize_fp8_blocks


def _m_e4m3_truncate(v):
    """Rounds toward zero instead of to nearest."""
    c = _RNE_E4M3(v)
    back = M.E4M3_VALUES[c]
    return np.where(back > np.asarray(v, dtype=np.float64), c - 1, c)


def _m_fp8_scale_low(x, block=32):
    """Takes a scale one power of two too small (the largest elements saturate)."""
    codes, scales = _QUANT_FP8(x, block)
    scales = scales - 1
    v = np.asarray(x, dtype=np.float64).reshape(x.shape[0], -1, block) * np.ldexp(1.0, -(scales.astype(np.int64) - 127))[:, :, None]
    mag = np.minimum(_RNE_E4M3(np.minimum(np.abs(v), 448.0)), 0x7E)
    codes = (mag | ((v < 0).astype(np.int64) << 7)).reshape(x.shape).astype(np.uint8)
    return codes, scales


def _m_combine_wrong_index(y_perm, inv_pos, topk_w, act, shared_y=None):
    T, k = topk_w.shape
    out = np.zeros((T, y_perm.shape[1]))
    for j in range(k):
        out += topk_w[:, j: j + 1] * y_perm[np.arange(T) * 0 + j]
    if shared_y is not None:
        out += shared_y
    return M.round_act(out, act)


def _m_round_truncate(a):
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)
    e = np.maximum(e, -125)
    return np.ldexp(np.trunc(np.ldexp(a, 8 - e)), e - 8)


def _margin_variant(shift=0, unmasked=False, big_at=-1):
    """selection_margin_ok with one planted change: the checked pairs end
    `shift` ranks late (or early), masked experts are ranked too, or the
    k-th/(k+1)-th margin goes to the pair `big_at` ranks away."""

    def bad(x, w_router, bias, spec, margin=1e-3, ranks=0, order_margin=2e-5):
        s = M.expert_scores(M.router_logits(x, w_router, bias), spec.score)
        T, E = s.shape
        ok = np.ones(T, dtype=bool)
        masked = s if unmasked else np.where(M.eligible(s, spec), s, -np.inf)
        srt = -np.sort(-masked, axis=1)
        for i in range(max(0, min(max(spec.k, ranks) + shift, E - 1))):
            need = margin if i == spec.k - 1 + (big_at + 1) else order_margin
            hi, lo = srt[:, i], srt[:, i + 1]
            ok &= ~np.isfinite(lo) | ((hi - lo) >= need)
        if spec.n_group and spec.topk_group < spec.n_group:
            g = -np.sort(-M.group_scores(s, spec.n_group), axis=1)
            ok &= (g[:, spec.topk_group - 1] - g[:, spec.topk_group]) >= margin
        return ok

    return bad


def _m_margin_short(*a, **kw):
    return _margin_variant(shift=-1)(*a, **kw)


def _m_margin_long(*a, **kw):
    return _margin_variant(shift=1)(*a, **kw)


def _m_margin_unmasked(*a, **kw):
    return _margin_variant(unmasked=True)(*a, **kw)


def _m_margin_wrong_pair(*a, **kw):
    return _margin_variant(big_at=0)(*a, **kw)


MUTATIONS = [
    ("silu", _m_silu_dropped),
    ("expert_scores", _m_softmax_sign),
    ("router_logits", _m_bias_dropped),
    ("swiglu_expert", _m_w2_transposed),
    ("_order_desc", _m_tie_high_id),
    ("gate_weights", _m_gate_no_renorm),
    ("group_scores", _m_group_top1),
    ("dispatch", _m_dispatch_unstable),
    ("combine", _m_combine_wrong_index),
    ("dispatch", _m_capacity_off_by_one),
    ("dispatch", _m_capacity_keeps_last),
    ("_rne_e4m3_magnitude", _m_e4m3_truncate),
    ("quantize_fp8_blocks", _m_fp8_scale_low),
    ("round_bf16", _m_round_truncate),
    ("reroute_candidates", _m_candidates_skip_one),
    ("dispatch_reroute", _m_reroute_ignores_pass1),
    ("dispatch_reroute", _m_reroute_keeps_gate),
    ("selection_margin_ok", _m_margin_short),
    ("selection_margin_ok", _m_margin_long),
    ("selection_margin_ok", _m_margin_unmasked),
    ("selection_margin_ok", _m_margin_wrong_pair),
]


@pytest.mark.parametrize("name,bad", MUTATIONS, ids=[m[0] + "_" + m[1].__name__.lstrip("_") for m in MUTATIONS])
def test_planted_mistakes(monkeypatch, name, bad):
    monkeypatch.setattr(M, name, bad)
    # O.* re-exports bind the original objects: patch those names too
    if hasattr(O, name):
        monkeypatch.setattr(O, name, bad)
    caught = []
    for c in CHECKS:
        try:
            c()
        except (AssertionError, ValueError, IndexError, TypeError):
            caught.append(c.__name__)
    assert caught, f"mutant {name} escaped every check"
