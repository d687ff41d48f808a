"""CPU oracle of the MoE layer forward -- TEST INFRASTRUCTURE, not product code.

Plain, slow, float64 NumPy.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import it; the HIP library never calls it and shares no
code, table or helper with it.

What it computes follows the per-token routing path the pages describe:
a small linear gate scores every expert, a softmax turns the scores into
probabilities, the top-k experts are kept, each transforms the token, and their
outputs are summed weighted by the gate scores ("Expert-Parallel MoE
Inference: Serving Sparse Models at Scale", §Deeper Analysis: Routing, Balance,
and a Capacity Worked Example, Figure 2; the same chain router -> top-k ->
dispatch -> expert FFN -> combine -> original token order in "MoE Expert
Parallelism in Practice", §Core Principles 1; experts run as grouped GEMMs and
combine is a weighted sum in "Tensor vs Expert vs Data Parallelism for MoE
Serving", §Deeper Analysis, Figure 2).  Dispatch is drop-free by default
(the path preferred in "Expert-Parallel MoE Inference", §Capacity factor and
token dropping); the same section's capacity variant is here too: a fixed
number of slots per expert, with overflow dropped (dispatch) or rerouted to
the token's next-best expert (dispatch_reroute).

Readings the pages leave open, and the workload definitions fix:
  * expert FFN is SwiGLU: h = silu(x W1) * (x W3), y = h W2, silu(u) = u*sigmoid(u);
  * score is softmax or sigmoid; gates renormalised over the chosen k;
  * optional group limit: E experts in n_group contiguous groups, a group's
    score is the sum of its two largest expert scores, only the best
    topk_group groups stay eligible (the single-GPU form of the node-limited
    routing in "Expert-Parallel MoE Inference", §Load imbalance and how to
    fight it, and "Expert Parallelism for MoE Serving", §Real-World
    Implementation);
  * the router bias is added to the logits and used for both selection and
    gates;
  * ties go to the lower expert (group) id; the k outputs are in descending
    score order;
  * a shared expert, when present, is always on with coefficient 1 (the
    "shared expert" of DeepSeek-V3 in "Tensor vs Expert vs Data Parallelism",
    §Context and Background);
  * the activation dtype rounding (round to nearest even) is applied exactly
    where the layer stores an activation tensor: h, y_perm, the shared
    expert's h and y, and out.  Everything else is exact float64 on the stored
    input values.

Storage conventions: weights are stored out x in (W1[e][j][i] is the math's
W1_e[i, j]); bf16 as uint16 bit patterns; e4m3 as uint8 OCP E4M3 codes with a
float32 scale per output channel.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Callable, Optional, Sequence

import numpy as np

# --------------------------------------------------------------------------
# Storage decoding and activation rounding (exact)
# --------------------------------------------------------------------------


def bf16_to_f64(u16: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact: bf16 is the top half of a float32)."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    """Value of every OCP E4M3 code: 1 sign, 4 exponent (bias 7), 3 mantissa bits.

    Exponent 0 is subnormal (m * 2^-9); code S.1111.111 is NaN; no infinities.
    """
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


# --------------------------------------------------------------------------
# fp8 dispatch payload (block-scaled E4M3)
# --------------------------------------------------------------------------

FP8_BLOCK = 32      # elements of a row sharing one scale
E4M3_MAX = 448.0


def _rne_e4m3_magnitude(v: np.ndarray) -> np.ndarray:
    """Nearest OCP E4M3 magnitude code (ties to even) of 0 <= v <= 448: normal
    codes hold (1 + m/8) * 2^(e-7) for exponent field e = 1..15, subnormal
    codes m * 2^-9.  Written from the format, step by step."""
    v = np.asarray(v, dtype=np.float64)
    code = np.zeros(v.shape, dtype=np.int64)
    nz = v > 0
    _, ex = np.frexp(np.where(nz, v, 1.0))          # v = f * 2^ex, f in [0.5, 1)
    e_unb = ex - 1                                   # v in [2^e_unb, 2^(e_unb+1))
    normal = nz & (e_unb >= -6)
    # normal: v / 2^(e_unb - 3) in [8, 16) -> round to an integer in [8, 16]
    q = np.rint(np.where(normal, np.ldexp(v, -(e_unb - 3)), 0.0)).astype(np.int64)
    carry = q == 16                                  # rounded up into the next binade
    e_field = np.where(carry, e_unb + 8, e_unb + 7)
    mant = np.where(carry, 0, q - 8)
    code = np.where(normal, (e_field << 3) | mant, code)
    # subnormal: v / 2^-9 in [0, 8) -> integer 0..8 (8 is the smallest normal, code 8)
    sub = nz & (e_unb < -6)
    qs = np.rint(np.where(sub, np.ldexp(v, 9), 0.0)).astype(np.int64)
    code = np.where(sub, qs, code)
    return code


def quantize_fp8_blocks(x: np.ndarray, block: int = FP8_BLOCK):
    """The fp8 dispatch payload: each row cut into blocks of `block` elements;
    a block with largest magnitude amax gets the power-of-two scale 2^s with s
    the smallest integer such that amax <= 448 * 2^s (no element saturates),
    stored as an E8M0 byte (s + 127, s clamped to [-127, 127]; an all-zero
    block gets s = 0); its elements become E4M3 codes of x / 2^s rounded to
    nearest, ties to even.  ("Tensor vs Expert vs Data Parallelism for MoE
    Serving", section "Deeper Analysis", Figure 2: dispatch sends FP8 token
    copies, combine returns BF16.)  Returns codes uint8 [rows][d] and scales
    uint8 [rows][d / block]."""
    x = np.asarray(x, dtype=np.float64)
    rows, d = x.shape
    xb = x.reshape(rows, d // block, block)
    amax = np.abs(xb).max(axis=2)
    s = np.zeros(amax.shape, dtype=np.int64)
    nz = amax > 0
    # smallest s with amax <= 448 * 2^s: start from 2^s ~ amax / 448 and step
    s0 = np.floor(np.log2(np.where(nz, amax, 1.0) / E4M3_MAX)).astype(np.int64) - 1
    for _ in range(4):
        up = nz & (np.ldexp(E4M3_MAX, s0) < amax)
        s0 = np.where(up, s0 + 1, s0)
    s = np.where(nz, np.clip(s0, -127, 127), 0)
    v = np.abs(xb) * np.ldexp(1.0, -s)[:, :, None]
    mag = _rne_e4m3_magnitude(v)
    sign = (xb < 0).astype(np.int64) << 7
    codes = np.where(mag == 0, 0, mag | sign).reshape(rows, d).astype(np.uint8)
    return codes, (s + 127).astype(np.uint8)


def dequantize_fp8_blocks(codes: np.ndarray, scales: np.ndarray, block: int = FP8_BLOCK) -> np.ndarray:
    """Values of a block-scaled E4M3 payload: code value * 2^(scale - 127)."""
    v = e4m3_to_f64(codes)
    rows, d = v.shape
    e = np.asarray(scales, dtype=np.int64) - 127
    return (v.reshape(rows, d // block, block) * np.ldexp(1.0, e)[:, :, None]).reshape(rows, d)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(a)
    if dtype == "e4m3":
        return e4m3_to_f64(a)
    raise ValueError(dtype)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    bf16 keeps 8 significant bits; the smallest normal is 2^-126 and below it
    the spacing is fixed at 2^-133.
    """
    a = np.asarray(a, dtype=np.float64)
    _, e = np.frexp(a)                      # a = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)
    r = np.rint(np.ldexp(a, 8 - e))         # exact scaling, then half-to-even
    out = np.ldexp(r, e - 8)
    return np.where(np.abs(out) > 3.3895313892515355e38, np.copysign(np.inf, a), out)


def round_act(a: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)
    if act == "bf16":
        return round_bf16(a)
    raise ValueError(act)


# --------------------------------------------------------------------------
# Routing
# --------------------------------------------------------------------------


@dataclass(frozen=True)
class RouteSpec:
    k: int
    score: str = "softmax"     # "softmax" | "sigmoid"
    renorm: bool = True
    n_group: int = 0
    topk_group: int = 0


def router_logits(x: np.ndarray, w_router: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """z[t, e] = sum_i x[t, i] * Wr[e][i] + b[e]: the small linear gate that
    scores every expert for every token ("Expert-Parallel MoE Inference",
    §Deeper Analysis, first paragraph).  Wr is stored out x in, [E][d]."""
    z = x @ w_router.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def expert_scores(z: np.ndarray, score: str) -> np.ndarray:
    """Softmax over the E logits (same passage), or the element-wise sigmoid."""
    if score == "softmax":
        m = z.max(axis=1, keepdims=True)
        p = np.exp(z - m)
        return p / p.sum(axis=1, keepdims=True)
    if score == "sigmoid":
        return 1.0 / (1.0 + np.exp(-z))
    raise ValueError(score)


def _order_desc(values: np.ndarray) -> np.ndarray:
    """Per row, indices ordered by (value descending, index ascending)."""
    ids = np.broadcast_to(np.arange(values.shape[1]), values.shape)
    return np.lexsort((ids, -values), axis=-1)


def group_scores(s: np.ndarray, n_group: int) -> np.ndarray:
    """Score of each contiguous expert group: the sum of its two largest scores."""
    T, E = s.shape
    sg = np.sort(s.reshape(T, n_group, E // n_group), axis=2)
    return sg[:, :, -1] + sg[:, :, -2]


def eligible(s: np.ndarray, spec: RouteSpec) -> np.ndarray:
    """Boolean [T, E]: experts a token may choose.  With a group limit only the
    experts of the topk_group best groups (ties to the lower group id)."""
    T, E = s.shape
    if spec.n_group == 0:
        return np.ones((T, E), dtype=bool)
    gs = group_scores(s, spec.n_group)
    keep = _order_desc(gs)[:, : spec.topk_group]
    gmask = np.zeros((T, spec.n_group), dtype=bool)
    np.put_along_axis(gmask, keep, True, axis=1)
    return np.repeat(gmask, E // spec.n_group, axis=1)


def select_topk(s: np.ndarray, spec: RouteSpec) -> np.ndarray:
    """The k eligible experts of each token in (score descending, id ascending)
    order: the top-k the router keeps."""
    masked = np.where(eligible(s, spec), s, -np.inf)
    return _order_desc(masked)[:, : spec.k].astype(np.int32)


def gate_weights(s: np.ndarray, idx: np.ndarray, renorm: bool) -> np.ndarray:
    """Gate of each chosen expert: its score, divided by the sum over the chosen
    k when renormalised."""
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    return sel / sel.sum(axis=1, keepdims=True) if renorm else sel


def route(x, w_router, bias, spec: RouteSpec):
    """-> (topk_idx [T,k] int32, topk_w [T,k] float64, scores [T,E] float64)."""
    s = expert_scores(router_logits(x, w_router, bias), spec.score)
    idx = select_topk(s, spec)
    return idx, gate_weights(s, idx, spec.renorm), s


def selection_margin_ok(x, w_router, bias, spec: RouteSpec, margin: float = 1e-3,
                        ranks: int = 0, order_margin: float = 2e-5) -> np.ndarray:
    """Rows whose routing decisions are separated, so that a float32 router
    must reach the same decisions as this one (used to redraw synthetic token
    rows).  Over the eligible scores sorted descending, s_0 >= s_1 >= ...:
      * the k-th vs (k+1)-th score (in or out) by at least ``margin``;
      * with a group limit, the topk_group-th vs next group score by ``margin``;
      * every other adjacent pair (s_i, s_i+1) for i < max(k, ranks) by at
        least ``order_margin``: i < k-1 fixes the order of the k outputs,
        k <= i < ranks the order of reroute candidates (ranks = 2k).
    A pair whose lower score is not eligible (-inf) always passes."""
    s = expert_scores(router_logits(x, w_router, bias), spec.score)
    T, E = s.shape
    ok = np.ones(T, dtype=bool)
    masked = np.where(eligible(s, spec), s, -np.inf)
    srt = -np.sort(-masked, axis=1)
    for i in range(min(max(spec.k, ranks), E - 1)):
        need = margin if i == spec.k - 1 else order_margin
        hi, lo = srt[:, i], srt[:, i + 1]
        ok &= ~np.isfinite(lo) | ((hi - lo) >= need)
    if spec.n_group and spec.topk_group < spec.n_group:
        g = -np.sort(-group_scores(s, spec.n_group), axis=1)
        ok &= (g[:, spec.topk_group - 1] - g[:, spec.topk_group]) >= margin
    return ok


# --------------------------------------------------------------------------
# Dispatch: counts, offsets, stable permutation, gather
# --------------------------------------------------------------------------


def expert_capacity(capacity_factor, T: int, k: int, E: int) -> int:
    """Slots per expert, capacity = capacity_factor * (T * k / E) ("Expert-
    Parallel MoE Inference", §Capacity factor and token dropping), rounded up
    to whole slots (so a factor of 1.0 provisions at least the average load).
    Exact: the factor is taken as the decimal it is written as (1.1 is 11/10).
    0 means no limit (the dropless path) and is returned for factors <= 0."""
    cf = capacity_factor if isinstance(capacity_factor, Fraction) else Fraction(str(capacity_factor))
    if cf <= 0:
        return 0
    return int(math.ceil(cf * T * k / E))


def dispatch(topk_idx: np.ndarray, E: int, capacity: int = 0):
    """Expert-contiguous layout of the T*k assignments a = t*k + j.

    counts[e] = number of assignments to e (the demand); assignments claim
    their expert's rows in increasing a.  With capacity > 0 each expert has
    that many slots ("each routed token checks whether the target expert
    still has a free capacity slot", "Expert-Parallel MoE Inference",
    §Deeper Analysis, Figure 2): an assignment finding its expert full is
    dropped (inv_pos = -1, no row).  offsets = exclusive prefix sum of the
    kept counts.
    Returns counts[E], offsets[E+1], perm_token[offsets[E]] (row -> token),
    inv_pos[T*k] (assignment -> row, or -1).  This buffer is what the dispatch
    exchange ships to the expert owners (same page, §The all-to-all dispatch
    and combine, step by step, Figure 3).
    """
    T, k = topk_idx.shape
    a_exp = topk_idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in a_exp:
        counts[e] += 1
    kept = counts if capacity <= 0 else np.minimum(counts, capacity)
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + kept[e]
    nxt = offsets[:-1].copy()
    used = np.zeros(E, dtype=np.int64)
    perm_token = np.empty(offsets[E], dtype=np.int64)
    inv_pos = np.empty(T * k, dtype=np.int64)
    for a, e in enumerate(a_exp):
        if capacity > 0 and used[e] == capacity:
            inv_pos[a] = -1  # overflow: dropped
            continue
        used[e] += 1
        p = nxt[e]
        nxt[e] += 1
        inv_pos[a] = p
        perm_token[p] = a // k
    return (counts.astype(np.int32), offsets.astype(np.int32),
            perm_token.astype(np.int32), inv_pos.astype(np.int32))


# --------------------------------------------------------------------------
# Capacity overflow rerouted to the next-best expert
# --------------------------------------------------------------------------


def reroute_candidates(s: np.ndarray, spec: RouteSpec):
    """The experts a token's overflow may move to, best first: its eligible
    experts ranked right after its top-k (ranks k .. 2k-1 in the same
    (score descending, id ascending) order; -1 past the eligible ones), and
    the gate each would carry: its score, divided by the sum of the chosen
    k's scores when the gates are renormalised (the denominator of the
    token's other gates), else the score itself.  ("Expert-Parallel MoE
    Inference", §Capacity factor and token dropping: overflow tokens are
    rerouted to their next-best expert.)
    -> (cand_idx [T, k] int32, cand_w [T, k] float64)."""
    T, E = s.shape
    k = spec.k
    masked = np.where(eligible(s, spec), s, -np.inf)
    order = _order_desc(masked)
    cand = np.full((T, k), -1, dtype=np.int64)
    n = min(k, E - k)
    if n > 0:
        c = order[:, k:k + n]
        ok = np.isfinite(np.take_along_axis(masked, c, axis=1))
        cand[:, :n] = np.where(ok, c, -1)
    if spec.renorm:
        den = np.take_along_axis(s, order[:, :k], axis=1).sum(axis=1, keepdims=True)
    else:
        den = np.ones((T, 1))
    cw = np.where(cand >= 0, np.take_along_axis(s, np.maximum(cand, 0), axis=1) / den, 0.0)
    return cand.astype(np.int32), cw


def dispatch_reroute(topk_idx: np.ndarray, topk_w: np.ndarray, cand_idx: np.ndarray,
                     cand_w: np.ndarray, E: int, capacity: int):
    """Expert capacity with overflow rerouted to the next-best expert.

    Pass 1 is dispatch() with the capacity: assignments a = t*k + j claim a
    slot of their own expert in increasing a; those finding it full overflow.
    Pass 2: the m-th overflowed assignment of a token (counting in increasing
    j) is offered the token's candidate m (reroute_candidates); the offers
    claim the slots their expert has left after pass 1, in increasing a.  An
    offer finding no slot, or an overflow with no candidate, is dropped.
    Rows of an expert: its pass-1 rows, then its pass-2 rows, each group in
    increasing a.
    Returns counts[E] (the demand of the top-k, as dispatch()), offsets[E+1],
    perm_token[offsets[E]], inv_pos[T*k] (row of the copy that serves the
    assignment, or -1), gates [T, k] (the gate of the serving copy: topk_w
    for its own expert, the candidate's gate when rerouted, 0 when dropped)
    and served [T, k] (the serving expert, -1 when dropped)."""
    T, k = topk_idx.shape
    n = T * k
    a_exp = topk_idx.reshape(-1).astype(np.int64)
    counts = np.zeros(E, dtype=np.int64)
    for e in a_exp:
        counts[e] += 1
    # pass 1
    used = np.zeros(E, dtype=np.int64)
    own = np.zeros(n, dtype=bool)
    for a, e in enumerate(a_exp):
        if used[e] < capacity:
            used[e] += 1
            own[a] = True
    kept1 = used.copy()
    # offers: the token's m-th overflow gets its candidate m
    offer = np.full(n, -1, dtype=np.int64)
    offer_m = np.full(n, -1, dtype=np.int64)
    for t in range(T):
        m = 0
        for j in range(k):
            a = t * k + j
            if not own[a]:
                offer[a] = cand_idx[t, m]
                offer_m[a] = m
                m += 1
    # pass 2: offers claim what pass 1 left, in increasing a
    rer = np.zeros(n, dtype=bool)
    for a in range(n):
        c = offer[a]
        if c >= 0 and used[c] < capacity:
            used[c] += 1
            rer[a] = True
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + used[e]
    nxt = offsets[:-1].copy()
    perm_token = np.empty(offsets[E], dtype=np.int64)
    inv_pos = np.full(n, -1, dtype=np.int64)
    served = np.full(n, -1, dtype=np.int64)
    gates = np.zeros(n)
    for a in range(n):          # pass-1 rows of every expert
        if own[a]:
            e = a_exp[a]
            inv_pos[a], served[a], gates[a] = nxt[e], e, topk_w[a // k, a % k]
            perm_token[nxt[e]] = a // k
            nxt[e] += 1
    assert np.array_equal(nxt, offsets[:-1] + kept1)
    for a in range(n):          # then the rerouted rows
        if rer[a]:
            c = offer[a]
            inv_pos[a], served[a], gates[a] = nxt[c], c, cand_w[a // k, offer_m[a]]
            perm_token[nxt[c]] = a // k
            nxt[c] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32), perm_token.astype(np.int32),
            inv_pos.astype(np.int32), gates.reshape(T, k), served.astype(np.int32).reshape(T, k))


def gather_rows(x: np.ndarray, perm_token: np.ndarray) -> np.ndarray:
    """x_perm[p] = x[perm_token[p]] (the dispatch payload, one copy per
    assignment)."""
    return x[np.asarray(perm_token, dtype=np.int64)]


# --------------------------------------------------------------------------
# Expert FFN (grouped) and combine
# --------------------------------------------------------------------------


def silu(u: np.ndarray) -> np.ndarray:
    return u / (1.0 + np.exp(-u))


def swiglu_expert(xr, w1, w3, w2, act: str):
    """One expert on its rows: h = round(silu(x W1) * (x W3)), y = round(h W2).
    w1, w3: [f][d]; w2: [d][f] (out x in, float64)."""
    u = xr @ w1.T
    v = xr @ w3.T
    h = round_act(silu(u) * v, act)
    y = round_act(h @ w2.T, act)
    return h, y


ExpertFn = Callable[[int], Sequence[np.ndarray]]  # e -> (w1, w3, w2) float64


def grouped_ffn(x_perm: np.ndarray, offsets: np.ndarray, expert_weights: ExpertFn, act: str,
                rows: Optional[np.ndarray] = None):
    """Expert e transforms rows [offsets[e], offsets[e+1]) of x_perm; experts
    with no rows are skipped.  ``rows`` (optional, sorted) restricts the
    computation to those rows of the buffer; other rows are left NaN.
    -> (h [R, f], y_perm [R, d])."""
    R = x_perm.shape[0]
    want = np.ones(R, dtype=bool) if rows is None else np.isin(np.arange(R), rows)
    h = y = None
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = np.nonzero(want[lo:hi])[0] + lo
        if sel.size == 0:
            continue
        w1, w3, w2 = expert_weights(e)
        he, ye = swiglu_expert(x_perm[sel], w1, w3, w2, act)
        if h is None:
            h = np.full((R, he.shape[1]), np.nan)
            y = np.full((R, ye.shape[1]), np.nan)
        h[sel] = he
        y[sel] = ye
    if h is None:
        raise ValueError("no rows")
    return h, y


def combine(y_perm: np.ndarray, inv_pos: np.ndarray, topk_w: np.ndarray, act: str,
            shared_y: Optional[np.ndarray] = None) -> np.ndarray:
    """out[t] = round(sum_j g[t,j] * y_perm[inv_pos[t*k+j]] (+ shared_y[t])):
    expert outputs brought back to token order and summed weighted by the
    gates (the weighted-sum combine of "Tensor vs Expert vs Data Parallelism",
    §Deeper Analysis, Figure 2)."""
    T, k = topk_w.shape
    out = np.zeros((T, y_perm.shape[1]))
    pos = np.asarray(inv_pos, dtype=np.int64).reshape(T, k)
    for j in range(k):
        # a dropped assignment (inv_pos -1) skips the expert: no contribution
        kept = pos[:, j] >= 0
        out[kept] += topk_w[kept, j: j + 1] * y_perm[pos[kept, j]]
    if shared_y is not None:
        out += shared_y
    return round_act(out, act)


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------


@dataclass
class LayerResult:
    topk_idx: np.ndarray
    topk_w: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    perm_token: np.ndarray
    inv_pos: np.ndarray
    x_perm: np.ndarray
    h: np.ndarray
    y_perm: np.ndarray
    shared_h: Optional[np.ndarray]
    shared_y: Optional[np.ndarray]
    out: np.ndarray
    gates: Optional[np.ndarray] = None    # gate of each assignment's serving copy (reroute)
    served: Optional[np.ndarray] = None   # serving expert per assignment, -1: dropped (reroute)


def layer_forward(x, w_router, bias, spec: RouteSpec, E: int, expert_weights: ExpertFn, act: str,
                  shared: Optional[Sequence[np.ndarray]] = None, capacity: int = 0,
                  fp8_dispatch: bool = False, overflow: str = "drop") -> LayerResult:
    """The whole layer: route, dispatch, grouped SwiGLU FFN, shared expert,
    combine.  x, w_router and the weights are float64 values of the stored
    inputs.  Without a capacity the layer is token-wise: running it on a
    subset of the tokens gives exactly those tokens' results.  With a
    capacity (slots per expert) overflow assignments are dropped and the
    kept ones keep their gates; with overflow="reroute" they go to their
    token's next-best expert first (dispatch_reroute) and carry that
    expert's gate.  With fp8_dispatch the dispatched rows are the
    block-scaled E4M3 payload of x (quantize_fp8_blocks) as the routed
    experts' input; the router and the shared expert read x itself."""
    idx, gw, s = route(x, w_router, bias, spec)
    gates = served = None
    if capacity > 0 and overflow == "reroute":
        cand, cw = reroute_candidates(s, spec)
        counts, offsets, perm_token, inv_pos, gates, served = dispatch_reroute(idx, gw, cand, cw, E, capacity)
    elif overflow in ("drop", "reroute"):
        counts, offsets, perm_token, inv_pos = dispatch(idx, E, capacity)
    else:
        raise ValueError(overflow)
    payload = dequantize_fp8_blocks(*quantize_fp8_blocks(x)) if fp8_dispatch else x
    x_perm = gather_rows(payload, perm_token)
    h, y_perm = grouped_ffn(x_perm, offsets, expert_weights, act)
    sh = sy = None
    if shared is not None:
        sh, sy = swiglu_expert(x, shared[0], shared[1], shared[2], act)
    out = combine(y_perm, inv_pos, gw if gates is None else gates, act, sy)
    return LayerResult(idx, gw, counts, offsets, perm_token, inv_pos, x_perm, h, y_perm, sh, sy, out,
                       gates, served)
