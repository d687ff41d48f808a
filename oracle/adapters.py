"""Glue between the seeded inputs (synth) and the float64 oracle.

TEST INFRASTRUCTURE.  Decodes stored inputs exactly to float64 and exposes the
oracle's margin rule as the row-acceptance callback the input generator takes.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import RouteSpec, decode, selection_margin_ok


def workload_spec(w) -> RouteSpec:
    return RouteSpec(k=w.k, score=w.score, renorm=w.renorm, n_group=w.n_group,
                     topk_group=w.topk_group)


def decoded_router(L):
    w = L.w
    wr = decode(L.w_router, w.act)
    bias = None if L.bias is None else L.bias.astype(np.float64)
    return wr, bias


def decoded_inputs(L):
    """-> (x, w_router, bias) as float64 values of the stored inputs."""
    wr, bias = decoded_router(L)
    return decode(L.x, L.w.act), wr, bias


def decoded_expert(L, e: int):
    """Expert e's (W1, W3, W2) as float64 values; e4m3 codes times their
    per-output-channel scale (exact in float64)."""
    w = L.w
    ew = L.expert(e)
    w1, w3, w2 = decode(ew.w1, w.wdt), decode(ew.w3, w.wdt), decode(ew.w2, w.wdt)
    if w.wdt == "e4m3":
        w1 = w1 * ew.s1.astype(np.float64)[:, None]
        w3 = w3 * ew.s3.astype(np.float64)[:, None]
        w2 = w2 * ew.s2.astype(np.float64)[:, None]
    return w1, w3, w2


def decoded_shared(L):
    sh = L.shared()
    if sh is None:
        return None
    a = L.w.act
    return decode(sh.w1, a), decode(sh.w3, a), decode(sh.w2, a)


def margin_acceptor(margin: float = 1e-3, order_margin: float = 2e-5):
    """Row-acceptance callback for synth.LayerInputs(accept=...).  The chosen
    set is kept ``margin`` from the next expert (and the kept groups from the
    next group); the order of the k outputs, and for a workload that reroutes
    capacity overflow the order of its reroute candidates (ranks k .. 2k), is
    kept by ``order_margin`` between adjacent scores, twenty times the float32
    router's score error (~1e-6)."""

    def accept(L, rows, x_rows):
        wr, bias = decoded_router(L)
        w = L.w
        rr = getattr(w, "overflow", "drop") == "reroute" and getattr(w, "capacity_factor", 0) > 0
        return selection_margin_ok(decode(x_rows, w.act), wr, bias, workload_spec(w), margin,
                                   ranks=2 * w.k if rr else 0, order_margin=order_margin)

    return accept
