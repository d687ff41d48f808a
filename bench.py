#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

One step = one moe_layer_forward (router, dispatch, grouped SwiGLU FFN, shared
expert when present, combine) over one batch of seeded synthetic tokens, with
inputs already resident in HBM.  Prints one JSON line:

  value       tokens/s = T * steps / wall time of the timed steps
  roofline    the routed gate-up GEMM (+SwiGLU) kernel against the bf16 MFMA
              peak, or, for decode-shaped layers, the whole layer's
              algorithmic bytes against HBM bandwidth; its duration comes from
              HIP events the library records around each stage inside the
              timed steps, on the stream the kernels run on
  cpu_baseline the float64 oracle on a bounded token sample, host cores
  stages_gbps achieved GB/s of the route, dispatch and combine stages
              (algorithmic bytes over the stage's event time)
  cold_cache  after the timed steps, as many more steps each preceded by a
              512 MiB write that evicts the L2s and the 256 MB Infinity Cache,
              each timed by its own events: medians of the step and stages

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s per MI355X; grouped-GEMM % MFMA peak; decode % HBM BW"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # dense fp8 MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
DEFAULT_WORKLOAD = "mixtral8x7b_prefill_bf16"
DECODE_WORKLOADS = {"dsv3_decode_bf16"}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=None, help="tokens for the oracle timing")
    p.add_argument("--capacity-factor", type=float, default=0.0,
                   help="expert capacity = factor * T * k / E slots (0: dropless); overflow is dropped")
    p.add_argument("--overflow", choices=("drop", "reroute"), default="drop",
                   help="with --capacity-factor: drop overflow assignments, or reroute them to the token's "
                        "next-best expert first")
    p.add_argument("--dispatch-fp8", action="store_true",
                   help="dispatch the block-scaled E4M3 payload of x (fp8 x fp8 gate-up GEMM with E4M3 weights)")
    p.add_argument("--graph", action="store_true",
                   help="time replays of one HIP graph of the layer forward (captured once); the per-stage "
                        "times then come from a separate traced eager pass")
    p.add_argument("--no-cold", action="store_true", help="skip the cold-cache repetitions")
    p.add_argument("--w-layout", choices=("auto", "rowmajor", "kblocked"), default="auto",
                   help="routed expert weight layout; auto: kblocked for bf16 / fp8 weights (packed "
                        "once after upload, before any timing), rowmajor for fp32")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the library's sources without their comments and blank lines:
    it changes with the code the counters in profiles/traffic.json were
    taken on, not with its documentation."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "mixture_experts_layer_36_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            code = [ln.split("//", 1)[0].rstrip() for ln in fh]
        h.update(name.encode() + "\n".join(ln for ln in code if ln).encode())
    return h.hexdigest()[:16]


def layer_bytes(w, counts) -> float:
    """Algorithmic HBM bytes of one layer forward: x, router weight and bias,
    the touched experts' weights (+ scales), the shared expert, out, and the
    routing outputs (topk idx + w)."""
    ab = 4 if w.act == "f32" else 2
    wb = {"f32": 4, "bf16": 2, "e4m3": 1}[w.wdt]
    touched = int((counts > 0).sum())
    per_expert = 3 * w.d * w.f * wb + (2 * w.f + w.d) * 4 * (w.wdt == "e4m3")
    b = w.T * w.d * ab * 2 + w.E * w.d * ab + w.E * 4 + touched * per_expert
    b += 3 * w.d * w.f_shared * ab + 8 * w.T * w.k
    return float(b)


def fp8_gate_up(w) -> bool:
    """Whether the library runs the gate-up GEMM fp8 x fp8 for w: the fp8
    payload with E4M3 weights on the prefill kernel's shapes (at least 1024
    routed rows and 128 per expert on average, K a multiple of 64)."""
    rows = w.T * w.k
    return (w.dispatch_fp8 and w.wdt == "e4m3" and rows >= 1024 and rows // w.E >= 128
            and w.d % 64 == 0)


def gathers_blocked(w) -> bool:
    """Whether the layer gathers x_perm into K-blocked planes rather than
    fusing the gather into the gate-up GEMM: bf16 activations without the
    payload, f >= 4096, on the prefill kernel's shapes (the library's rule)."""
    rows = w.T * w.k
    return (w.act == "bf16" and not w.dispatch_fp8 and w.f >= 4096 and rows >= 1024
            and rows // w.E >= 128 and rows * w.d * 2 < (1 << 31))


def stage_bytes(w, has_bias: bool, kept: int) -> dict:
    """Algorithmic bytes of the memory-bound stages of the layer path:
    route = x + router weight (+ bias) + the top-k indices and gates written;
    dispatch = the index work (top-k ids read, per-expert counts and offsets,
    perm_token and inv_pos written) -- the row gather itself is fused into the
    gate-up GEMM's activation loads, or, for wide experts, the kept rows of x
    read and x_perm written; combine = the routed rows read (T*k, or
    those kept under a capacity), the
    indices and gates, out written (+ the shared expert's rows read)."""
    ab = 4 if w.act == "f32" else 2
    tk = w.T * w.k
    route = w.T * w.d * ab + w.E * w.d * ab + (w.E * 4 if has_bias else 0) + 8 * tk
    dispatch = 4 * tk + 8 * tk + 8 * w.E
    if gathers_blocked(w):
        dispatch += 2 * kept * w.d * ab
    if w.dispatch_fp8:  # x read once, its payload (codes + scale rows) written in token order
        dispatch += w.T * w.d * ab + w.T * (w.d + (w.d // 32 + 15) // 16 * 16)
    combine = kept * w.d * ab + 8 * tk + w.T * w.d * ab + (w.T * w.d * ab if w.f_shared else 0)
    return {"route": float(route), "dispatch": float(dispatch), "combine": float(combine)}


# Ceilings measured on MI355X by separate probes (not in this run): a
# register-only loop of 32x32x16 bf16 MFMAs on every SIMD, the same with the
# block-scaled fp8 32x32x64 MFMA, and a streaming read of 8 GiB with 16-byte
# loads.
MFMA_LOOP_TFLOPS = 1785.0
MFMA_LOOP_TFLOPS_FP8 = 4614.0
STREAM_READ_GBS = 6300.0
EVICT_BYTES = 512 << 20


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


def cpu_baseline(w, L, host_experts, sample):
    """The float64 oracle on the first `sample` tokens (the layer is
    token-wise, so this is exactly those tokens' forward)."""
    import oracle as O
    from threadpoolctl import threadpool_info

    x, wr, b = O.decoded_inputs(L)
    xs = x[:sample]

    def expert(e):
        ew = host_experts[e]
        w1, w3, w2 = O.decode(ew.w1, w.wdt), O.decode(ew.w3, w.wdt), O.decode(ew.w2, w.wdt)
        if w.wdt == "e4m3":
            w1 = w1 * ew.s1.astype(np.float64)[:, None]
            w3 = w3 * ew.s3.astype(np.float64)[:, None]
            w2 = w2 * ew.s2.astype(np.float64)[:, None]
        return w1, w3, w2

    shared = O.adapters.decoded_shared(L)
    # with a capacity factor the sample gets its own slots (factor * sample * k / E)
    cap = O.expert_capacity(getattr(w, "capacity_factor", 0), sample, w.k, w.E)
    t0 = time.perf_counter()
    O.layer_forward(xs, wr, b, O.workload_spec(w), w.E, expert, w.act, shared, capacity=cap,
                    fp8_dispatch=w.dispatch_fp8, overflow=w.overflow)
    dt = time.perf_counter() - t0
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] or [1])
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in pools if p.get("user_api") == "blas"})
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(sample / dt, 3), "unit": "tokens/s", "cores": int(threads),
            "cpu_model": cpu_model, "blas": blas,
            "kind": "oracle",
            "sample": f"first {sample} of {w.T} tokens, full layer forward in float64 "
                      f"(routing, dispatch, experts, combine), {dt:.2f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_36_amd as moe
    from synth import DEFAULT_SEED, BY_NAME, LayerInputs
    from synth.device import DeviceLayer

    if args.calibrate_copy:
        calibrate_copy()
        return
    w = BY_NAME[args.workload]
    seed = DEFAULT_SEED[w.name] if args.seed is None else args.seed
    if args.capacity_factor > 0:
        w = w.scaled(capacity_factor=args.capacity_factor)
    if args.dispatch_fp8:
        w = w.scaled(dispatch_fp8=True)
    if args.overflow != "drop":
        w = w.scaled(overflow=args.overflow)
    L = LayerInputs(w, seed)
    host_experts = {}

    # upload expert by expert, keeping host copies for the CPU baseline
    orig = L.expert

    def keep(e):
        ew = orig(e)
        if not args.no_cpu_baseline:
            host_experts[e] = ew
        return ew

    L.expert = keep
    dev = DeviceLayer(L)
    L.expert = orig

    layout = args.w_layout if args.w_layout != "auto" else ("rowmajor" if w.wdt == "f32" else "kblocked")
    if layout == "kblocked":  # the one-time load-time transform; weights stay resident
        dev.w1, dev.w3, dev.w2 = (moe.pack_weights(t) for t in (dev.w1, dev.w3, dev.w2))
        torch.cuda.synchronize()
    desc = moe.Desc.from_attrs(w)
    desc.w_layout = moe.W_KBLOCKED if layout == "kblocked" else moe.W_ROWMAJOR
    out = torch.empty((w.T, w.d), dtype=dev.x.dtype, device="cuda")
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    ws = moe.workspace(desc)

    def step(trace=None):
        moe.layer_forward(desc, dev.x, dev.w_router, dev.bias, dev.w1, dev.w3, dev.w2, dev.s1,
                          dev.s3, dev.s2, dev.sw1, dev.sw3, dev.sw2, out, idx, gw, counts, ws,
                          trace=trace)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    traces = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.TRACE_EVENTS)]
              for _ in range(args.steps)]
    for tr in traces:  # create the HIP events before the timed region
        for ev in tr:
            ev.record()
    torch.cuda.synchronize()

    if args.graph:
        # per-stage times from a traced eager pass; the timed steps replay
        # one captured graph of the forward
        for i in range(args.steps):
            step(traces[i])
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(traces[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

    cold = None
    if not args.no_cold:
        # cold-cache repetitions, outside the timed region: the eviction
        # write runs between a step's events, never inside them
        evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
        cold_tr = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.TRACE_EVENTS)]
                   for _ in range(args.steps)]
        for tr in cold_tr:
            for ev in tr:
                ev.record()
        torch.cuda.synchronize()
        for i in range(args.steps):
            evict.fill_(i & 0xff)
            step(cold_tr[i])
        torch.cuda.synchronize()
        cms = np.array([[tr[j].elapsed_time(tr[j + 1]) for j in range(moe.TRACE_EVENTS - 1)]
                        for tr in cold_tr])
        cstep = float(np.median([tr[0].elapsed_time(tr[-1]) for tr in cold_tr]))
        cold = {"evict_bytes": EVICT_BYTES, "reps": args.steps, "step_ms_median": round(cstep, 4),
                "tokens_per_s": round(w.T / (cstep * 1e-3), 1),
                "stages_us_median": {name: round(float(np.median(cms[:, j])) * 1e3, 2)
                                     for j, name in enumerate(moe.TRACE_STAGES)}}
        del evict

    stage_ms = np.array([[tr[j].elapsed_time(tr[j + 1]) for j in range(moe.TRACE_EVENTS - 1)]
                         for tr in traces])
    stage_us = {name: round(float(stage_ms[:, j].mean()) * 1e3, 2)
                for j, name in enumerate(moe.TRACE_STAGES)}
    step_events = [tr[0].elapsed_time(tr[-1]) for tr in traces]
    step_event_ms = float(np.mean(step_events))
    c = counts.cpu().numpy()
    assert int(c.sum()) == w.T * w.k, "routing lost assignments"
    cap = desc.capacity
    rows_dev = torch.empty(w.E, dtype=torch.int32, device="cuda")
    moe.layer_rows(desc, ws, rows_dev)
    kept = rows_dev.cpu().numpy()
    n_assign = int(kept.sum())  # rows the experts process (dropped ones removed, rerouted ones added)
    own_kept = int(np.minimum(c, cap).sum()) if cap > 0 else n_assign

    ms_per_step = elapsed * 1e3 / args.steps
    value = w.T * args.steps / elapsed
    gemm1_s = stage_ms[:, 2].mean() * 1e-3
    flops_gemm1 = 4.0 * w.d * w.f * n_assign
    flops_all = 6.0 * w.d * w.f * n_assign + 6.0 * w.d * w.f_shared * w.T
    if w.name in DECODE_WORKLOADS:
        layer_s = step_event_ms * 1e-3
        achieved = layer_bytes(w, c) / layer_s / 1e9
        roof = {"bound": "hbm", "kernel": "whole layer (all kernels)", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "algorithmic_bytes": layer_bytes(w, c),
                "frac_of_measured_read_ceiling": round(achieved / STREAM_READ_GBS, 4)}
    else:
        achieved = flops_gemm1 / gemm1_s / 1e12
        f8 = fp8_gate_up(w)
        peak = PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS
        kern = ("gemm_big_fp8_kernel: fp8 x fp8 block-scaled MFMA" if f8 else
                "gemm_big_kernel / gemm_mfma_kernel, EPI_SWIGLU")
        roof = {"bound": "mfma", "kernel": f"routed gate-up GEMM + SwiGLU ({kern})",
                "mfma_dtype": "fp8" if f8 else "bf16",
                "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "algorithmic_flops": flops_gemm1,
                "avg_launch_us": round(gemm1_s * 1e6, 2)}
        roof["frac_of_measured_mfma_ceiling"] = round(achieved / (MFMA_LOOP_TFLOPS_FP8 if f8 else MFMA_LOOP_TFLOPS),
                                                      4)
    # HBM bytes per launch of that kernel from the committed rocprofv3
    # FETCH_SIZE / WRITE_SIZE passes, valid only while the kernels are unchanged
    roof["traffic"] = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get(w.name + ("+dispatch_fp8" if w.dispatch_fp8 else ""))
        if ent and ent.get("source_hash") == kernel_source_hash():
            roof["traffic"] = ent.get("bytes_per_launch")

    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16, fp8 gate-up" if fp8_gate_up(w) else "bf16") if w.act == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k,
                   "score": w.score, "n_group": w.n_group, "topk_group": w.topk_group,
                   "f_shared": w.f_shared, "act": w.act, "weights": w.wdt, "seed": seed,
                   "capacity_factor": w.capacity_factor, "overflow": w.overflow,
                   "dispatch_fp8": w.dispatch_fp8, "weight_layout": layout,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "roofline": roof,
        # all expert GEMMs (routed gate-up and down, shared expert) over their stages
        "ffn_tflops": round(flops_all / (float(stage_ms[:, 2:5].sum(axis=1).mean()) * 1e-3) / 1e12, 1),
        "ffn_frac_of_bf16_peak": round(flops_all / (float(stage_ms[:, 2:5].sum(axis=1).mean()) * 1e-3) / 1e12
                                       / PEAK_BF16_TFLOPS, 4),
        "stages_us": stage_us,
        "stages_gbps": {k: round(v / (stage_us[k] * 1e-6) / 1e9, 1)
                        for k, v in stage_bytes(w, dev.bias is not None, n_assign).items()},
        "step_event_ms": round(step_event_ms, 4),
        "step_event_ms_median": round(float(np.median(step_events)), 4),
        "load": {"max_over_mean": round(float(c.max() / c.mean()), 3),
                 "experts_touched": int((c > 0).sum()), "experts": w.E},
        "capacity": {"factor": w.capacity_factor, "slots_per_expert": cap,
                     "overflow": w.overflow, "dropped_fraction": round(1.0 - n_assign / (w.T * w.k), 5),
                     "rerouted_fraction": round((n_assign - own_kept) / (w.T * w.k), 5)},
        "cold_cache": cold,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or {"mixtral8x7b_prefill_bf16": 4096, "tiny_f32": 64}.get(w.name, 16)
        rec["cpu_baseline"] = cpu_baseline(w, L, host_experts, min(sample, w.T))
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
