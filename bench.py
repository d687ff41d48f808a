#!/usr/bin/env python3
"""Throughput of the MoE layer forward on one MI355X.

One step = one moe_layer_forward (router, dispatch, grouped SwiGLU FFN, shared
expert when present, combine) over one batch of seeded synthetic tokens, with
inputs already resident in HBM.  The default workload is the DeepSeek-V3-shaped
prefill layer with skewed routing (T=16384, the largest single-GPU
configuration); the same line carries a `decode` record for the
DeepSeek-V3-shaped decode layer (T=256), which is bound by HBM bandwidth.
Prints one JSON line:

  value       tokens/s = T * steps / wall time of the timed steps
  roofline    the gate-up GEMM (+SwiGLU) launch against the peak of the MFMA
              type it runs (its flops include the shared expert's when the
              shared expert runs as a segment of the same launch), or, for
              decode-shaped layers, the whole layer's algorithmic bytes against
              HBM bandwidth; durations come from HIP events the library
              records around each stage inside the timed steps, on the stream
              the kernels run on
  ceilings    measured in this run: the GEMM's MFMA pattern alone (bf16 and fp8,
              random and constant operands, each sustained ~1.6 s, with the
              socket power and graphics clock read meanwhile) and a streaming
              read (calib/ceilings.hip)
  sustained   the same step repeated for ~2 s after the timed steps, with the
              socket power and graphics clock read meanwhile (amdsmi)
  cpu_baseline the float64 oracle's forward of a bounded token sample on the
              host cores (the fp64 decode of the expert weights timed apart)
  stages_gbps achieved GB/s of the route, dispatch and combine stages
              (algorithmic bytes over the stage's event time)
  cold_cache  after the timed steps, as many more steps each preceded by a
              512 MiB write that evicts the L2s and the 256 MB Infinity Cache,
              each timed by its own events: medians of the step and stages

    python bench.py [--steps K] [--warmup W] [--workload NAME]
    python bench.py --calibrate-mfma | --calibrate-stream | --calibrate-copy
    python bench.py --summarize-trace DIR --warmup W --steps K
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
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
CALIB_LIB = os.path.join(ROOT, "mixture_experts_layer_36_amd", "lib", "libmoe_calib.so")
DEFAULT_WORKLOAD = "dsv3_prefill_skew_bf16"
DECODE_WORKLOAD = "dsv3_decode_bf16"
DECODE_WORKLOADS = {"dsv3_decode_bf16"}
# the decode leg times this many steps per prefill step: at least 100 with the
# default 20 (a decode step is ~4 ms)
DECODE_STEPS_PER_STEP = 5
EVICT_BYTES = 512 << 20
XCDS = 8  # MI355X: 8 XCDs of 32 compute units
# oracle tokens timed per workload: about 10 s of float64 compute on a
# 16-core host (the whole batch where it is small enough)
CPU_SAMPLE = {"tiny_f32": 64, "mixtral8x7b_prefill_bf16": 4096, "dsv3_decode_bf16": 256,
              "dsv3_prefill_skew_bf16": 4096, "qwen_moe_fp8_skew": 8192, "dsv3_ep8_shard_bf16": 2048}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=None, help="tokens for the oracle timing")
    p.add_argument("--no-decode-leg", action="store_true",
                   help=f"skip the {DECODE_WORKLOAD} record the default workload's line carries")
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
    p.add_argument("--no-ceilings", action="store_true", help="skip the in-run MFMA / stream ceiling probes")
    p.add_argument("--sustain-seconds", type=float, default=2.0,
                   help="after the timed steps, repeat the step this long with power sampling (0: skip)")
    p.add_argument("--w-layout", choices=("auto", "rowmajor", "kblocked"), default="auto",
                   help="routed expert weight layout; auto: kblocked for bf16 / fp8 weights (packed "
                        "once after upload, before any timing), rowmajor for fp32")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (counter calibration)")
    p.add_argument("--calibrate-mfma", action="store_true", help="only run the bf16 and fp8 MFMA-loop probes")
    p.add_argument("--calibrate-stream", action="store_true", help="only run the streaming-read probe")
    p.add_argument("--summarize-counters", metavar="DIR", default=None,
                   help="summarise rocprofv3 --pmc counter CSVs under DIR (no GPU): per kernel, the mean of "
                        "each counter over the dispatches of the timed steps (--warmup / --steps as above)")
    p.add_argument("--write-traffic", metavar="WORKLOAD", default=None,
                   help="(no GPU) HBM bytes per launch of --kernel from rocprofv3 --pmc FETCH_SIZE (--fetch DIR) "
                        "and WRITE_SIZE (--write DIR) passes of the timed steps, each scaled by what the same "
                        "counter reads for --calibrate-copy (--copy-fetch DIR, --copy-write DIR); written into "
                        "profiles/traffic.json with the kernel source hash, and the algorithmic bytes from the "
                        "experts the --bench-line JSON of the same build touched")
    p.add_argument("--kernel", default=None, help="with --write-traffic: kernel name substring ('*': every kernel "
                                                  "the --pmc runs collected, i.e. those of one layer step)")
    p.add_argument("--fetch", default=None)
    p.add_argument("--write", default=None)
    p.add_argument("--copy-fetch", default=None)
    p.add_argument("--copy-write", default=None)
    p.add_argument("--bench-line", default=None)
    p.add_argument("--profile", default=None, help="with --write-traffic: the trace summary the entry refers to")
    p.add_argument("--summarize-trace", metavar="DIR", default=None,
                   help="summarise a rocprofv3 --kernel-trace CSV under DIR (no GPU): per-kernel calls and "
                        "average, and the steady-state average over the timed steps given by --warmup and "
                        "--steps")
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


def progress(msg: str):
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------ algorithmic work

def layer_bytes(w, counts=None, touched=None) -> float:
    """Algorithmic HBM bytes of one layer forward: x, router weight and bias,
    the touched experts' weights (+ scales), the shared expert, out, and the
    routing outputs (topk idx + w)."""
    ab = 4 if w.act == "f32" else 2
    wb = {"f32": 4, "bf16": 2, "e4m3": 1}[w.wdt]
    if touched is None:
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


def shared_fused(w) -> bool:
    """Whether the shared expert runs as one more segment of the routed GEMM
    launches (the library does so when its weights share the routed dtype)."""
    return w.f_shared > 0 and w.wdt == w.act


def gathers_blocked(w) -> bool:
    """Whether the layer gathers x_perm into K-blocked planes rather than
    fusing the gather into the gate-up GEMM: bf16 activations without the
    payload, f >= 4096, on the prefill kernel's shapes (the library's rule)."""
    rows = w.T * w.k
    return (w.act == "bf16" and not w.dispatch_fp8 and w.f >= 4096 and rows >= 1024
            and rows // w.E >= 128 and rows * w.d * 2 < (1 << 31))


def gate_up_bytes(w, touched: int) -> tuple:
    """Algorithmic HBM (read, write) bytes of the gate-up launch: the routed
    rows of x (T*k of them, as the fp8 payload where the launch takes it) and
    the touched experts' W1 and W3 (+ fp8 scales)
    read, h written; with the shared expert fused into the launch, also x and
    its W1, W3 read and its h written."""
    ab = 4 if w.act == "f32" else 2
    wb = {"f32": 4, "bf16": 2, "e4m3": 1}[w.wdt]
    rows = w.T * w.k
    # a routed row: bf16 x, or (fp8 x fp8 gate-up) its E4M3 codes and E8M0 scale row
    row_b = w.d + (w.d // 32 + 15) // 16 * 16 if fp8_gate_up(w) else w.d * ab
    rd = rows * row_b + touched * (2 * w.f * w.d * wb + 2 * w.f * 4 * (w.wdt == "e4m3"))
    wr = rows * w.f * ab
    if shared_fused(w):
        rd += w.T * w.d * ab + 2 * w.f_shared * w.d * ab
        wr += w.T * w.f_shared * ab
    return float(rd), float(wr)


def _counter_per_step(d: str, counter: str, kernel: str, warmup: int, steps: int) -> float:
    """Sum of `counter` over the dispatches of the kernels whose name holds
    `kernel` ('*': all) in the timed steps of a --pmc run, divided by steps: the
    value per launch when one such kernel runs per step."""
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    per = {}  # kernel -> {dispatch: value}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] != counter or (kernel != "*" and kernel not in row["Kernel_Name"]):
                    continue
                dd = per.setdefault(row["Kernel_Name"], {})
                key = (f, int(row["Dispatch_Id"]))
                dd[key] = dd.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernel {kernel!r} under {d}")
    total = 0.0
    for name, dd in per.items():
        v = [x for _, x in sorted(dd.items())]
        if len(v) % (warmup + steps):
            raise SystemExit(f"{name}: {len(v)} dispatches do not split into {warmup} + {steps} steps")
        total += sum(v[len(v) // (warmup + steps) * warmup:])
    return total / steps


# How the counter passes behind profiles/traffic.json are taken (repository
# root, on the GPU); <wl> is the workload, <flags> e.g. --dispatch-fp8.
TRAFFIC_COMMANDS = [
    "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <copy_f> -o run -- python3 bench.py --calibrate-copy",
    "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <copy_w> -o run -- python3 bench.py --calibrate-copy",
    "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex gemm_big --output-format csv -d <f> -o run -- python3 bench.py "
    "--no-cpu-baseline --no-decode-leg --no-cold --no-ceilings --sustain-seconds 0 --workload <wl> <flags> --steps 2 "
    "--warmup 1   (WRITE_SIZE into <w> likewise; the decode layer: --kernel-include-regex 'moe::' "
    "--kernel-exclude-regex 'pack_kblocked|segment_rows')",
    "python bench.py --write-traffic <wl>[+dispatch_fp8] --kernel '<gate-up kernel name>' (or '*') --fetch <f> "
    "--write <w> --copy-fetch <copy_f> --copy-write <copy_w> --bench-line <that workload's bench.py JSON line> "
    "--warmup 1 --steps 2",
]


def write_traffic(args):
    """profiles/traffic.json entry of one workload (see --write-traffic)."""
    from synth import BY_NAME
    name = args.write_traffic
    w = BY_NAME[name.split("+")[0]]
    if name.endswith("+dispatch_fp8"):
        w = w.scaled(dispatch_fp8=True)
    fetch = _counter_per_step(args.fetch, "FETCH_SIZE", args.kernel, args.warmup, args.steps)
    write = _counter_per_step(args.write, "WRITE_SIZE", args.kernel, args.warmup, args.steps)
    # the copy calibration: the 3 launches of the runtime's 1 GiB device copy
    cf = _counter_per_step(args.copy_fetch, "FETCH_SIZE", "copyBuffer", 0, 3)
    cw = _counter_per_step(args.copy_write, "WRITE_SIZE", "copyBuffer", 0, 3)
    n = 1 << 30
    rf, wf = n / (cf * 1024), n / (cw * 1024)
    ent = {"kernel": args.kernel if args.kernel != "*" else "whole layer (all kernels of one moe_layer_forward)",
           "source_hash": kernel_source_hash(),
           "read_bytes": round(fetch * 1024 * rf), "write_bytes": round(write * 1024 * wf),
           "fetch_size_kib": fetch, "write_size_kib": write,
           "copy_calibration": {"bytes": n, "read_factor": rf, "write_factor": wf}}
    ent["bytes_per_launch"] = ent["read_bytes"] + ent["write_bytes"]
    if args.bench_line:
        with open(args.bench_line) as fh:
            line = json.loads(fh.read().strip().splitlines()[-1])
        touched = line["load"]["experts_touched"]
        if args.kernel == "*":
            ent["algorithmic_bytes"] = layer_bytes(w, touched=touched)
        else:
            ent["algorithmic_read_bytes"], ent["algorithmic_write_bytes"] = gate_up_bytes(w, touched)
    if args.profile:
        ent["profile"] = args.profile
    tr = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
    tr["_commands"] = TRAFFIC_COMMANDS
    tr[name] = ent
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(tr, fh, indent=1)
        fh.write("\n")
    print(json.dumps({name: ent}, indent=1))


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


# ------------------------------------------------------------------ ceilings

def _calib_lib():
    if not os.path.exists(CALIB_LIB):
        raise ImportError(f"{CALIB_LIB} is missing: build with `python -m mixture_experts_layer_36_amd.build`")
    lib = ctypes.CDLL(CALIB_LIB)
    for fn in (lib.moe_calib_mfma_bf16_gemm, lib.moe_calib_mfma_fp8_gemm):
        fn.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.moe_calib_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_longlong), ctypes.c_int, ctypes.c_void_p]
    return lib


def _timed(launch, reps):
    """Median ms of `reps` launches, each bracketed by events on the current
    stream (the one the probe is launched on), after one untimed launch."""
    import torch
    launch()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        launch()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


class PowerSampler:
    """Socket power and graphics clock, read from the GPU's metrics table
    (amdsmi, read-only) every few ms on a thread while a sustained run goes on.
    Without amdsmi, or on any error from it, the summary is None."""

    # samples in the first 0.6 s of a window are dropped: the table's power
    # and clock readings trail the work by a fraction of a second
    SETTLE_S = 0.6

    def __init__(self):
        import threading
        self.samples, self.h, self.cap_w = [], None, None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self.h = amdsmi.amdsmi_get_processor_handles()[0]
            cap = amdsmi.amdsmi_get_power_cap_info(self.h).get("power_cap")
            self.cap_w = round(cap / 1e6, 1) if isinstance(cap, (int, float)) and cap > 0 else None
        except Exception:
            self.h = None

    def _run(self):
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self.h)
                self.samples.append((time.perf_counter(), m.get("current_socket_power"), m.get("current_gfxclk")))
            except Exception:
                pass
            time.sleep(0.004)

    def start(self):
        import threading
        if self.h is None:
            return
        self.samples = []
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self, t0: float, t1: float):
        """Medians over [t0 + SETTLE_S, t1], or None."""
        if self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        self._thread = None
        return self.summarize(self.samples, t0 + self.SETTLE_S, t1, self.cap_w)

    @staticmethod
    def summarize(samples, t0: float, t1: float, cap_w=None):
        """Medians of (time, socket W, gfx MHz) samples taken in [t0, t1];
        readings the table marks unavailable (0, 0xffff) are skipped."""
        win = [x for x in samples if t0 <= x[0] <= t1]

        def med(i):
            v = [x[i] for x in win if isinstance(x[i], (int, float)) and 0 < x[i] < 0xffff]
            return round(float(np.median(v)), 1) if v else None
        if not win:
            return None
        return {"socket_power_w_median": med(1), "gfxclk_mhz_median": med(2), "power_cap_w": cap_w,
                "samples": len(win)}


def _sustained(launch, seconds: float, sampler=None):
    """Launch repeatedly, in batches, until `seconds` have passed; returns
    (launches, wall seconds, power summary or None)."""
    import torch
    launch()
    torch.cuda.synchronize()
    if sampler:
        sampler.start()
    n, t0 = 0, time.perf_counter()
    while True:
        for _ in range(8):
            launch()
        n += 8
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    t1 = time.perf_counter()
    return n, t1 - t0, (sampler.stop(t0, t1) if sampler else None)


def ceilings(which=("mfma", "stream")) -> dict:
    """MFMA and streaming-read rates measured now, on this GPU."""
    import torch
    lib = _calib_lib()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"compute_units": cus}
    if "mfma" in which:
        # the MFMA pattern of a GEMM stage (bf16: 16x16x32 as the bf16-operand
        # tiles; fp8: 32x32x64 as the fp8 x fp8 tiles), one wavefront per
        # SIMD, each probe sustained for ~1.6 s (long enough for the
        # clock to settle); both do 32 x 32768 flops per wavefront and iteration
        sampler = PowerSampler()
        blocks = cus
        sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
        power = {}
        for name, fn, iters, flop in (("bf16", lib.moe_calib_mfma_bf16_gemm, 3000, 2 * 16 * 16 * 32 * 2),
                                      ("fp8", lib.moe_calib_mfma_fp8_gemm, 1500, 32 * 32 * 64 * 2)):
            for const in (0, 1):
                def launch(fn=fn, iters=iters, const=const):
                    rc = fn(blocks, iters, const, ctypes.c_void_p(sink.data_ptr()), stream)
                    if rc != 0:
                        raise RuntimeError(f"calibration launch failed: hipError {rc}")
                n, secs, pw = _sustained(launch, 1.6, sampler)
                key = f"mfma_{name}_{'constant' if const else 'random'}_tflops"
                out[key] = round(n * blocks * 4 * iters * 32 * flop / secs / 1e12, 1)
                power[key] = pw
        out["mfma_power"] = power
        out["mfma_probe"] = (f"{blocks} blocks x 4 wavefronts (one per SIMD); bf16: 16x16x32 MFMAs on an 8 x 4 "
                             "grid of 16x16 accumulators, fp8: 32x32x64 block-scaled MFMAs on a 4 x 4 grid of 32x32 "
                             "accumulators; operands from two alternating register sets, random or constant, each "
                             "sustained ~1.6 s (calib/ceilings.hip)")
    if "stream" in which:
        nbytes = 4 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
        blocks = 4096
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        read = ctypes.c_longlong(0)

        for nt, key in ((0, "stream_read_plain_gbs"), (1, "stream_read_nt_gbs")):
            def launch(nt=nt):
                rc = lib.moe_calib_stream_read(ctypes.c_void_p(src.data_ptr()), nbytes, blocks,
                                               ctypes.c_void_p(sink.data_ptr()), ctypes.byref(read), nt, stream)
                if rc != 0:
                    raise RuntimeError(f"calibration launch failed: hipError {rc}")
            ms = _timed(launch, 5)
            out[key] = round(read.value / (ms * 1e-3) / 1e9, 1)
            n, secs, pw = _sustained(launch, 1.6, PowerSampler())
            out[key.replace("_gbs", "_sustained_gbs")] = round(n * read.value / secs / 1e9, 1)
            out[key.replace("_gbs", "_power")] = pw
        # the ceiling: the faster of the two access kinds
        out["stream_read_gbs"] = max(out["stream_read_plain_gbs"], out["stream_read_nt_gbs"])
        out["stream_probe"] = (f"{read.value >> 20} MiB read by {blocks} blocks, one contiguous chunk each, "
                               "16-byte loads, 8 in flight per thread, plain and non-temporal "
                               "(calib/ceilings.hip); stream_read_gbs is the faster")
        del src
    return out


def calibrate_copy():
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read": n, "bytes_written": n, "launches": 3}))


# ------------------------------------------------------------ rocprofv3 trace

def summarize_trace(d: str, warmup: int, steps: int):
    """Per-kernel table of a rocprofv3 --kernel-trace CSV: calls, average,
    min and max over all launches, and the steady-state average over the
    launches of the timed steps (a kernel launched c times per step in W
    warm-up and K timed steps: its last c*K launches)."""
    files = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {d}")
    durs = {}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                name = row["Kernel_Name"]
                durs.setdefault(name, []).append((int(row["Start_Timestamp"]), int(row["End_Timestamp"])))
    total = sum(e - s for v in durs.values() for s, e in v) / 1e3  # us
    rows = []
    for name, v in durs.items():
        v.sort()
        us = np.array([(e - s) / 1e3 for s, e in v])
        steady = None
        if len(v) % (warmup + steps) == 0:
            per = len(v) // (warmup + steps)
            steady = float(us[per * warmup:].mean())
        rows.append((float(us.sum()), name, len(v), float(us.mean()), float(us.min()), float(us.max()), steady))
    rows.sort(reverse=True)
    print(f"| kernel | calls | avg µs | min µs | max µs | steady-state avg µs (last {steps} of {warmup + steps} "
          f"steps) | % of GPU time |")
    print("|---|---|---|---|---|---|---|")
    for tot, name, n, avg, lo, hi, st in rows:
        short = name if len(name) < 120 else name[:117] + "..."
        sts = f"{st:.1f}" if st is not None else "—"
        print(f"| `{short}` | {n} | {avg:.1f} | {lo:.1f} | {hi:.1f} | {sts} | {100 * tot / total:.2f} |")


def summarize_counters(d: str, warmup: int, steps: int):
    """Per kernel and counter of rocprofv3 --pmc CSVs: the mean value per
    dispatch over the timed steps (a kernel dispatched c times per step in W
    warm-up and K timed steps: its last c*K dispatches), and derived ratios
    where their inputs are present: MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES per
    SIMD over the kernel's cycles), TA and TD busy per CU, and L1 stalls.
    GRBM_GUI_ACTIVE comes summed over the 8 XCDs (8x the cycles of the
    kernel's span at the clock: checked against its duration), so one XCD's
    count, GRBM_GUI_ACTIVE / 8, is the kernel's cycles."""
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    vals = {}  # (kernel, counter) -> {dispatch: value}
    for f in files:
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                key = (row["Kernel_Name"], row["Counter_Name"])
                did = (f, int(row["Dispatch_Id"]))
                vals.setdefault(key, {})
                vals[key][did] = vals[key].get(did, 0.0) + float(row["Counter_Value"])
    kernels = sorted({k for k, _ in vals})
    for kern in kernels:
        ctrs = sorted(c for k, c in vals if k == kern)
        mean = {}
        n_disp = 0
        for c in ctrs:
            per = [v for _, v in sorted(vals[(kern, c)].items())]
            n_disp = len(per)
            if len(per) % (warmup + steps) == 0:
                per = per[len(per) // (warmup + steps) * warmup:]
            mean[c] = float(np.mean(per))
        print(f"### `{kern}` ({n_disp} dispatches)\n")
        print("| counter | mean per dispatch (timed steps) |\n|---|---|")
        for c in ctrs:
            print(f"| {c} | {mean[c]:.6g} |")
        g = mean.get("GRBM_GUI_ACTIVE")
        g = g / XCDS if g else g
        derived = []
        if g:
            if "SQ_VALU_MFMA_BUSY_CYCLES" in mean:
                derived.append(("MFMA busy, % of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x "
                                "1024 SIMDs))", 100 * mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (g * 1024)))
            for c, what in (("TA_TA_BUSY", "TA busy"), ("TD_TD_BUSY", "TD busy"),
                            ("TA_ADDR_STALLED_BY_TC_CYCLES", "TA address stalled by the L1 (TC)"),
                            ("TD_TC_STALL", "TD stalled by the L1 (TC)"),
                            ("TCP_TCR_TCP_STALL_CYCLES", "L1 stalled by the L2 request path (TCR)"),
                            ("TCP_PENDING_STALL_CYCLES", "L1 stalled on pending misses"),
                            ("SQ_BUSY_CU_CYCLES", "CU busy (SQ_BUSY_CU_CYCLES)")):
                if c in mean:
                    derived.append((f"{what}, % of cycles per CU ({c} / (GRBM_GUI_ACTIVE / 8 x 256 CUs))",
                                    100 * mean[c] / (g * 256)))
        if "SQ_INSTS_MFMA" in mean and "SQ_INSTS_VALU" in mean:
            derived.append(("non-MFMA VALU instructions per MFMA", (mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"])
                            / max(mean["SQ_INSTS_MFMA"], 1.0)))
        if "SQ_INSTS_LDS" in mean and "SQ_INSTS_MFMA" in mean:
            derived.append(("LDS instructions per MFMA", mean["SQ_INSTS_LDS"] / max(mean["SQ_INSTS_MFMA"], 1.0)))
        if derived:
            print("\n| derived | value |\n|---|---|")
            for what, v in derived:
                print(f"| {what} | {v:.4g} |")
        print()


# ------------------------------------------------------------- CPU baseline

def cpu_baseline(w, L, host_experts, sample):
    """The float64 oracle on the first `sample` tokens (without a capacity the
    layer is token-wise, so this is exactly those tokens' forward).  The
    expert weights' decode to float64 is timed apart and not counted: it is
    a property of the storage format, done once per weight load."""
    import oracle as O
    from threadpoolctl import threadpool_info

    x, wr, b = O.decoded_inputs(L)
    xs = x[:sample]
    in_forward = [0.0]  # decode time spent inside the timed forward

    def expert(e):
        t0 = time.perf_counter()
        ew = host_experts[e]
        w1, w3, w2 = O.decode(ew.w1, w.wdt), O.decode(ew.w3, w.wdt), O.decode(ew.w2, w.wdt)
        if w.wdt == "e4m3":
            w1 = w1 * ew.s1.astype(np.float64)[:, None]
            w3 = w3 * ew.s3.astype(np.float64)[:, None]
            w2 = w2 * ew.s2.astype(np.float64)[:, None]
        in_forward[0] += time.perf_counter() - t0
        return w1, w3, w2

    t0 = time.perf_counter()
    shared = O.adapters.decoded_shared(L)
    shared_s = time.perf_counter() - t0
    # with a capacity factor the sample gets its own slots (factor * sample * k / E)
    cap = O.expert_capacity(getattr(w, "capacity_factor", 0), sample, w.k, w.E)
    t0 = time.perf_counter()
    O.layer_forward(xs, wr, b, O.workload_spec(w), w.E, expert, w.act, shared, capacity=cap,
                    fp8_dispatch=w.dispatch_fp8, overflow=w.overflow)
    dt = time.perf_counter() - t0 - in_forward[0]
    decode_s = [shared_s + in_forward[0]]
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
            "cpu_model": cpu_model, "blas": blas, "kind": "oracle",
            "sample": f"first {sample} of {w.T} tokens, full layer forward in float64 (routing, dispatch, "
                      f"experts, combine): {dt:.2f} s of compute; the float64 decode of the stored expert "
                      f"weights ({decode_s[0]:.2f} s) is excluded",
            "compute_s": round(dt, 3), "weight_decode_s": round(decode_s[0], 3)}


# ------------------------------------------------------------------ one layer

def measure(w, seed, args, keep_host=False, steps=None, warmup=None, cold=True):
    """Times `steps` layer forwards of workload w after `warmup` untimed ones.
    Returns (record fields, LayerInputs, host expert bytes or None)."""
    import torch

    import mixture_experts_layer_36_amd as moe
    from synth import LayerInputs
    from synth.device import DeviceLayer

    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
    progress(f"{w.name}: generating and uploading inputs (seed {seed})")
    L = LayerInputs(w, seed)
    host_experts = {} if keep_host else None
    orig = L.expert

    def keep(e):
        ew = orig(e)
        if keep_host:
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

    progress(f"{w.name}: {warmup} warm-up and {steps} timed steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    traces = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.TRACE_EVENTS)] for _ in range(steps)]
    for tr in traces:  # create the HIP events before the timed region
        for ev in tr:
            ev.record()
    torch.cuda.synchronize()

    if args.graph:
        # per-stage times from a traced eager pass; the timed steps replay
        # one captured graph of the forward
        for i in range(steps):
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
        for i in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    else:
        t0 = time.perf_counter()
        for i in range(steps):
            step(traces[i])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

    sustained = None
    if args.sustain_seconds > 0:
        # the step over and over for a few seconds, outside the timed region:
        # the rate once power management has settled, with the socket power
        # and graphics clock meanwhile
        n, secs, pw = _sustained(step, args.sustain_seconds, PowerSampler())
        sustained = {"steps": n, "seconds": round(secs, 3), "ms_per_step": round(secs * 1e3 / n, 4),
                     "tokens_per_s": round(w.T * n / secs, 1), "power": pw}

    cold_rec = None
    if cold and not args.no_cold:
        # cold-cache repetitions, outside the timed region: the eviction
        # write runs between a step's events, never inside them
        evict = torch.empty(EVICT_BYTES, dtype=torch.uint8, device="cuda")
        cold_tr = [[torch.cuda.Event(enable_timing=True) for _ in range(moe.TRACE_EVENTS)] for _ in range(steps)]
        for tr in cold_tr:
            for ev in tr:
                ev.record()
        torch.cuda.synchronize()
        for i in range(steps):
            evict.fill_(i & 0xff)
            step(cold_tr[i])
        torch.cuda.synchronize()
        cms = np.array([[tr[j].elapsed_time(tr[j + 1]) for j in range(moe.TRACE_EVENTS - 1)] for tr in cold_tr])
        cstep = float(np.median([tr[0].elapsed_time(tr[-1]) for tr in cold_tr]))
        cold_rec = {"evict_bytes": EVICT_BYTES, "reps": steps, "step_ms_median": round(cstep, 4),
                    "tokens_per_s": round(w.T / (cstep * 1e-3), 1),
                    "stages_us_median": {name: round(float(np.median(cms[:, j])) * 1e3, 2)
                                         for j, name in enumerate(moe.TRACE_STAGES)}}
        del evict

    stage_ms = np.array([[tr[j].elapsed_time(tr[j + 1]) for j in range(moe.TRACE_EVENTS - 1)] for tr in traces])
    stage_us = {name: round(float(stage_ms[:, j].mean()) * 1e3, 2) for j, name in enumerate(moe.TRACE_STAGES)}
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

    ms_per_step = elapsed * 1e3 / steps
    value = w.T * steps / elapsed
    gemm1_s = stage_ms[:, 2].mean() * 1e-3
    fused_sh = shared_fused(w)
    flops_gemm1 = 4.0 * w.d * w.f * n_assign + (4.0 * w.d * w.f_shared * w.T if fused_sh else 0.0)
    flops_all = 6.0 * w.d * w.f * n_assign + 6.0 * w.d * w.f_shared * w.T
    if w.name in DECODE_WORKLOADS:
        layer_s = step_event_ms * 1e-3
        achieved = layer_bytes(w, c) / layer_s / 1e9
        roof = {"bound": "hbm", "kernel": "whole layer (all kernels of one moe_layer_forward)",
                "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "algorithmic_bytes": layer_bytes(w, c),
                "avg_launch_us": round(layer_s * 1e6, 2)}
    else:
        achieved = flops_gemm1 / gemm1_s / 1e12
        f8 = fp8_gate_up(w)
        peak = PEAK_FP8_TFLOPS if f8 else PEAK_BF16_TFLOPS
        kern = ("gemm_big_fp8_kernel: fp8 x fp8 block-scaled MFMA" if f8 else
                "gemm_big_kernel / gemm_mfma_kernel, EPI_SWIGLU, with its split-tile fixup")
        roof = {"bound": "mfma",
                "kernel": f"gate-up GEMM + SwiGLU ({kern})" + (", routed and shared segments" if fused_sh else ""),
                "mfma_dtype": "fp8" if f8 else "bf16",
                "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "algorithmic_flops": flops_gemm1,
                "flops_formula": "4*d*f*rows" + (" + 4*d*f_shared*T" if fused_sh else ""),
                "avg_launch_us": round(gemm1_s * 1e6, 2)}
    # HBM bytes per launch of that kernel from the committed rocprofv3
    # FETCH_SIZE / WRITE_SIZE passes, valid only while the kernels are unchanged
    roof["traffic"] = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        ent = tr.get(w.name + ("+dispatch_fp8" if w.dispatch_fp8 else ""))
        if ent and ent.get("source_hash") == kernel_source_hash():
            roof["traffic"] = ent.get("bytes_per_launch")

    ffn_s = float(stage_ms[:, 2:5].sum(axis=1).mean()) * 1e-3
    rec = {
        "value": round(value, 1), "ms_per_step": round(ms_per_step, 4),
        "config": {"workload": w.name, "T": w.T, "d": w.d, "f": w.f, "E": w.E, "k": w.k,
                   "score": w.score, "n_group": w.n_group, "topk_group": w.topk_group,
                   "f_shared": w.f_shared, "act": w.act, "weights": w.wdt, "seed": seed,
                   "capacity_factor": w.capacity_factor, "overflow": w.overflow,
                   "dispatch_fp8": w.dispatch_fp8, "weight_layout": layout,
                   "launch": "hip graph replay" if args.graph else "eager"},
        "roofline": roof,
        # all expert GEMMs (routed gate-up and down, shared expert) over their stages
        "ffn_tflops": round(flops_all / ffn_s / 1e12, 1),
        "ffn_frac_of_bf16_peak": round(flops_all / ffn_s / 1e12 / PEAK_BF16_TFLOPS, 4),
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
        "sustained": sustained,
        "cold_cache": cold_rec,
    }
    del dev, out, idx, gw, counts, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, L, host_experts


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.warmup, args.steps)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.warmup, args.steps)
        return
    if args.write_traffic:
        write_traffic(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch  # noqa: F401

    import mixture_experts_layer_36_amd as moe  # noqa: F401  (fails loudly if libmoe.so is missing)
    from synth import BY_NAME, DEFAULT_SEED

    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.calibrate_mfma or args.calibrate_stream:
        which = (("mfma",) if args.calibrate_mfma else ()) + (("stream",) if args.calibrate_stream else ())
        print(json.dumps({"calibration": "ceilings", **ceilings(which)}))
        return
    w = BY_NAME[args.workload]
    seed = DEFAULT_SEED[w.name] if args.seed is None else args.seed
    if args.capacity_factor > 0:
        w = w.scaled(capacity_factor=args.capacity_factor)
    if args.dispatch_fp8:
        w = w.scaled(dispatch_fp8=True)
    if args.overflow != "drop":
        w = w.scaled(overflow=args.overflow)

    rec, L, host_experts = measure(w, seed, args, keep_host=not args.no_cpu_baseline)
    line = {
        "metric": METRIC, "value": rec.pop("value"), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": rec.pop("ms_per_step"),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16, fp8 gate-up" if fp8_gate_up(w) else "bf16") if w.act == "bf16" else "f32",
        "data": "synthetic",
    }
    line.update(rec)
    ceil = None
    if not args.no_ceilings:
        progress("ceiling probes")
        ceil = ceilings()
        r = line["roofline"]
        if r["bound"] == "mfma":
            key = f"mfma_{r['mfma_dtype']}_random_tflops"  # random operands, like the layer's data
            r["frac_of_measured_mfma_ceiling"] = round(r["achieved"] / ceil[key], 4)
        else:
            r["frac_of_measured_read_ceiling"] = round(r["achieved"] / ceil["stream_read_gbs"], 4)
    line["ceilings"] = ceil
    line["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        sample = args.cpu_sample or CPU_SAMPLE.get(w.name, 256)
        progress(f"oracle on {min(sample, w.T)} tokens")
        line["cpu_baseline"] = cpu_baseline(w, L, host_experts, min(sample, w.T))
    del host_experts, L

    line["decode"] = None
    if w.name == DEFAULT_WORKLOAD and not args.no_decode_leg and args.workload == DEFAULT_WORKLOAD:
        # the decode-shaped layer, bound by HBM bandwidth: its own steps
        # (more of them: a step is ~4 ms), no cold repetitions
        wd = BY_NAME[DECODE_WORKLOAD]
        d_rec, _, _ = measure(wd, DEFAULT_SEED[wd.name], args, steps=DECODE_STEPS_PER_STEP * args.steps,
                              warmup=args.warmup, cold=False)
        r = d_rec["roofline"]
        if ceil:
            r["frac_of_measured_read_ceiling"] = round(r["achieved"] / ceil["stream_read_gbs"], 4)
        line["decode"] = {"metric": "MoE-layer tokens/s per MI355X; decode % HBM BW",
                          "value": d_rec["value"], "unit": "tokens/s", "steps": DECODE_STEPS_PER_STEP * args.steps,
                          "ms_per_step": d_rec["ms_per_step"], "config": d_rec["config"], "roofline": r,
                          "stages_us": d_rec["stages_us"], "stages_gbps": d_rec["stages_gbps"],
                          "load": d_rec["load"], "sustained": d_rec["sustained"]}
    print(json.dumps(line))


if __name__ == "__main__":
    main()
