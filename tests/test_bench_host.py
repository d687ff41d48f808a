"""bench.py's host logic, without a GPU: the one-GPU refusal, the rocprofv3
trace summary (steady-state averages over the timed steps) and the
algorithmic-work formulas the roofline divides by."""
import argparse
import json
import os
import subprocess
import sys

import numpy as np

import bench
from synth import BY_NAME

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_summarize_trace_steady_state(tmp_path, capsys):
    # kernel A: once per step, 2 warm-up steps of 100 us then 3 of 10 us;
    # kernel B: twice per step, always 5 us
    rows = ["Kernel_Name,Start_Timestamp,End_Timestamp"]
    t = 0
    for step in range(5):
        dur = 100_000 if step < 2 else 10_000
        rows.append(f"A,{t},{t + dur}")
        t += dur + 1000
        for _ in range(2):
            rows.append(f"B,{t},{t + 5000}")
            t += 6000
    sub = tmp_path / "host"
    sub.mkdir()
    (sub / "123_kernel_trace.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_trace(str(tmp_path), warmup=2, steps=3)
    out = capsys.readouterr().out.splitlines()
    a = next(ln for ln in out if ln.startswith("| `A`"))
    b = next(ln for ln in out if ln.startswith("| `B`"))
    cols = [c.strip() for c in a.split("|")]
    assert cols[2] == "5" and cols[3] == "46.0" and cols[6] == "10.0"  # all-launch avg vs steady state
    cols = [c.strip() for c in b.split("|")]
    assert cols[2] == "10" and cols[6] == "5.0"


def test_gate_up_flops_count_the_fused_shared_expert():
    w4 = BY_NAME["dsv3_prefill_skew_bf16"]
    assert bench.shared_fused(w4)  # bf16 shared weights beside bf16 routed weights: one launch
    assert not bench.shared_fused(BY_NAME["qwen_moe_fp8_skew"])  # no shared expert
    assert not bench.shared_fused(BY_NAME["mixtral8x7b_prefill_bf16"])


def test_layer_bytes_counts_touched_experts_only():
    w = BY_NAME["dsv3_decode_bf16"]
    c = np.zeros(w.E, dtype=np.int64)
    c[:10] = 1
    b10 = bench.layer_bytes(w, c)
    c[:11] = 1
    assert bench.layer_bytes(w, c) - b10 == 3 * w.d * w.f * 2


def test_summarize_counters_timed_dispatches(tmp_path, capsys):
    # one kernel, 1 warm-up + 2 timed steps; the warm-up dispatch is excluded
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for disp, (mfma, gui) in enumerate(((900.0, 1000.0), (512.0, 1000.0), (256.0, 1000.0))):
        rows.append(f"{disp},K,SQ_VALU_MFMA_BUSY_CYCLES,{mfma * 1024}")
        rows.append(f"{disp},K,GRBM_GUI_ACTIVE,{gui * 8}")  # summed over the 8 XCDs
        rows.append(f"{disp},K,TA_TA_BUSY,{250.0 * 256}")
    (tmp_path / "run_counter_collection.csv").write_text("\n".join(rows) + "\n")
    bench.summarize_counters(str(tmp_path), warmup=1, steps=2)
    out = capsys.readouterr().out
    assert "| SQ_VALU_MFMA_BUSY_CYCLES | 393216 |" in out  # mean of 512 and 256 (x1024)
    assert "MFMA busy" in out and "| 38.4 |" in out
    assert "TA busy" in out and "| 25 |" in out


def test_power_summary_window_and_unavailable_readings():
    # (time s, socket W, gfx MHz); 0xffff marks a reading the metrics table lacks
    samples = [(0.0, 900, 2400), (1.0, 1390, 1700), (1.5, 1400, 1600), (2.0, 0xffff, 1650), (3.5, 500, 2400)]
    r = bench.PowerSampler.summarize(samples, 0.5, 3.0, cap_w=1400.0)
    assert r == {"socket_power_w_median": 1395.0, "gfxclk_mhz_median": 1650.0, "power_cap_w": 1400.0, "samples": 3}
    assert bench.PowerSampler.summarize(samples, 5.0, 6.0) is None


def test_write_traffic_scales_by_the_copy_and_keeps_timed_steps(tmp_path, monkeypatch):
    # gate-up kernel G once per step (1 warm-up + 2 timed), one other kernel O;
    # the copy run: one fill kernel and 3 copies of 1 GiB whose counters read
    # half the bytes (read factor 2) and all of them (write factor 1)
    def pmc(d, counter, rows):
        d.mkdir()
        lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        lines += [f"{i},\"{k}\",{counter},{v}" for i, (k, v) in enumerate(rows)]
        (d / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")
    G = "gemm_big_kernel<256, 2, 1, 1>(moe::GemmArgs)"
    pmc(tmp_path / "f", "FETCH_SIZE", [(G, 9e9), ("O", 1.0), (G, 100.0), ("O", 1.0), (G, 300.0), ("O", 1.0)])
    pmc(tmp_path / "w", "WRITE_SIZE", [(G, 9e9), (G, 10.0), (G, 30.0)])
    gib_kib = float(1 << 20)
    pmc(tmp_path / "cf", "FETCH_SIZE", [("fill", 5.0)] + [("__amd_rocclr_copyBuffer", gib_kib / 2)] * 3)
    pmc(tmp_path / "cw", "WRITE_SIZE", [("fill", 5.0)] + [("__amd_rocclr_copyBuffer", gib_kib)] * 3)
    line = tmp_path / "line.json"
    line.write_text('{"load": {"experts_touched": 76}}\n')
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    args = argparse.Namespace(write_traffic="dsv3_prefill_skew_bf16", kernel="gemm_big_kernel<256, 2, 1, 1>",
                              fetch=str(tmp_path / "f"), write=str(tmp_path / "w"), copy_fetch=str(tmp_path / "cf"),
                              copy_write=str(tmp_path / "cw"), bench_line=str(line), profile=None, warmup=1, steps=2)
    bench.write_traffic(args)
    ent = json.loads(out.read_text())["dsv3_prefill_skew_bf16"]
    assert ent["fetch_size_kib"] == 200.0 and ent["write_size_kib"] == 20.0
    assert ent["copy_calibration"]["read_factor"] == 2.0 and ent["copy_calibration"]["write_factor"] == 1.0
    assert ent["read_bytes"] == 200 * 1024 * 2 and ent["write_bytes"] == 20 * 1024
    assert ent["source_hash"] == bench.kernel_source_hash()
    w = BY_NAME["dsv3_prefill_skew_bf16"]
    # routed rows + 76 experts' W1, W3 + the fused shared expert's x, W1, W3
    rd = w.T * w.k * w.d * 2 + 76 * 2 * w.f * w.d * 2 + w.T * w.d * 2 + 2 * w.f_shared * w.d * 2
    assert ent["algorithmic_read_bytes"] == rd == 6635388928
    assert ent["algorithmic_write_bytes"] == (w.T * w.k * w.f + w.T * w.f_shared) * 2
