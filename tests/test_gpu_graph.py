"""The layer under HIP-graph capture: moe_layer_forward enqueues only kernel
launches on the caller's stream (no host sync, no allocation, no memset
nodes), so a whole forward can be captured once and replayed.  Every replay,
with the program's own eager work and synchronisations in between, must
reproduce the eager result bit for bit (the kernels are deterministic)."""
import pytest
import torch

import mixture_experts_layer_36_amd as moe
import oracle as O
from synth import LayerInputs
from synth.workloads import DSV3_DECODE, MIXTRAL_PREFILL, QWEN_FP8_SKEW
from tests.helpers import DeviceLayer

pytestmark = pytest.mark.gpu

CASES = {
    # decode kernels, shared expert
    "decode": DSV3_DECODE.scaled(T=40, d=512, f=256, E=64, f_shared=256),
    # 256-row kernel with split tiles and the fixup
    "prefill_split": MIXTRAL_PREFILL.scaled(T=1200, d=1024, f=512, E=4),
    # fp8 payload and the fp8 x fp8 gate-up kernel, with a capacity
    "fp8_payload": QWEN_FP8_SKEW.scaled(T=800, d=512, f=384, E=16, k=4, capacity_factor=1.25,
                                        dispatch_fp8=True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_captured_layer_replays_match_eager(name):
    w = CASES[name]
    L = LayerInputs(w, 1, accept=O.margin_acceptor())
    dev = DeviceLayer(L)
    desc = moe.Desc.from_attrs(w)
    out = torch.empty((w.T, w.d), dtype=dev.x.dtype, device="cuda")
    idx = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    gw = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    ws = moe.workspace(desc)

    def step():
        moe.layer_forward(desc, dev.x, dev.w_router, dev.bias, dev.w1, dev.w3, dev.w2, dev.s1, dev.s3,
                          dev.s2, dev.sw1, dev.sw3, dev.sw2, out, idx, gw, counts, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # eager, on the stream the capture will use
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, idx, gw, counts)]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        for t in (out, idx, gw, counts):  # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip((out, idx, gw, counts), ref):
            assert torch.equal(t, e), f"replay {r} differs from the eager forward"
    print(f"{name}: 3 replays equal the eager forward")
