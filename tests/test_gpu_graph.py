"""The whole layer (w8a8_moe_forward) captured into a HIP graph and replayed, through the C ABI.

The entry points enqueue kernels only (no allocation, no memset, no host synchronisation, no host
read of device data), so a captured layer must replay exactly: each replay is compared bit for
bit with an eager run of the same inputs (the layer is deterministic), with eager work and
synchronisations between replays, and once more after the inputs are changed in place (new
routing, so new expert segments and tile lists built on the device during the replay).
Covers the staged engine (tiny, decode), the W4A8 streaming engine (W4A8 decode), the ring
engine (block-wise T=2048) and the DMA engine (prefill).
"""
import dataclasses
import sys

import pytest

import synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

from w8a8_int8_quantized_quant_amd import workload  # noqa: E402

DEV = "cuda"

CASES = {
    "tiny": synth.CONFIGS["tiny"],
    "decode": synth.CONFIGS["decode"],
    "w4a8-decode": dataclasses.replace(synth.CONFIGS["decode"], name="w4a8-decode", scale_mode="w4a8"),
    "block": synth.CONFIGS["block"],
    "prefill": synth.CONFIGS["prefill"],
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", list(CASES))
def test_forward_graph_replay(name):
    cfg = CASES[name]
    say(f"[graph] {name}: drawing the layer")
    torch.cuda.empty_cache()
    L = workload.make_layer(cfg, device=DEV)
    T, H = cfg.T, cfg.H
    ws = workload.forward_workspace(L)
    out_e = torch.empty((T, H), dtype=torch.float32, device=DEV)
    out_g = torch.empty((T, H), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        workload.forward(L, out_e, ws, stream=s)
    torch.cuda.synchronize()
    ref = out_e.clone()

    say(f"[graph] {name}: capturing")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        workload.forward(L, out_g, ws, stream=s)
    torch.cuda.synchronize()

    for i in range(3):
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {i} differs from the eager run"
        out_e.fill_(float("nan"))
        workload.forward(L, out_e, ws)  # eager work on the default stream between replays
        torch.cuda.synchronize()
        assert torch.equal(out_e, ref)

    # new inputs in place: other tokens in each row slot, other routing
    L.x.copy_(torch.roll(L.x, 1, 0).flip(1))
    L.logits.copy_(torch.roll(L.logits, 3, 1))
    torch.cuda.synchronize()
    workload.forward(L, out_e, ws)
    torch.cuda.synchronize()
    ref2 = out_e.clone()
    assert not torch.equal(ref2, ref)
    out_g.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out_g, ref2), "replay after new inputs differs from the eager run"
    say(f"[graph] {name}: 4 replays bit-equal to eager runs")
    del g, L, ws, out_e, out_g
    torch.cuda.empty_cache()
