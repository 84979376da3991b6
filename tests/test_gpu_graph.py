"""moe_layer captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

A call is a sequence of kernel launches on the caller's stream; the status
word, the fused kernel's counters and the split workspace are cleared by
fill kernels or written by the kernels themselves (no memset nodes), so
every replay must give the eager call's bits: with new values in the
captured input buffers, and with eager work and synchronisations between
the replays.
"""
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import problem_of, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,fused", [("bf16", 0), ("bf16", 1), ("bf16_mxfp8", 0)])
def test_layer_graph_replays_equal_eager(dtype, fused):
    cfg = moe_synth.Config("graph", 1024, 512, 768, 8, 2, 1, dtype, 41)
    print(f"[graph] {cfg} fused={fused}", flush=True)
    g = upload(moe_synth.make_inputs(cfg))
    if dtype == "bf16_mxfp8":
        wd = torch.empty(moe.mx_bytes(cfg.E * cfg.H, cfg.F), dtype=torch.uint8, device="cuda")
        moe.moe_quantize_mxfp8(g["w_down"], wd)
        g["w_down"] = wd
    p = problem_of(cfg)
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda")
    out_e = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
    out_g = torch.empty_like(out_e)
    inputs = [(g["x"].clone(), g["logits"].clone()),
              ((g["x"].float() * -0.5).to(g["x"].dtype), g["logits"].flip(1).contiguous()),
              (g["x"].clone(), g["logits"].clone())]

    def call(out):
        # fused: the fused kernel with the combine in the shared queue; else the chain
        moe.moe_layer(p, g["x"], g["logits"], None, g["w_gate"], g["w_up"], g["w_down"], out, ws,
                      fused=fused, n_mover=0 if fused else -1)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_g)  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g)
    torch.cuda.synchronize()
    for rep, (xv, lv) in enumerate(inputs):
        g["x"].copy_(xv)
        g["logits"].copy_(lv)
        call(out_e)
        torch.cuda.synchronize()
        assert moe.moe_debug_device_status(p, ws) == moe.MOE_OK
        float((out_e * 2.0).sum())  # unrelated eager work between replays
        out_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert moe.moe_debug_device_status(p, ws) == moe.MOE_OK
        assert torch.equal(out_g, out_e), rep
    assert not torch.equal(inputs[0][0], inputs[1][0])
