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


@pytest.mark.parametrize("name,cfg", [
    ("summed", moe_synth.Config("gdisp", 2048, 4096, 256, 8, 2, 1, "bf16", 43)),
    # 32 chunks x 1024 segments: past what one workgroup sums, so the
    # histograms are scanned by a third launch first
    ("scanned", moe_synth.Config("gdisp_s", 8192, 256, 256, 128, 8, 8, "bf16", 44, 0.0, 1024)),
])
def test_dispatch_noalloc_graph_replays_equal_eager(name, cfg):
    """The allocation-free dispatch is for callers that cannot allocate, such
    as code under graph capture: captured once, each replay must give what the
    allocating moe_dispatch gives eagerly on the same (changed) inputs."""
    print(f"[graph] dispatch_noalloc {name} {cfg}", flush=True)
    g = upload(moe_synth.make_inputs(cfg))
    p = problem_of(cfg)
    M, k, H, G, R = cfg.M, cfg.k, cfg.H, cfg.S * cfg.EL, cfg.M * cfg.k
    idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")

    def bufs():
        return dict(counts=torch.empty(G, dtype=torch.int32, device="cuda"),
                    offsets=torch.empty(G + 1, dtype=torch.int32, device="cuda"),
                    s2f=torch.empty(R, dtype=torch.int32, device="cuda"),
                    f2s=torch.empty(R, dtype=torch.int32, device="cuda"),
                    xp=torch.empty((R, H), dtype=torch.bfloat16, device="cuda"))

    e, gr = bufs(), bufs()
    ws = torch.empty(max(moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH), 4), dtype=torch.uint8, device="cuda")
    src = g.get("src_block")

    def noalloc():
        moe.moe_dispatch_noalloc(p, g["x"], idx, src, gr["counts"], gr["offsets"], gr["s2f"], gr["f2s"], gr["xp"])

    moe.moe_route(p, g["logits"], idx, w)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        noalloc()  # warm-up outside the capture (the scratch address is looked up once)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        noalloc()
    torch.cuda.synchronize()
    inputs = [(g["x"].clone(), g["logits"].clone()),
              ((g["x"].float() * -0.5).to(torch.bfloat16), g["logits"].flip(1).contiguous()),
              (g["x"].clone(), g["logits"].clone())]
    for rep, (xv, lv) in enumerate(inputs):
        g["x"].copy_(xv)
        g["logits"].copy_(lv)
        moe.moe_route(p, g["logits"], idx, w)
        moe.moe_dispatch(p, g["x"], idx, src, e["counts"], e["offsets"], e["s2f"], e["f2s"], e["xp"], ws)
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "s2f", "f2s"):
            gr[key].fill_(-7)
        gr["xp"].fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for key in ("counts", "offsets", "s2f", "f2s"):
            assert torch.equal(gr[key], e[key]), (name, rep, key)
        n = int(e["offsets"][-1])
        assert n == R, (name, n)  # every expert is held: every pair kept
        assert torch.equal(gr["xp"][:n].view(torch.int16), e["xp"][:n].view(torch.int16)), (name, rep)
    assert not torch.equal(inputs[0][1], inputs[1][1])
