"""Two moe_layer calls (the kernel chain) in flight at once on two streams,
each with its own workspace and outputs: the library keeps no state between
calls besides what the caller passes, so each must give the serial result
bit for bit."""
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import problem_of, upload

pytestmark = pytest.mark.gpu


def test_concurrent_chain_calls_equal_serial():
    cfgs = [moe_synth.Config("s1", 2048, 1024, 1536, 8, 2, 1, "bf16", 51),
            moe_synth.Config("s2", 1024, 2048, 1024, 16, 4, 1, "bf16", 52)]
    runs = []
    for cfg in cfgs:
        g = upload(moe_synth.make_inputs(cfg))
        p = problem_of(cfg)
        ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda")
        runs.append((cfg, g, p, ws))

    def call(run, out, stream=None):
        cfg, g, p, ws = run
        moe.moe_layer(p, g["x"], g["logits"], None, g["w_gate"], g["w_up"], g["w_down"], out, ws, fused=0,
                      stream=stream)

    serial = []
    for run in runs:
        out = torch.empty((run[0].M, run[0].H), dtype=torch.float32, device="cuda")
        call(run, out)
        torch.cuda.synchronize()
        serial.append(out)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.full_like(o, float("nan")) for o in serial]
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        for run, out, st in zip(runs, outs, streams):
            with torch.cuda.stream(st):
                for _ in range(4):  # several calls each, so the two streams overlap
                    call(run, out, stream=st)
        torch.cuda.synchronize()
        for i, (o, s) in enumerate(zip(outs, serial)):
            assert torch.equal(o, s), (rep, i)
