"""Expert weights past 2^32 elements per tensor: the grouped GEMMs address
each expert's weights with 64-bit offsets, so the last expert of a large
stack (its rows start past 2^32 elements) must give the same results as
the first.  The reference is plain torch on the GPU (f32 products of the
same bf16 values, Hact rounded to bf16 as the layer does)."""
import pytest
import torch

import combine_topk_gate_amd as moe

pytestmark = pytest.mark.gpu


def test_last_expert_past_2_32_weight_elements():
    E, H, F, k, M = 160, 4096, 8192, 1, 512
    assert (E - 1) * F * H > 1 << 32  # the last expert's gate/up rows start past 2^32 elements
    print(f"[big weights] E={E} H={H} F={F}: {E * H * F / 2**30:.1f} G elements per tensor", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((M, H), generator=gen, device="cuda").to(torch.bfloat16)
    ws = []
    for shape in ((E, F, H), (E, F, H), (E, H, F)):
        w = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        for e in range(E):  # chunked, so no f32 copy of the whole stack exists
            w[e] = (torch.randn(shape[1:], generator=gen, device="cuda") * 0.02).to(torch.bfloat16)
        ws.append(w)
    wg, wu, wd = ws
    # tokens alternate between the first and the last expert
    logits = torch.full((M, E), -10.0, device="cuda")
    first = torch.arange(M, device="cuda") % 2 == 0
    logits[first, 0] = 10.0
    logits[~first, E - 1] = 10.0
    p = moe.problem(M, H, F, E, k, 1, "bf16")
    wsb = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    moe.moe_layer(p, x, logits, None, wg, wu, wd, out, wsb)
    torch.cuda.synchronize()
    assert moe.moe_debug_device_status(p, wsb) == moe.MOE_OK
    for e, rows in ((0, first), (E - 1, ~first)):
        xe = x[rows].float()
        g = xe @ wg[e].float().t()
        u = xe @ wu[e].float().t()
        h = (g / (1.0 + torch.exp(-g)) * u).to(torch.bfloat16).float()
        y = h @ wd[e].float().t()
        got = out[rows]
        rel = float(torch.linalg.norm(got - y) / torch.linalg.norm(y))
        mx = float((got - y).abs().max())
        print(f"[big weights] expert {e}: relF {rel:.2e} max abs {mx:.2e}", flush=True)
        assert rel <= 5e-3 and mx <= 2e-2, (e, rel, mx)
