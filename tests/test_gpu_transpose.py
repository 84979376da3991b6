"""moe_transpose_weights: the batched transpose that turns weight matrices
as the math writes them (W_gate, W_up of H x F, W_down of F x H, per
expert) into the storage the layer reads.  A pure data movement, so the
check is bitwise against torch's transpose."""
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 64, 64), (3, 128, 192), (5, 320, 64), (2, 4096, 14336)])
def test_transpose_is_exact(dtype, shape):
    if dtype == torch.float32 and shape[1] * shape[2] > 1 << 24:
        pytest.skip("one large case per dtype is enough")
    print(f"[transpose] {shape} {dtype}", flush=True)
    gen = torch.Generator(device="cuda").manual_seed(sum(shape))
    src = torch.randn(shape, generator=gen, device="cuda").to(dtype)
    dst = torch.full((shape[0], shape[2], shape[1]), float("nan"), dtype=dtype, device="cuda")
    moe.moe_transpose_weights(src, dst)
    torch.cuda.synchronize()
    want = src.transpose(1, 2).contiguous()
    bits = torch.int16 if dtype == torch.bfloat16 else torch.int32
    assert torch.equal(dst.view(bits), want.view(bits))


def test_math_layout_weights_give_the_library_storage():
    # the workload's weights as the math writes them, back to the storage
    # the layer reads: bit for bit the generator's [EL,F,H] / [EL,H,F]
    cfg = moe_synth.Config("tw", 256, 512, 768, 8, 2, 1, "bf16", 47)
    g = upload(moe_synth.make_inputs(cfg))
    for key, (rows, cols) in (("w_gate", (cfg.H, cfg.F)), ("w_up", (cfg.H, cfg.F)), ("w_down", (cfg.F, cfg.H))):
        math = g[key].transpose(1, 2).contiguous()  # [EL, rows, cols]
        assert math.shape == (cfg.EL, rows, cols)
        back = torch.empty_like(g[key])
        moe.moe_transpose_weights(math, back)
        torch.cuda.synchronize()
        assert torch.equal(back.view(torch.int16), g[key].view(torch.int16)), key


def test_overlapping_buffers_are_rejected():
    a = torch.empty((2, 128, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_transpose_weights(a, a)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARGUMENT
