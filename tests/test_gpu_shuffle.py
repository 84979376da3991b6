"""Reordering check (MOE_DEBUG_SHUFFLE): the results must not depend on the
order in which tiles and combine items run.

COMET paper review §4.1.2: the rescheduled (column-wise, chunked) GEMM must
give the same results as the original order.  Here every output element is
computed by one tile (or one combine item) with a fixed k order of its own,
so permuting the tiles of a grouped GEMM (inside the full rounds, and
separately inside a last round that is split or halved), or the fused
kernel's items inside their sections (Layer0 tiles, each chunk's Layer1
tiles, each chunk's combine items), must reproduce every bit.  A difference
would be a race, a tile written twice or not at all, or state carried from
one tile to the next.  The switch is read by the library at each call, so
each run below sets the environment variable around its calls.
"""
import contextlib
import os

import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import run_chain, run_layer, upload
from test_gpu_mx import run_chain_mx
from test_gpu_random_shapes import _multi_shape

pytestmark = pytest.mark.gpu

SEEDS = [1, 977, 4000000000]


@contextlib.contextmanager
def shuffle(seed):
    old = os.environ.get("MOE_DEBUG_SHUFFLE")
    os.environ["MOE_DEBUG_SHUFFLE"] = str(seed)
    try:
        yield
    finally:
        if old is None:
            del os.environ["MOE_DEBUG_SHUFFLE"]
        else:
            os.environ["MOE_DEBUG_SHUFFLE"] = old


def _bits(t):
    # bit patterns, so that NaN rows nothing writes compare equal too
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _same(a, b, keys, name):
    for key in keys:
        assert torch.equal(_bits(a[key]), _bits(b[key])), (name, key)


CHAIN_CASES = {
    # multi-round shapes: halves in Layer0's last round, a 3-way k split of
    # Layer1's, held experts of two source blocks, many small experts
    "l0_halves": lambda: _multi_shape("l0_halves"),
    "l1_split3": lambda: _multi_shape("l1_split3"),
    "held_src_blocks": lambda: _multi_shape("held_src_blocks"),
    "many_experts": lambda: _multi_shape("many_experts"),
    # 8 source blocks of 256 tokens, 128-row segments: the combined-segment tiles
    "combined_segments": lambda: moe_synth.Config("ep2k", 2048, 1024, 512, 16, 8, 8, "bf16", 32, 0.0, 256),
    "f32": lambda: moe_synth.config("tiny"),
}

KEYS = ("topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted", "x_perm", "hact", "y", "out")


@pytest.mark.parametrize("name", list(CHAIN_CASES))
def test_chain_is_order_invariant(name):
    cfg = CHAIN_CASES[name]()
    print(f"[shuffle] chain {cfg}", flush=True)
    g = upload(moe_synth.make_inputs(cfg))
    base = run_chain(cfg, g)
    for seed in SEEDS:
        print(f"[shuffle] {name} seed {seed}", flush=True)
        with shuffle(seed):
            got = run_chain(cfg, g)
        _same(base, got, KEYS, f"{name} seed {seed}")


def test_mxfp8_chain_is_order_invariant():
    cfg = moe_synth.config("qwen2", dtype="bf16_mxfp8")
    print(f"[shuffle] mxfp8 chain {cfg}", flush=True)
    g = upload(moe_synth.make_inputs(cfg))
    wd = g["w_down"]
    wd_mx = torch.empty(moe.mx_bytes(cfg.EL * cfg.H, cfg.F), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(wd.view(cfg.EL * cfg.H, cfg.F), wd_mx)
    _, base = run_chain_mx(cfg, g, wd_mx)
    for seed in SEEDS:
        with shuffle(seed):
            _, got = run_chain_mx(cfg, g, wd_mx)
        _same(base, got, KEYS, f"mxfp8 seed {seed}")


@pytest.fixture(scope="module")
def fused_cases():
    out = {}
    for name, cfg in (("qwen2", moe_synth.config("qwen2")),
                      ("mix2k", moe_synth.Config("mix2k", 2048, 4096, 14336, 8, 2, 1, "bf16", 31))):
        out[name] = (cfg, upload(moe_synth.make_inputs(cfg)))
    return out


@pytest.mark.parametrize("name", ["qwen2", "mix2k"])
@pytest.mark.parametrize("n_mover,gather", [(0, 1), (8, 1), (0, 0)])
def test_fused_is_order_invariant(fused_cases, name, n_mover, gather):
    cfg, g = fused_cases[name]
    print(f"[shuffle] fused {name} n_mover={n_mover} gather={gather}", flush=True)
    base, aux0, st = run_layer(cfg, g, aux=True, n_mover=n_mover, gather=gather)
    assert st == moe.MOE_OK
    for seed in SEEDS[:2]:
        with shuffle(seed):
            got, aux, st = run_layer(cfg, g, aux=True, n_mover=n_mover, gather=gather)
        assert st == moe.MOE_OK
        assert torch.equal(_bits(got), _bits(base)), (name, seed)
        _same(aux0, aux, ("hact", "y"), f"fused {name} seed {seed}")
