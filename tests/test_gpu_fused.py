"""The fused moe_layer: schedule invariance (race detector), intermediates,
grid sizes and the bounded-wait watchdog.

Every output element of the fused kernel is computed by the same routine in
the same order as in the kernel chain, whatever the split between mover and
matrix-core workgroups or the grid size; so any bitwise difference from the
chain is a race or a flag bug.
"""
import os

import numpy as np
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import layer_runs_chain, run_chain, run_layer, upload

pytestmark = pytest.mark.gpu


def _case(cfg):
    # the fused kernel reproduces the unsplit chain (no grouped-GEMM workspace)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    return cfg, g, run_chain(cfg, g, gemm_ws=False)


@pytest.fixture(scope="module")
def qwen():
    return _case(moe_synth.config("qwen2"))


@pytest.fixture(scope="module")
def mix():
    # Mixtral-shaped expert widths, fewer tokens, skewed-free routing
    return _case(moe_synth.Config("mix2k", 2048, 4096, 14336, 8, 2, 1, "bf16", 31))


@pytest.fixture(scope="module")
def ep():
    # source-block tagged rows, 8 blocks x 256 tokens
    return _case(moe_synth.Config("ep2k", 2048, 1024, 512, 16, 8, 8, "bf16", 32, 0.0, 256))


@pytest.mark.parametrize("gather", [0, 1])
@pytest.mark.parametrize("n_mover", [0, 1, 2, 8, 32, 64])
def test_schedule_invariance_movers(qwen, n_mover, gather):
    cfg, g, chain = qwen
    out, _, status = run_layer(cfg, g, n_mover=n_mover, gather=gather)
    assert status == moe.MOE_OK
    assert torch.equal(out, chain["out"])


@pytest.mark.parametrize("grid,n_mover,gather", [(7, 0, 0), (16, 2, 1), (64, 8, 0), (200, 3, 1), (256, 0, 0),
                                                 (256, 0, 1), (256, 16, 0)])
def test_schedule_invariance_grid(mix, grid, n_mover, gather):
    cfg, g, chain = mix
    out, _, status = run_layer(cfg, g, n_mover=n_mover, grid=grid, gather=gather)
    assert status == moe.MOE_OK
    assert torch.equal(out, chain["out"])


@pytest.mark.parametrize("gather", [0, 1])
@pytest.mark.parametrize("n_mover", [0, 8])
def test_source_blocks(ep, n_mover, gather):
    cfg, g, chain = ep
    out, _, status = run_layer(cfg, g, n_mover=n_mover, gather=gather)
    assert status == moe.MOE_OK
    assert torch.equal(out, chain["out"])


def test_intermediates_equal_chain(qwen):
    cfg, g, chain = qwen
    if layer_runs_chain(cfg):
        # the default options run the kernel chain, whose GEMM splits the last round
        chain = run_chain(cfg, g, gemm_ws=True)
    out, aux, status = run_layer(cfg, g, aux=True)
    assert status == moe.MOE_OK
    for key in ("topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted", "y"):
        assert torch.equal(aux[key], chain[key]), key
    for key in ("x_perm", "hact"):
        assert torch.equal(aux[key].view(torch.int16), chain[key].view(torch.int16)), key
    assert torch.equal(out, chain["out"])


@pytest.mark.parametrize("gather", [0, 1])
def test_fused_intermediates_equal_unsplit_chain(qwen, gather):
    # forced fused: X_perm (written by the dispatch unless gathering), Hact
    # and Y bit for bit those of the chain without a grouped-GEMM workspace
    cfg, g, chain = qwen
    out, aux, status = run_layer(cfg, g, aux=True, n_mover=0, gather=gather)
    assert status == moe.MOE_OK
    for key in ("topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat", "flat_to_sorted", "y"):
        assert torch.equal(aux[key], chain[key]), key
    for key in ("x_perm", "hact"):
        # aux given: the gathering path writes X_perm too
        assert torch.equal(aux[key].view(torch.int16), chain[key].view(torch.int16)), key
    assert torch.equal(out, chain["out"])


def test_unfused_option_equals_chain(qwen):
    # moe_layer's chain gives its grouped GEMM the workspace (split last round)
    cfg, g, _ = qwen
    chain = run_chain(cfg, g, gemm_ws=True)
    out, _, status = run_layer(cfg, g, fused=0)
    assert status == moe.MOE_OK
    assert torch.equal(out, chain["out"])


def test_default_split_comes_from_table():
    for name in ("qwen2", "mixtral", "phi35", "epshare", "epshare_b"):
        c = moe_synth.config(name)
        m = moe.moe_layer_default_movers(moe.problem(c.M, c.H, c.F, c.E, c.k, c.S, c.dtype, c.base, c.local))
        assert -1 <= m < 64, (name, m)
    assert moe.moe_layer_default_movers(moe.problem(256, 256, 512, 8, 2, 1, "f32")) == -1


def test_watchdog_reports_timeout_and_recovers(mix):
    """A one-poll bound on every wait forces the timeout path from the host:
    the kernel must end (no hang) and report MOE_ERR_DEVICE_TIMEOUT; the next
    call with the default bound must be correct again."""
    cfg, g, chain = mix
    out, _, status = run_layer(cfg, g, n_mover=1, spin_limit=1)
    assert status == moe.MOE_ERR_DEVICE_TIMEOUT
    out, _, status = run_layer(cfg, g, n_mover=8)
    assert status == moe.MOE_OK
    assert torch.equal(out, chain["out"])


def test_invalid_split_is_rejected(qwen):
    cfg, g, _ = qwen
    with pytest.raises(moe.MoeError) as ei:
        run_layer(cfg, g, n_mover=10000, grid=64)
    assert ei.value.status == moe.MOE_ERR_INVALID_ARGUMENT
    with pytest.raises(moe.MoeError) as ei:
        run_layer(cfg, g, n_mover=4, grid=1 << 20)
    assert ei.value.status == moe.MOE_ERR_UNSUPPORTED


def test_unusable_tuning_table_is_an_error(qwen, tmp_path):
    # the plan comes from MOE_TUNING_TABLE when set: a file that cannot be
    # parsed fails the call before anything is launched; an explicit split
    # needs no plan
    cfg, g, chain = qwen
    bad = tmp_path / "bad.json"
    bad.write_text('{"entries": [{"M": 1}]}')
    old = os.environ.get("MOE_TUNING_TABLE")
    os.environ["MOE_TUNING_TABLE"] = str(bad)
    try:
        with pytest.raises(moe.MoeError) as ei:
            run_layer(cfg, g)
        assert ei.value.status == moe.MOE_ERR_INVALID_ARGUMENT
        out, _, status = run_layer(cfg, g, n_mover=0)
        assert status == moe.MOE_OK
        assert torch.equal(out, chain["out"])
    finally:
        if old is None:
            del os.environ["MOE_TUNING_TABLE"]
        else:
            os.environ["MOE_TUNING_TABLE"] = old
