"""MOE_DEBUG_VALIDATE=1: the entry points check the device-resident inputs
they trust on the host before launching anything and return
MOE_ERR_INVALID_ARGUMENT for inconsistent ones.  The inconsistent inputs
here are also harmless when not caught (the kernels keep every access
inside the buffers), so a checker that missed them would fail this test
rather than the device."""
import os

import numpy as np
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import run_chain, upload

pytestmark = pytest.mark.gpu


@pytest.fixture
def validating(monkeypatch):
    monkeypatch.setenv("MOE_DEBUG_VALIDATE", "1")
    yield


def _case():
    cfg = moe_synth.Config("validate", 300, 128, 128, 8, 2, 1, "bf16", 77)
    g = upload(moe_synth.make_inputs(cfg))
    return cfg, g


def test_consistent_inputs_pass_and_give_the_same_bits(validating):
    cfg, g = _case()
    a = run_chain(cfg, g)
    os.environ.pop("MOE_DEBUG_VALIDATE")
    b = run_chain(cfg, g)
    for key in ("topk_idx", "offsets", "sorted_to_flat", "out"):
        assert torch.equal(a[key], b[key]), key


def test_inconsistent_offsets_are_rejected_before_the_gemm(validating):
    cfg, g = _case()
    o = run_chain(cfg, g)
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k)
    R = cfg.M * cfg.k
    # (an end past R is rejected too, but is not fed to the device here: a
    # GEMM that ran on it would read past the token rows)
    bad = {"decreasing": [0, 90, 60] + [R] * (cfg.E - 2), "not_from_zero": [5] + list(range(6, 6 + cfg.E))}
    for name, offs in bad.items():
        offs = torch.tensor(offs, dtype=torch.int32, device="cuda")
        assert offs.numel() == cfg.E + 1
        hact = o["hact"].clone()
        with pytest.raises(moe.MoeError) as ex:
            moe.moe_grouped_gemm(p, 0, o["x_perm"], g["w_gate"], g["w_up"], offs, hact)
        assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT, name
        torch.cuda.synchronize()
        assert torch.equal(hact.view(torch.int16), o["hact"].view(torch.int16)), name  # nothing launched


def test_out_of_range_routing_is_rejected(validating):
    cfg, g = _case()
    o = run_chain(cfg, g)
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k)
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH), dtype=torch.uint8, device="cuda")
    for bad_val in (cfg.E, -1):
        idx = o["topk_idx"].clone()
        idx[7, 1] = bad_val
        with pytest.raises(moe.MoeError) as ex:
            moe.moe_dispatch(p, g["x"], idx, None, o["counts"], o["offsets"], o["sorted_to_flat"],
                             o["flat_to_sorted"], o["x_perm"], ws)
        assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT
    # source blocks out of range
    pS = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, S=2)
    src = torch.zeros(cfg.M, dtype=torch.int32, device="cuda")
    src[3] = 2
    counts2 = torch.empty(2 * cfg.E, dtype=torch.int32, device="cuda")
    offs2 = torch.empty(2 * cfg.E + 1, dtype=torch.int32, device="cuda")
    ws2 = torch.empty(moe.moe_workspace_bytes(pS, moe.MOE_OP_DISPATCH), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_dispatch(pS, g["x"], o["topk_idx"], src, counts2, offs2, o["sorted_to_flat"], o["flat_to_sorted"],
                         o["x_perm"], ws2)
    assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT
    # combine: a row index past R
    f2s = o["flat_to_sorted"].clone()
    f2s[0] = cfg.M * cfg.k
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_combine(p, o["y"], o["topk_w"], f2s, o["out"])
    assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT


def test_non_finite_logits_are_rejected(validating):
    cfg, g = _case()
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k)
    lg = g["logits"].clone()
    lg[11, 3] = float("nan")
    idx = torch.empty((cfg.M, cfg.k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.M, cfg.k), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_route(p, lg, idx, w)
    assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_layer(p, g["x"], lg, None, g["w_gate"], g["w_up"], g["w_down"], out, ws)
    assert ex.value.status == moe.MOE_ERR_INVALID_ARGUMENT


def test_out_of_range_expert_ids_stay_inside_the_buffers_without_validation():
    """Without the checker an out-of-range expert id makes its pair a dropped
    one: it gets no sorted position (-1) and the others keep theirs."""
    cfg, g = _case()
    o = run_chain(cfg, g)
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k)
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH), dtype=torch.uint8, device="cuda")
    idx = o["topk_idx"].clone()
    idx[7, 1] = cfg.E + 3
    R = cfg.M * cfg.k
    s2f = torch.full((R,), -5, dtype=torch.int32, device="cuda")
    f2s = torch.empty(R, dtype=torch.int32, device="cuda")
    counts = torch.empty(cfg.E, dtype=torch.int32, device="cuda")
    offs = torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda")
    xp = torch.zeros_like(o["x_perm"])
    moe.moe_dispatch(p, g["x"], idx, None, counts, offs, s2f, f2s, xp, ws)
    torch.cuda.synchronize()
    assert int(f2s[7 * cfg.k + 1]) == -1
    assert int(offs[-1]) == R - 1 and int(counts.sum()) == R - 1
    kept = np.sort(s2f[: R - 1].cpu().numpy())
    assert np.array_equal(kept, np.setdiff1d(np.arange(R), [7 * cfg.k + 1]))
