"""Helpers of the GPU parity tests: upload seeded inputs, run the C-ABI
chain step by step, and compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import combine_topk_gate_amd as moe


def dev(a, device="cuda:0"):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def host(t):
    """device tensor -> numpy; bf16 comes back as float64 values."""
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def problem_of(cfg):
    return moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, cfg.dtype, cfg.base, cfg.local)


def upload(d, device="cuda:0"):
    return {k: dev(v, device) for k, v in d.items()}


def run_chain(cfg, g, device="cuda:0", gemm_ws=True, nan_fill=True):
    """moe_route -> moe_dispatch -> moe_grouped_gemm(0) -> (1) -> moe_combine.
    g: dict of device tensors x, logits, src_block, w_gate, w_up, w_down.
    gemm_ws: give the grouped GEMM its workspace (the grid's last round is
    then split along k, as in moe_layer's chain); without it the GEMM runs
    unsplit, which is what the fused kernel reproduces bit for bit.
    nan_fill: X_perm, Hact and Y start as NaN, so a row below offsets[G]
    that no tile writes stays NaN (rows past it, of pairs of experts not
    held, are never written nor read)."""
    p = problem_of(cfg)
    M, k, H, F, G, R = cfg.M, cfg.k, cfg.H, cfg.F, cfg.S * cfg.EL, cfg.M * cfg.k
    act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    fill = float("nan") if nan_fill else 0.0
    o = dict(
        topk_idx=torch.empty((M, k), dtype=torch.int32, device=device),
        topk_w=torch.empty((M, k), dtype=torch.float32, device=device),
        counts=torch.empty(G, dtype=torch.int32, device=device),
        offsets=torch.empty(G + 1, dtype=torch.int32, device=device),
        sorted_to_flat=torch.empty(R, dtype=torch.int32, device=device),
        flat_to_sorted=torch.empty(R, dtype=torch.int32, device=device),
        x_perm=torch.full((R, H), fill, dtype=act, device=device),
        hact=torch.full((R, F), fill, dtype=act, device=device),
        y=torch.full((R, H), fill, dtype=torch.float32, device=device),
        out=torch.full((M, H), fill, dtype=torch.float32, device=device),
    )
    ws = torch.empty(max(moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH), 4), dtype=torch.uint8, device=device)
    moe.moe_route(p, g["logits"], o["topk_idx"], o["topk_w"])
    moe.moe_dispatch(p, g["x"], o["topk_idx"], g.get("src_block"), o["counts"], o["offsets"], o["sorted_to_flat"],
                     o["flat_to_sorted"], o["x_perm"], ws)
    gws = None
    nws = moe.moe_workspace_bytes(p, moe.MOE_OP_GROUPED_GEMM)
    if gemm_ws and nws > 0:
        gws = torch.empty(nws, dtype=torch.uint8, device=device)
    moe.moe_grouped_gemm(p, 0, o["x_perm"], g["w_gate"], g["w_up"], o["offsets"], o["hact"], gws)
    moe.moe_grouped_gemm(p, 1, o["hact"], g["w_down"], None, o["offsets"], o["y"], gws)
    moe.moe_combine(p, o["y"], o["topk_w"], o["flat_to_sorted"], o["out"])
    torch.cuda.synchronize()
    return o


def layer_runs_chain(cfg):
    """True if moe_layer's default plan for cfg is the kernel chain."""
    return cfg.dtype != "bf16" or moe.moe_layer_default_movers(problem_of(cfg)) < 0


def run_layer(cfg, g, device="cuda:0", aux=False, **opts):
    p = problem_of(cfg)
    M, k, H, F, G, R = cfg.M, cfg.k, cfg.H, cfg.F, cfg.S * cfg.EL, cfg.M * cfg.k
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device=device)
    out = torch.empty((M, H), dtype=torch.float32, device=device)
    a = None
    if aux:
        act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        a = dict(
            topk_idx=torch.empty((M, k), dtype=torch.int32, device=device),
            topk_w=torch.empty((M, k), dtype=torch.float32, device=device),
            counts=torch.empty(G, dtype=torch.int32, device=device),
            offsets=torch.empty(G + 1, dtype=torch.int32, device=device),
            sorted_to_flat=torch.empty(R, dtype=torch.int32, device=device),
            flat_to_sorted=torch.empty(R, dtype=torch.int32, device=device),
            # NaN: rows the layer does not write stay NaN
            x_perm=torch.full((R, H), float("nan"), dtype=act, device=device),
            hact=torch.full((R, F), float("nan"), dtype=act, device=device),
            y=torch.full((R, H), float("nan"), dtype=torch.float32, device=device),
        )
    moe.moe_layer(p, g["x"], g["logits"], g.get("src_block"), g["w_gate"], g["w_up"], g["w_down"], out, ws, aux=a,
                  **opts)
    torch.cuda.synchronize()
    status = moe.moe_debug_device_status(p, ws)
    return out, a, status


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def tolerances(cfg):
    """(relative Frobenius, max abs) bounds for outputs: bf16 layers with f32
    accumulation 5e-3 / 2e-2; the f32 layer 1e-5 relative."""
    return (5e-3, 2e-2) if cfg.dtype == "bf16" else (1e-5, None)


def kept_rows(o):
    """Number of sorted rows the chain wrote (offsets[G])."""
    return int(o["offsets"][-1])


def assert_written(o, M):
    """Every row below offsets[G] of X_perm, Hact and Y, and every row of
    out, was written (the NaN fill is gone) and is finite."""
    n = kept_rows(o)
    for key in ("x_perm", "hact", "y"):
        assert bool(torch.isfinite(o[key][:n]).all()), key
    assert bool(torch.isfinite(o["out"][:M]).all()), "out"
