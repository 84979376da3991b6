"""Benchmark of the MoE layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config mixtral]

A step is one pass of the whole layer over one batch of seeded synthetic
input already resident in HBM: route -> dispatch (counts, offsets,
permutation, gather) -> Layer0 grouped GEMM + SwiGLU -> Layer1 grouped GEMM ->
top-k combine, issued through the library's C ABI (``--mode chain``, one
launch per step with HIP events between them) or as one ``moe_layer`` call
(``--mode layer``).  Prints ONE JSON line.

`value` is the layer's algorithmic throughput, 6*R*H*F flop per step / step
time, in TFLOP/s; the JSON also carries the layer time in microseconds, the
grouped-GEMM TFLOP/s and its fraction of the bf16 matrix-core peak, the
per-step times, a roofline object for the dominant kernel (Layer0 grouped
GEMM) timed live with HIP events on the launch stream, and the CPU oracle
timed on a bounded token sample on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3     # MI355X f32 matrix peak
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="mixtral")
    ap.add_argument("--mode", choices=("chain", "layer"), default="layer",
                    help="layer: moe_layer with the library's per-shape choice; chain: moe_layer forced unfused")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--n-mover", type=int, default=-1)
    ap.add_argument("--act", choices=("bf16", "mxfp8"), default="bf16",
                    help="mxfp8: Hact and W_down in MXFP8 (W_down quantised on the GPU before timing)")
    ap.add_argument("--no-dense-ref", action="store_true",
                    help="skip the context line: this GEMM and torch.matmul (hipBLASLt) on one dense expert")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed layer steps before the first timed loop, until this much GPU time has passed "
                         "(the clock takes ~100 ms of load to settle; a short layer's warmup steps alone do "
                         "not cover that)")
    ap.add_argument("--no-extras", action="store_true",
                    help="time only the layer step and the chain (no epilogue, cold-cache, fused or dense "
                         "context measurements): for profiler runs")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mixtral_layer_hbm_traffic.txt")
GEMM_SOURCES = ("combine_topk_gate_amd/csrc/gemm_bf16.hpp", "combine_topk_gate_amd/csrc/ggemm.hip",
                "combine_topk_gate_amd/csrc/tiles.hpp", "combine_topk_gate_amd/csrc/common.hpp")


def gemm_sources_sha() -> str:
    import hashlib
    h = hashlib.sha1()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, or None if it is missing or was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            text = fh.read()
    except OSError:
        return None
    sha = None
    val = None
    for line in text.splitlines():
        if line.startswith("kernel_sources_sha:"):
            sha = line.split(":", 1)[1].strip()
        if line.startswith(f"traffic_bytes_per_launch {kernel_key}:"):
            val = float(line.split(":", 1)[1])
    return val if (sha == gemm_sources_sha() and val) else None


def copy_calibration():
    """A plain device-to-device copy of known size: its FETCH_SIZE and
    WRITE_SIZE counter readings give the scale that turns those counters
    into HBM bytes for the other kernels."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def cpu_baseline(cfg, d, target_s):
    """The oracle as it stands, on a seeded token sample sized for ~target_s."""
    import moe_synth
    import oracle
    flop_pair = 6.0 * cfg.H * cfg.F
    held = dict(expert_base=cfg.base, local_experts=cfg.local)

    def timed(n_tok, tag):
        toks = moe_synth.token_sample(cfg, n_tok, seed_tag=tag)
        t0 = time.perf_counter()
        oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                         src_block=d["src_block"], tokens=toks, **held)
        return len(toks), time.perf_counter() - t0

    # two probe sizes separate the fixed cost (full routing of every token)
    # from the per-token FFN cost, so the sample lands near target_s
    n1, t1 = timed(max(cfg.S, 2), 11)
    n2, t2 = timed(max(cfg.S, 16), 13)
    per_tok = max((t2 - t1) / max(n2 - n1, 1), 1e-6)
    fixed = max(t1 - n1 * per_tok, 0.0)
    n = int(max(cfg.S, min(cfg.M, round((target_s - fixed) / per_tok))))
    toks = moe_synth.token_sample(cfg, n, seed_tag=12)
    t0 = time.perf_counter()
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                         src_block=d["src_block"], tokens=toks, **held)
    dt = time.perf_counter() - t0
    # FFN work only for the pairs whose expert is held
    pairs = int((r["flat_to_sorted"].reshape(cfg.M, cfg.k)[toks] >= 0).sum())
    flops = flop_pair * pairs
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "cpu": model,
            "sample": f"{len(toks)} of {cfg.M} tokens ({pairs} held routed rows, seeded), full routing; "
                      f"{dt:.1f} s fp64 on the host; per-token work is exactly linear, so the full layer "
                      f"would take {dt * cfg.M / len(toks):.0f} s"}


def dense_reference(moe, R, H, F, warmup=3, steps=10):
    """Context, not the metric: the grouped GEMM on one expert of R rows (no
    padding rows, whole rounds of tiles) beside torch.matmul (hipBLASLt) on
    the same products, bf16 inputs, same process and box.  Layer0 here
    writes the SwiGLU activation [R, F]; torch writes both [R, 2F] halves."""
    import torch
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(11)
    p = moe.problem(R, H, F, 1, 1, 1, "bf16")
    x = torch.randn(R, H, device=dev, generator=gen).to(torch.bfloat16)
    wg = (torch.randn(1, F, H, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    wu = (torch.randn(1, F, H, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    wd = (torch.randn(1, H, F, device=dev, generator=gen) * 0.02).to(torch.bfloat16)
    offs = torch.tensor([0, R], dtype=torch.int32, device=dev)
    hact = torch.empty(R, F, dtype=torch.bfloat16, device=dev)
    y = torch.empty(R, H, dtype=torch.float32, device=dev)
    n_ws = moe.moe_workspace_bytes(p, moe.MOE_OP_GROUPED_GEMM)
    gws = torch.empty(n_ws, dtype=torch.uint8, device=dev) if n_ws > 0 else None
    wcat_t = torch.cat([wg[0], wu[0]], 0).t().contiguous()  # [H, 2F]
    wd_t = wd[0].t().contiguous()                             # [F, H]

    def timeit(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / steps  # us

    fl0, fl1 = 4.0 * R * H * F, 2.0 * R * H * F
    t = {"ours_l0": timeit(lambda: moe.moe_grouped_gemm(p, 0, x, wg, wu, offs, hact, gws)),
         "hipblaslt_l0": timeit(lambda: torch.matmul(x, wcat_t)),
         "ours_l1": timeit(lambda: moe.moe_grouped_gemm(p, 1, hact, wd, None, offs, y, gws)),
         "hipblaslt_l1": timeit(lambda: torch.matmul(hact, wd_t))}
    out = {"shape": f"one expert: R={R} H={H} F={F}"}
    for key, us in t.items():
        out[key + "_tflops"] = (fl0 if key.endswith("l0") else fl1) / (us * 1e-6) / 1e12
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the MoE layer benchmark runs on one GPU only; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import combine_topk_gate_amd as moe
    import moe_synth

    def upload(arrs):
        outd = {}
        for key, a in arrs.items():
            if a is None:
                outd[key] = None
            elif a.dtype == np.uint16:
                outd[key] = torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
            else:
                outd[key] = torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")
        return outd

    moe.load_library()
    cfg = moe_synth.config(args.config)
    if args.act == "mxfp8":
        cfg = moe_synth.config(args.config, dtype="bf16_mxfp8")
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    mx = cfg.dtype == "bf16_mxfp8"
    w_down = g["w_down"]
    if mx:
        # the layer's input format: W_down in MXFP8, quantised once before timing
        w_down = torch.empty(moe.mx_bytes(cfg.EL * cfg.H, cfg.F), dtype=torch.uint8, device="cuda:0")
        moe.moe_quantize_mxfp8(g["w_down"], w_down)
        torch.cuda.synchronize()
    dev = torch.device("cuda:0")
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, cfg.dtype, cfg.base, cfg.local)
    M, k, H, F, G, R = cfg.M, cfg.k, cfg.H, cfg.F, cfg.S * cfg.EL, cfg.R
    act = torch.float32 if cfg.dtype == "f32" else torch.bfloat16
    idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    w = torch.empty((M, k), dtype=torch.float32, device=dev)
    counts = torch.empty(G, dtype=torch.int32, device=dev)
    offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    s2f = torch.empty(R, dtype=torch.int32, device=dev)
    f2s = torch.empty(R, dtype=torch.int32, device=dev)
    xp = torch.empty((R, H), dtype=act, device=dev)
    hact = torch.empty(moe.mx_bytes(R, F), dtype=torch.uint8, device=dev) if mx else \
        torch.empty((R, F), dtype=act, device=dev)
    y = torch.empty((R, H), dtype=torch.float32, device=dev)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws_d = torch.empty(max(4, moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH)), dtype=torch.uint8, device=dev)
    ws_l = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device=dev)
    n_gws = moe.moe_workspace_bytes(p, moe.MOE_OP_GROUPED_GEMM)
    ws_g = torch.empty(n_gws, dtype=torch.uint8, device=dev) if n_gws > 0 else None
    stream = torch.cuda.current_stream()
    src = g.get("src_block")

    def time_steps(fn, nev, warmup, steps):
        for _ in range(warmup):
            fn(None)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(steps)]
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(steps):
            fn(evs[i])
        t1.record(stream)
        torch.cuda.synchronize()
        per = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nev - 1)]
                        for i in range(steps)]) * 1e3  # us
        return t0.elapsed_time(t1) / steps, per

    def step_chain(ev):
        if ev: ev[0].record(stream)
        moe.moe_route(p, g["logits"], idx, w, stream)
        if ev: ev[1].record(stream)
        moe.moe_dispatch(p, g["x"], idx, src, counts, offsets, s2f, f2s, xp, ws_d, stream)
        if ev: ev[2].record(stream)
        moe.moe_grouped_gemm(p, 0, xp, g["w_gate"], g["w_up"], offsets, hact, ws_g, stream)
        if ev: ev[3].record(stream)
        moe.moe_grouped_gemm(p, 1, hact, w_down, None, offsets, y, ws_g, stream)
        if ev: ev[4].record(stream)
        moe.moe_combine(p, y, w, f2s, out, stream)
        if ev: ev[5].record(stream)

    def step_layer(ev):
        if ev: ev[0].record(stream)
        moe.moe_layer(p, g["x"], g["logits"], src, g["w_gate"], g["w_up"], w_down, out, ws_l,
                      n_mover=args.n_mover, fused=0 if args.mode == "chain" else 1, stream=stream)
        if ev: ev[1].record(stream)

    # (0) untimed layer steps until the clock has settled (a loop measured
    #     sooner reads 8-15% slow at Qwen2's 0.5 ms layer and runs behind
    #     the loops measured after it)
    settled_ms = 0.0
    if args.settle_ms > 0:
        t_start = torch.cuda.Event(enable_timing=True)
        t_now = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        while settled_ms < args.settle_ms:
            for _ in range(4):
                step_layer(None)
            t_now.record(stream)
            t_now.synchronize()
            settled_ms = t_start.elapsed_time(t_now)
    # (1) the step: one moe_layer call (the library's per-shape choice of the
    #     fused kernel or the chain), timed as a whole
    ms_step, per_layer = time_steps(step_layer, 2, args.warmup, args.steps)
    # (2) the same layer as the chain of C-ABI calls, with an event between
    #     calls: per-step times and the dominant kernel's live duration
    ms_chain, per = time_steps(step_chain, 6, args.warmup, args.steps)

    # (3) the combine with the output epilogue: a bf16 residual added and the
    #     result cast to bf16 (the option a model layer would use)
    res_in = torch.randn((M, H), generator=torch.Generator().manual_seed(3)).to(act).to(dev)
    out_bf16 = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    epi = moe.epilogue(res_in, "bf16")

    def step_epilogue(ev):
        if ev: ev[0].record(stream)
        moe.moe_combine_ex(p, y, w, f2s, epi, out_bf16, stream)
        if ev: ev[1].record(stream)

    per_epi = np.array([[np.nan]])
    if not args.no_extras:
        _, per_epi = time_steps(step_epilogue, 2, args.warmup, args.steps)

    # (4) cold cache: dispatch and combine alone with a 1 GiB scrub between
    #     repetitions, so the 256 MB last-level cache holds nothing of their
    #     inputs; only the call itself is timed.  The scrub is written (the
    #     cache is then full of dirty lines that must be written back as the
    #     call evicts them) or read (clean lines)
    scrub = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    scrub32 = scrub.view(torch.float32)

    def cold(fn, reps, mode="write"):
        ts = []
        for i in range(reps + 2):
            if mode == "write":
                scrub.fill_(i & 0xFF)
            else:
                float(scrub32.sum())
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            fn()
            b_.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a_.elapsed_time(b_) * 1e3)
        return np.array(ts)

    cold_t = {}
    if not args.no_extras:
        scrub.zero_()
        for mode in ("write", "read"):
            cold_t[mode] = {
                "dispatch": cold(lambda: moe.moe_dispatch(p, g["x"], idx, src, counts, offsets, s2f, f2s, xp, ws_d,
                                                          stream), args.steps, mode),
                "combine": cold(lambda: moe.moe_combine(p, y, w, f2s, out, stream), args.steps, mode)}
    del scrub, scrub32

    # (5) the fused kernel at this shape (whatever the table picks for the
    #     step above): shared queue, 8 dedicated combine workgroups, and the
    #     shared queue with Layer0 reading the dispatch's X_perm copy
    fused_us = {}
    if cfg.dtype == "bf16" and not args.no_extras:
        for nm, ga in ((0, 1), (8, 1), (0, 0)):
            def step_fused(ev, nm=nm, ga=ga):
                if ev: ev[0].record(stream)
                moe.moe_layer(p, g["x"], g["logits"], src, g["w_gate"], g["w_up"], w_down, out, ws_l,
                              n_mover=nm, fused=1, gather=ga, stream=stream)
                if ev: ev[1].record(stream)
            ms_f, _ = time_steps(step_fused, 2, 2, max(3, args.steps // 4))
            fused_us[f"n_mover={nm}" + ("" if ga else ",copy")] = ms_f * 1e3

    # pairs routed to held experts (all of them unless only some are held)
    Rk = int(offsets[-1].item())
    Tk = int((f2s.view(M, k) >= 0).any(dim=1).sum().item())
    flops = 6.0 * Rk * H * F
    movers = moe.moe_layer_default_movers(p) if args.n_mover < 0 else args.n_mover
    res = {"metric": "MoE layer us + grouped-GEMM TFLOP/s (% MFMA peak), Mixtral shape M=8192",
           "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "settle_ms": round(settled_ms, 1), "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": {"bf16": "bf16", "f32": "f32", "bf16_mxfp8": "bf16+mxfp8"}[cfg.dtype],
           "data": "synthetic (seeded N(0,1) tokens and logits, N(0,0.02^2) weights, random-init)",
           "config": {"workload": f"{cfg.name}: MoE layer M={M} H={H} F={F} E={cfg.E} topk={k} S={cfg.S}"
                      + (f" experts held {cfg.base}..{cfg.base + cfg.EL - 1}" if cfg.local else "")
                      + (", Hact and W_down MXFP8" if mx else ""),
                      "tokens": M, "hidden": H, "ffn": F, "experts": cfg.E, "topk": k, "src_blocks": cfg.S,
                      "experts_held": cfg.EL, "routed_rows_held": Rk,
                      "layer_call": "fused" if (args.mode == "layer" and movers >= 0 and cfg.dtype == "bf16")
                      else "chain", "n_mover": movers},
           "layer_us": ms_step * 1e3, "chain_us": ms_chain * 1e3,
           "layer_us_p10_p50_p90": [float(np.percentile(per_layer[:, 0], q)) for q in (10, 50, 90)]}
    mean = per.mean(axis=0)
    names = ["route", "dispatch", "gemm_l0", "gemm_l1", "combine"]
    res["step_us"] = {n: float(v) for n, v in zip(names, mean)}
    res["step_us_p10_p50_p90"] = {n: [float(np.percentile(per[:, i], q)) for q in (10, 50, 90)]
                                  for i, n in enumerate(names)}
    t_gemm = (mean[2] + mean[3]) * 1e-6
    peak = PEAK_F32_TFLOPS if cfg.dtype == "f32" else PEAK_BF16_TFLOPS
    res["grouped_gemm_tflops"] = flops / t_gemm / 1e12
    if mx:
        # Layer0 at the bf16 peak, Layer1 (MXFP8) at the fp8 peak
        ideal = (4.0 * Rk * H * F / PEAK_BF16_TFLOPS + 2.0 * Rk * H * F / PEAK_FP8_TFLOPS) / 1e12
        res["grouped_gemm_pct_peak"] = 100.0 * ideal / t_gemm
        res["gemm_l1_mxfp8_pct_peak"] = 100.0 * 2.0 * Rk * H * F / (mean[3] * 1e-6) / 1e12 / PEAK_FP8_TFLOPS
    else:
        res["grouped_gemm_pct_peak"] = 100.0 * res["grouped_gemm_tflops"] / peak
    eb = 4 if cfg.dtype == "f32" else 2  # bytes of an x / X_perm element
    # token rows read (those with a held pair), rows written, the index list
    disp_bytes = Tk * H * eb + Rk * H * eb + R * 4
    comb_bytes = Rk * H * 4 + M * H * 4 + M * k * 8
    epi_bytes = Rk * H * 4 + M * H * eb + M * H * 2 + M * k * 8
    if not args.no_extras:
        res["combine_epilogue_us"] = float(per_epi.mean())
        res["combine_epilogue_gbs"] = epi_bytes / (per_epi.mean() * 1e-6) / 1e9
    res["dispatch_gbs"] = disp_bytes / (mean[1] * 1e-6) / 1e9
    res["combine_gbs"] = comb_bytes / (mean[4] * 1e-6) / 1e9
    res["dispatch_pct_hbm"] = 100.0 * res["dispatch_gbs"] / PEAK_HBM_GBS
    res["combine_pct_hbm"] = 100.0 * res["combine_gbs"] / PEAK_HBM_GBS
    # the same two calls timed alone after a 1 GiB scrub (cold last-level cache)
    for mode, tt in cold_t.items():
        res[f"cold_{mode}_scrub_us_p10_p50_p90"] = {k_: [float(np.percentile(v_, q)) for q in (10, 50, 90)]
                                                   for k_, v_ in tt.items()}
        res[f"dispatch_cold_{mode}_scrub_pct_hbm"] = (100.0 * disp_bytes / (np.median(tt["dispatch"]) * 1e-6) / 1e9
                                                     / PEAK_HBM_GBS)
        res[f"combine_cold_{mode}_scrub_pct_hbm"] = (100.0 * comb_bytes / (np.median(tt["combine"]) * 1e-6) / 1e9
                                                    / PEAK_HBM_GBS)
    # single-GPU analogue of hidden communication (the pages' share of
    # communication hidden): 1 - (fused - route - L0 - L1) / (dispatch +
    # combine), with the chain's step times; negative when the fused kernel
    # costs more than the movement it overlaps
    move = mean[1] + mean[4]
    res["fused_us"] = fused_us or None
    if fused_us:
        best = min(fused_us.values())
        res["movement_hidden_pct"] = 100.0 * (1.0 - (best - mean[0] - mean[2] - mean[3]) / move)
    else:
        res["movement_hidden_pct"] = None
    l0_flops = 4.0 * Rk * H * F
    ach = l0_flops / (mean[2] * 1e-6) / 1e12
    # bf16 rows from several source blocks whose (block, expert) segments
    # average under one 256-row tile run the kernel over combined per-expert
    # segments (the library's rule, api.hip combine_blocks)
    rowmap = cfg.dtype == "bf16" and cfg.S > 1 and cfg.M * cfg.k < 256 * cfg.E * cfg.S
    l0_kernel = ("grouped_gemm_f32_kernel<0>" if cfg.dtype == "f32" else
                 "grouped_gemm_bf16_expert_kernel<0>" if rowmap else "grouped_gemm_bf16_kernel<0>")
    res["roofline"] = {"kernel": f"{l0_kernel} (Layer0 gate/up + SwiGLU), chain timing",
                       "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                       "traffic": measured_traffic("grouped_gemm_bf16_kernel<0>") if cfg.name == "mixtral" else None,
                       "traffic_scope": "bytes between the XCDs' L2 caches and the memory fabric per launch "
                                        "(rocprofv3 FETCH_SIZE / WRITE_SIZE scaled by a plain 1 GiB copy); "
                                        "reads the 256 MB last-level cache serves are included",
                       "launch_us": float(mean[2]),
                       "algorithmic": f"4*R*H*F = {l0_flops:.4g} flop per launch"}
    if cfg.dtype == "bf16" and not args.no_dense_ref and not args.no_extras:
        res["context_dense_same_shape"] = dense_reference(moe, R, H, F)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, d, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
