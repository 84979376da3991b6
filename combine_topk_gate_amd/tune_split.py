"""Profile the fused layer's split on this GPU and print the table entries.

    python -m combine_topk_gate_amd.tune_split [--configs qwen2,mixtral,...] [--reps 10]

For each workload it times moe_layer as the kernel chain and as the fused
kernel with every candidate number of dedicated combine workgroups
(0 = combine items in the shared queue), and prints one JSON line per
workload plus the C++ table rows (the split table in csrc/layer.hip) for the
fastest fused split; with --write PATH it also writes them as the JSON table
the library reads when MOE_TUNING_TABLE=PATH is set (the format of
combine_topk_gate_amd/tuning/mi355x.json).  The split is picked ahead of
time and looked up at run time, as COMET does with its profiled per-shape
metadata (paper review §4.2.2).
"""
from __future__ import annotations

import argparse
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--configs", default="qwen2,mixtral,phi35,epshare,epshare_b")
    ap.add_argument("--movers", default="0,2,4,8,16,32")
    ap.add_argument("--reps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed layer calls per workload before its first timing, until this much GPU time "
                         "has passed (the clock takes ~100 ms of load to settle)")
    ap.add_argument("--write", default="", help="write the table as JSON to this path")
    args = ap.parse_args()

    import torch

    import combine_topk_gate_amd as moe
    import moe_synth

    def up(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")

    rows, entries = [], []
    for name in args.configs.split(","):
        cfg = moe_synth.config(name)
        d = moe_synth.make_inputs(cfg)
        g = {k: up(v) for k, v in d.items()}
        del d
        p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, cfg.dtype, cfg.base, cfg.local)
        ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda:0")
        out = torch.empty((cfg.M, cfg.H), dtype=torch.float32, device="cuda:0")

        def run(**opts):
            moe.moe_layer(p, g["x"], g["logits"], g.get("src_block"), g["w_gate"], g["w_up"], g["w_down"], out,
                          ws, **opts)

        def timeit(**opts):
            for _ in range(args.warmup):
                run(**opts)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.reps):
                run(**opts)
            e1.record()
            torch.cuda.synchronize()
            assert moe.moe_debug_device_status(p, ws) == moe.MOE_OK
            return e0.elapsed_time(e1) / args.reps * 1e3

        # the clock settles under load before the first variant is timed, so
        # the variant timed first is not the one that pays for it
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        settled = 0.0
        while settled < args.settle_ms:
            for _ in range(4):
                run(fused=0)
            t1.record()
            t1.synchronize()
            settled = t0.elapsed_time(t1)
        res = {"config": name, "chain_us": timeit(fused=0)}
        for m in (int(v) for v in args.movers.split(",")):
            res[f"fused_m{m}_us"] = timeit(fused=1, n_mover=m)
        best = min((v, k) for k, v in res.items() if k.startswith("fused_"))
        res["best"] = best[1]
        print(json.dumps(res), flush=True)
        m = int(best[1].split("_m")[1].split("_")[0])
        # the chain where it beats every fused split
        m = -1 if res["chain_us"] < best[0] else m
        rows.append(f"    {{{cfg.M}, {cfg.H}, {cfg.F}, {cfg.E}, {cfg.k}, {cfg.S}, {cfg.EL}, {m}}},")
        entries.append({"config": name, "M": cfg.M, "H": cfg.H, "F": cfg.F, "E": cfg.E, "k": cfg.k, "S": cfg.S,
                        "EL": cfg.EL, "n_mover": m, "chain_us": round(res["chain_us"]),
                        "best_fused_us": round(best[0])})
        del g, ws, out
        torch.cuda.empty_cache()
    print("\n".join(rows))
    if args.write:
        props = torch.cuda.get_device_properties(0)
        table = {"device": f"{props.name} ({props.multi_processor_count} CUs, one workgroup per CU)",
                 "written_by": "python -m combine_topk_gate_amd.tune_split --write " + args.write,
                 "meaning": "n_mover: dedicated combine workgroups of the fused layer (0: combine items in the "
                            "shared queue); -1: the kernel chain, faster than every fused split. Shapes not "
                            "listed run the chain.",
                 "entries": entries}
        with open(args.write, "w") as fh:
            json.dump(table, fh, indent=2)
            fh.write("\n")


if __name__ == "__main__":
    main()
