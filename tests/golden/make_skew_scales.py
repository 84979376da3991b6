"""Calibrate the per-expert bias scale of the skewed synthetic layers.

For each skewed workload, find the scale s of the bias s * z (z the
standardised per-expert direction drawn by ``moe_synth``) for which the
standard deviation of the per-expert token fractions counts_e / (M*k),
routed by the ORACLE, equals the target skew (COMET paper review, §5.6.2:
std 0.032 is the production average, 0.05 leaves the lightest expert a few
hundred tokens).  Bisection on [0, 8]; writes ``moe_synth/skew_scales.json``.

Calls only the oracle (and the input generator for the raw draws).

    python tests/golden/make_skew_scales.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import moe_synth  # noqa: E402
import oracle  # noqa: E402


def fraction_std(cfg, scale):
    logits = moe_synth.logits_with_scale(cfg, scale)
    idx, _ = oracle.route(logits, cfg.k)
    counts, _ = oracle.counts_offsets(idx, cfg.E)
    frac = counts / float(cfg.M * cfg.k)
    return float(frac.std()), counts


def calibrate(cfg, steps=60):
    lo, hi = 0.0, 8.0
    for _ in range(steps):
        mid = 0.5 * (lo + hi)
        s, _ = fraction_std(cfg, mid)
        if s < cfg.skew:
            lo = mid
        else:
            hi = mid
    scale = 0.5 * (lo + hi)
    s, counts = fraction_std(cfg, scale)
    return scale, s, counts


def main():
    table = {}
    for name, cfg in moe_synth.CONFIGS.items():
        if cfg.skew == 0.0:
            continue
        scale, s, counts = calibrate(cfg)
        key = f"{cfg.name}:{cfg.seed}:{cfg.M}:{cfg.E}:{cfg.k}:{cfg.skew}"
        table[key] = dict(scale=scale, realised_std=s, counts_min=int(counts.min()),
                          counts_max=int(counts.max()))
        print(key, table[key])
        assert abs(s - cfg.skew) <= 5e-4, (name, s)
    with open(moe_synth.SKEW_FILE, "w") as fh:
        json.dump(table, fh, indent=1, sort_keys=True)
        fh.write("\n")


if __name__ == "__main__":
    main()
