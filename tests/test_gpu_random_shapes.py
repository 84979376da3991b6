"""GPU parity on seeded random shapes (needs an MI355X and the built library).

Each case draws its shape from its own seed -- tokens 1..699, hidden and
ffn 64..512 in steps of 64 (so ragged row tiles, partial column tiles of
both layers and K lengths of one to eight 64-wide steps all occur), 1 to 64
experts, top-k up to 8, 1, 2 or 4 source blocks, every fifth case f32 --
and checks every step of the C-ABI chain against the CPU oracle to the same
bars as the named layers: routing, counts, offsets and the permutation
bit-exact, the dispatch copy bitwise, Hact within one bf16 rounding step
(plus the f32 accumulation error near zero), Y and the output within the
bf16 / f32 tolerances; then moe_layer (its default plan, the fused kernel
with a shared queue, and with dedicated combine workgroups) must reproduce
the matching chain's output bit for bit (the fused kernel the chain run
without a grouped-GEMM workspace).
"""
import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_gpu_util import host, layer_runs_chain, rel_fro, run_chain, run_layer, tolerances, upload

pytestmark = pytest.mark.gpu

N_CASES = 16


def _shape(i):
    rng = np.random.default_rng(5000 + i)
    E = int(rng.choice([1, 2, 3, 5, 8, 16, 24, 40, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    S = int(rng.choice([1, 1, 2, 4]))
    M = int(rng.integers(1, 700))
    H = 64 * int(rng.integers(1, 9))
    F = 64 * int(rng.integers(1, 9))
    dtype = "f32" if i % 5 == 4 else "bf16"
    block = -(-M // S) if S > 1 else 0
    return moe_synth.Config(f"rand{i}", M, H, F, E, k, S, dtype, 7000 + i, 0.0, block)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    cfg = _shape(i)
    print(f"[random] case {i}: {cfg}", flush=True)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    o = run_chain(cfg, g)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                         src_block=d["src_block"], want_rows=True)
    for key in ("topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    assert np.max(np.abs(host(o["topk_w"]) - r["topk_w"])) <= 1e-6
    src = g["x"][o["sorted_to_flat"].long() // cfg.k]
    if cfg.dtype == "bf16":
        assert torch.equal(o["x_perm"].view(torch.int16), src.view(torch.int16))
    else:
        assert torch.equal(o["x_perm"], src)
    # Hact and Y rows in flat order (oracle row f = t*k + j is sorted row f2s[f])
    rows = torch.from_numpy(r["flat_to_sorted"].astype(np.int64)).cuda()
    hact = host(o["hact"][rows])
    if cfg.dtype == "bf16":
        assert np.all(np.abs(hact - r["hact"]) - 2.0 ** -7 * np.abs(r["hact"]) <= 5e-5)
    else:
        assert rel_fro(hact, r["hact"]) <= 1e-5
    rel, mabs = tolerances(cfg)
    y = host(o["y"][rows])
    assert rel_fro(y, r["y"]) <= rel
    out = host(o["out"])
    assert rel_fro(out, r["out"]) <= rel
    if mabs is not None:
        assert np.max(np.abs(y - r["y"])) <= mabs
        assert np.max(np.abs(out - r["out"])) <= mabs
    # the fused kernel reproduces the unsplit chain; moe_layer's own chain
    # (its default plan for some shapes) the split one
    o0 = run_chain(cfg, g, gemm_ws=False)
    for opts in ({}, {"n_mover": 0}, {"n_mover": 3}):
        got, _, status = run_layer(cfg, g, **opts)
        assert status == 0, opts
        ref = o if (not opts and layer_runs_chain(cfg)) or cfg.dtype != "bf16" else o0
        assert torch.equal(got, ref["out"]), opts
