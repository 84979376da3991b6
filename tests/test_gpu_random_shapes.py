"""GPU parity on seeded random shapes (needs an MI355X and the built library).

Small cases draw their shape from their own seed -- tokens 1..699, hidden
and ffn 64..512 in steps of 64 (so ragged row tiles, partial column tiles
of both layers and K lengths of one to eight 64-wide steps all occur), 1 to
64 experts, top-k up to 8, 1, 2 or 4 source blocks, every fifth case f32 --
and are compared with the full oracle layer.  Multi-round cases (3000..6000
tokens, hidden and ffn up to 4096) give the persistent grid more than one
round of tiles, a last round of half tiles or of k-split tiles, and
segments tall enough for the tile order's row blocks; they are compared on
rows covering every tile and on a token sample.  Every case:
routing, counts, offsets and the permutation bit-exact, the dispatch copy
bitwise, every row written (NaN-filled intermediates), Hact, Y and the
output element by element within the bounds of parity_bounds and the
layer tolerances; then moe_layer (its default plan, the fused kernel with a
shared queue, and with dedicated combine workgroups) must reproduce the
matching chain's output bit for bit (the fused kernel the chain run without
a grouped-GEMM workspace).
"""
import numpy as np
import pytest
import torch

import moe_synth
import tile_parity as tp
from moe_gpu_util import assert_written, host, layer_runs_chain, run_chain, run_layer, upload

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


# Shapes past one round of the 256-CU grid, each aimed at one part of the
# tile schedule (row tiles x column tiles per layer in the comments).
MULTI = {
    # 2 segments of ~3000 rows (12 row tiles: cut into row blocks); Layer0
    # 24 x 18 = 432 tiles (1.7 rounds); Layer1 96 tiles split 2 ways along k
    "tall_row_blocks": dict(M=6000, H=1024, F=2304, E=2, k=1),
    # Layer0 40 x 7 = 280 tiles: a last round of 24 tiles run as 48 halves
    "l0_halves": dict(M=5000, H=768, F=896, E=4, k=2),
    # Layer1 32 x 12 = 384 tiles: a last round of 128 tiles run as 256 halves
    "l1_halves": dict(M=4000, H=3072, F=512, E=2, k=2),
    # Layer0 32 x 32 = 1024 tiles (4 whole rounds); Layer1 32 x 10 = 320:
    # a last round of 64 tiles split 4 ways along k
    "l0_whole_rounds": dict(M=4000, H=2560, F=4096, E=2, k=2),
    # Layer1 28 x 12 = 336 tiles: a last round of 80 tiles split 3 ways along k
    "l1_split3": dict(M=3500, H=3072, F=4736, E=2, k=2),
    # held experts 2..5 of 8, two source blocks: ~750-row segments
    "held_src_blocks": dict(M=6000, H=1024, F=1536, E=8, k=2, S=2, base=2, local=4),
    # 32 experts of ~375 rows: 64 x 6 = 384 Layer0 tiles, halves in the last round
    "many_experts": dict(M=3000, H=512, F=768, E=32, k=4),
}


def _multi_shape(name):
    kw = dict(MULTI[name])
    S = kw.pop("S", 1)
    base, local = kw.pop("base", 0), kw.pop("local", 0)
    return moe_synth.Config(name, kw["M"], kw["H"], kw["F"], kw["E"], kw["k"], S, "bf16",
                            7100 + sorted(MULTI).index(name), 0.0, (kw["M"] // S) if S > 1 else 0, base, local)


def _check(cfg, toks, seed):
    print(f"[random] {cfg}", flush=True)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    o = run_chain(cfg, g)
    c = tp.oracle_case(cfg.name, cfg, d, g, o, toks, seed)
    r = c["ref"]
    for key in ("topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    assert np.max(np.abs(host(o["topk_w"]) - r["topk_w"])) <= 1e-6
    n = int(r["offsets"][-1])  # rows past the kept pairs are not written
    src = g["x"][o["sorted_to_flat"][:n].long() // cfg.k]
    if cfg.dtype == "bf16":
        assert torch.equal(o["x_perm"][:n].view(torch.int16), src.view(torch.int16))
    else:
        assert torch.equal(o["x_perm"][:n], src)
    assert_written(o, cfg.M)
    tp.check_ffn(c, o, "chain")
    tp.check_out(c, o, o["out"], "chain")
    # the fused kernel reproduces the unsplit chain; moe_layer's own chain
    # (its default plan for some shapes) the split one
    o0 = run_chain(cfg, g, gemm_ws=False)
    for opts in ({}, {"n_mover": 0}, {"n_mover": 3}):
        got, _, status = run_layer(cfg, g, **opts)
        assert status == 0, opts
        ref = o if (not opts and layer_runs_chain(cfg)) or cfg.dtype != "bf16" else o0
        assert torch.equal(got, ref["out"]), opts


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_parity(i):
    _check(_shape(i), None, 8000 + i)


@pytest.mark.parametrize("name", list(MULTI))
def test_multi_round_shape_parity(name):
    cfg = _multi_shape(name)
    _check(cfg, moe_synth.token_sample(cfg, 48), 8100 + sorted(MULTI).index(name))
