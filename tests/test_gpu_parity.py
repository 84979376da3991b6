"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs (needs an MI355X and the built library).

Routing indices, counts, offsets and the permutation are compared in full
and must be bit-exact; the dispatch copy must be bitwise; the top-k weights
within 1e-6 absolute.  The FFN is compared element by element on rows that
cover every tile of both grouped GEMMs (parity_bounds.covering_rows: a row
in every 128-row half of every 256-row tile of every segment, chosen from
the oracle's own offsets) and on every pair of a seeded token sample; the
combine on that token sample.  Each element must lie within the bound the
arithmetic allows (parity_bounds: f32 accumulation of exact products, the
SwiGLU derivatives, both sides' bf16 rounding of the activation, the
GPU's own Hact fed to Layer1), and the outputs within relative Frobenius
5e-3 and max abs 2e-2 (bf16 layers) or 1e-5 relative (the f32 layer).
Every intermediate starts as NaN, so a row no tile writes fails at any
size.
"""
import gc

import numpy as np
import pytest
import torch

import moe_synth
import oracle
import parity_bounds as pb
import tile_parity as tp
from moe_gpu_util import (assert_written, dev, host, kept_rows, layer_runs_chain, rel_fro, run_chain, run_layer,
                          tolerances, upload)

pytestmark = pytest.mark.gpu

# tokens of the combine sample (None: all tokens); covering rows are added for the FFN
SAMPLE = {"tiny": None, "qwen2": 64, "mixtral": 24, "phi35": 24, "epshare": 16, "epshare_b": 64}

NAMES = list(SAMPLE)


@pytest.fixture(scope="module", params=NAMES)
def case(request):
    """Inputs, GPU chain outputs and the oracle for one named layer; module
    scope, so pytest runs every test of one layer before building the next."""
    c = _build_case(request.param)
    yield c
    c.clear()
    gc.collect()
    torch.cuda.empty_cache()


def _build_case(name):
    cfg = moe_synth.config(name)
    print(f"[parity] preparing {name} {cfg}", flush=True)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    out = run_chain(cfg, g)
    toks = None if SAMPLE[name] is None else moe_synth.token_sample(cfg, SAMPLE[name])
    return tp.oracle_case(name, cfg, d, g, out, toks, cfg.seed + 1000)


def test_route_bit_exact(case):
    c = case
    assert np.array_equal(host(c["out"]["topk_idx"]), c["ref"]["topk_idx"])
    assert np.max(np.abs(host(c["out"]["topk_w"]) - c["ref"]["topk_w"])) <= 1e-6


def test_dispatch_bit_exact(case):
    c = case
    o, r, cfg = c["out"], c["ref"], c["cfg"]
    for key in ("counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    # X_perm[r] is token s2f[r] // k, bit for bit, for every kept row (checked
    # on the device in full); rows past the kept pairs are not written
    n = int(r["offsets"][-1])
    src = c["g"]["x"][(o["sorted_to_flat"][:n].long() // cfg.k)]
    xp = o["x_perm"][:n]
    assert torch.equal(xp.view(torch.int16) if cfg.dtype == "bf16" else xp,
                       src.view(torch.int16) if cfg.dtype == "bf16" else src)


def test_every_row_written(case):
    """NaN-filled intermediates: every tile of both GEMMs wrote its rows."""
    assert_written(case["out"], case["cfg"].M)


def test_layer0_and_layer1_every_tile(case):
    tp.check_ffn(case, case["out"], "chain")


def test_combine_output(case):
    tp.check_out(case, case["out"], case["out"]["out"], "chain")


def test_layer_equals_chain_bitwise(case):
    c = case
    out, _, status = run_layer(c["cfg"], c["g"])
    assert status == 0
    ref = c["out"] if layer_runs_chain(c["cfg"]) else run_chain(c["cfg"], c["g"], gemm_ws=False)
    assert torch.equal(out, ref["out"])


@pytest.mark.parametrize("n_mover,gather", [(0, 0), (8, 0), (0, 1), (8, 1)])
def test_fused_layer_against_oracle(case, n_mover, gather):
    """The fused kernel (Layer0 reading X_perm, or with gather = 1 the token
    rows straight from x; one ordered queue, ready counters) at the full
    shape, against the oracle directly: its Hact and Y on the tile-covering
    rows and its output on the token sample; and bitwise against the
    unsplit chain."""
    c = case
    if c["cfg"].dtype != "bf16":
        pytest.skip("the fused kernel runs bf16 layers")
    out, aux, status = run_layer(c["cfg"], c["g"], aux=True, n_mover=n_mover, gather=gather)
    assert status == 0
    n = kept_rows(aux)
    assert n == int(c["ref"]["offsets"][-1])
    keys = ("hact", "y") if gather else ("x_perm", "hact", "y")
    for key in keys:
        assert bool(torch.isfinite(aux[key][:n]).all()), key
    name = f"fused n_mover={n_mover} gather={gather}"
    tp.check_ffn(c, aux, name)
    tp.check_out(c, aux, out, name)
    un = run_chain(c["cfg"], c["g"], gemm_ws=False)
    assert torch.equal(out, un["out"])


def _check_against_exact(cfg, g, chain, elems, hacts):
    """Each Hact value at (row, col) in elems lies within the bound of
    parity_bounds.hact_allowance around the oracle-free exact value (the f64
    gate and up sums of the bf16 operands): used where two GPU runs differ
    by more than one bf16 step."""
    if not elems:
        return
    offs = chain["offsets"].cpu().numpy()
    rows = np.array([r for r, _ in elems], np.int64)
    cols = np.array([c_ for _, c_ in elems], np.int64)
    experts = pb.experts_of(offs, rows, cfg.EL)
    tok = chain["sorted_to_flat"][torch.from_numpy(rows).cuda()].long() // cfg.k
    sums = pb.gate_up_sums(g["x"][tok], g["w_gate"], g["w_up"], experts)
    allow = pb.hact_allowance(sums, True)
    exact = pb.silu64(sums["g"]) * sums["u"]
    sel = torch.arange(len(rows), device="cuda")
    ccol = torch.from_numpy(cols).cuda()
    for h in hacts:
        got = h[torch.from_numpy(rows).cuda(), ccol]
        assert bool(((got - exact[sel, ccol]).abs() <= allow[sel, ccol]).all())


def test_split_last_round_matches_unsplit(case):
    """The grouped GEMM with its workspace (last round split along k) against
    the same GEMM without it: identical routing and Hact/Y within f32
    regrouping error; and the split path is deterministic."""
    c = case
    if c["cfg"].dtype != "bf16":
        pytest.skip("f32 layers do not split")
    n = kept_rows(c["out"])
    un = run_chain(c["cfg"], c["g"], gemm_ws=False)
    again = run_chain(c["cfg"], c["g"], gemm_ws=True)
    for key in ("hact", "y"):
        assert torch.equal(again[key][:n].view(torch.int32 if key == "y" else torch.int16),
                           c["out"][key][:n].view(torch.int32 if key == "y" else torch.int16)), key
    assert torch.equal(again["out"], c["out"]["out"])
    y0, y1 = un["y"][:n].double(), c["out"]["y"][:n].double()
    assert float((y1 - y0).norm() / y0.norm()) <= 1e-5
    h0, h1 = un["hact"][:n].double(), c["out"]["hact"][:n].double()
    # a regrouped f32 sum may cross a bf16 rounding boundary: one step at most,
    # unless the gate or up sum cancels (|sum| << sum of |terms|); such
    # elements are checked against the exact f64 value instead
    far = ((h1 - h0).abs() > 2.0 ** -7 * h0.abs() + 1e-6).nonzero().tolist()
    assert len(far) <= 64, len(far)
    _check_against_exact(c["cfg"], c["g"], un, far, [h0, h1])
    o0, o1 = un["out"].double(), c["out"]["out"].double()
    assert float((o1 - o0).norm() / o0.norm()) <= 1e-4


# ------------------------------------------------------------ edge cases --

def _edge_inputs(M, H, F, E, k, S=1, dtype="bf16", seed=7, bias=None, base=0, local=0):
    cfg = moe_synth.Config("edge", M, H, F, E, k, S, dtype, seed, 0.0, (M // S) if S > 1 else 0, base, local)
    d = moe_synth.make_inputs(cfg)
    if bias is not None:
        d["logits"] = (d["logits"] + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    return cfg, d


EDGE = {
    "M1": dict(M=1, H=128, F=192, E=8, k=2),
    "ragged_M300": dict(M=300, H=256, F=320, E=4, k=2),
    "E1_k1": dict(M=70, H=64, F=128, E=1, k=1),
    "k_equals_E": dict(M=90, H=128, F=128, E=4, k=4),
    "empty_experts": dict(M=200, H=128, F=256, E=8, k=2, bias=[5, 5, 5, -50, -50, -50, -50, -50]),
    "one_hot_expert": dict(M=600, H=192, F=256, E=8, k=1, bias=[0, 0, 0, 100, 0, 0, 0, 0]),
    "src_blocks_empty_segment": dict(M=256, H=128, F=128, E=4, k=2, S=8, bias=[0, 0, 0, -60]),
    "f32_ragged": dict(M=77, H=64, F=192, E=5, k=3, dtype="f32"),
    "k16_E64": dict(M=40, H=64, F=64, E=64, k=16),
    # one partial round of layer-1 tiles, split 8 ways along F (100 steps: uneven ranges)
    "split_single_round": dict(M=300, H=512, F=6400, E=4, k=2),
    # ... with empty experts and ragged segments (128 steps)
    "split_empty_experts": dict(M=200, H=256, F=8192, E=8, k=2, bias=[4, 4, 0, 0, -50, -50, 0, -50]),
    # held experts (expert-parallel share): a middle group, the last group with source blocks,
    # one held expert, and a held group nothing is routed to
    "local_mid": dict(M=300, H=256, F=320, E=16, k=4, base=4, local=4),
    "local_last_src_blocks": dict(M=256, H=128, F=192, E=16, k=2, S=4, base=12, local=4),
    "local_one_expert_f32": dict(M=90, H=64, F=128, E=8, k=3, dtype="f32", base=5, local=1),
    "local_none_routed": dict(M=64, H=128, F=128, E=8, k=2, base=6, local=2,
                              bias=[0, 0, 0, 0, 0, 0, -60, -60]),
    # segments of 27 and 9 row tiles: the tile order cuts them into row
    # blocks of uneven height (6/7 rows); every output row still computed once
    "tall_segments": dict(M=9000, H=256, F=512, E=2, k=1, bias=[1, 0]),
    # the most segments a call may rank: 16 source blocks x 64 experts = 1024
    "max_segments": dict(M=2048, H=64, F=128, E=64, k=2, S=16),
    # ... and with held experts: 15 blocks x 68 held + the dropped pairs' = 1021
    "max_segments_held": dict(M=1920, H=64, F=128, E=128, k=4, S=15, base=30, local=68),
    # 1024 segments over 65536 pairs: too many chunk histograms for each dispatch
    # workgroup to sum, so a scan kernel turns them into bases first
    "scanned_bookkeeping": dict(M=16384, H=64, F=64, E=64, k=4, S=16),
}
SPLIT_EDGES = ["split_single_round", "split_empty_experts"]


@pytest.mark.parametrize("edge", list(EDGE))
def test_edge_case_full_parity(edge):
    kw = dict(EDGE[edge])
    bias = kw.pop("bias", None)
    cfg, d = _edge_inputs(**kw, bias=bias)
    g = upload(d)
    o = run_chain(cfg, g)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                         src_block=d["src_block"], expert_base=cfg.base, local_experts=cfg.local)
    for key in ("topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    assert np.max(np.abs(host(o["topk_w"]) - r["topk_w"])) <= 1e-6
    assert_written(o, cfg.M)
    # element-wise: every tile's rows and every token
    c = tp.oracle_case(edge, cfg, d, g, o, None, 3000 + len(edge))
    tp.check_ffn(c, o, "chain")
    tp.check_out(c, o, o["out"], "chain")
    out, _, status = run_layer(cfg, g)
    ref = o if layer_runs_chain(cfg) else run_chain(cfg, g, gemm_ws=False)
    assert status == 0 and torch.equal(out, ref["out"])


@pytest.mark.parametrize("n_mover", [0, 4])
@pytest.mark.parametrize("edge", [e for e in EDGE if EDGE[e].get("dtype", "bf16") == "bf16"])
def test_edge_case_fused_equals_chain(edge, n_mover):
    """The fused kernel forced on every bf16 edge case (slots of experts not
    held, k from 1 to 16, one token, empty experts and segments, 1024
    segments), its combine items in the shared queue and on 4 dedicated
    workgroups: bitwise the unsplit chain's output, which the case above
    pins to the oracle."""
    kw = dict(EDGE[edge])
    bias = kw.pop("bias", None)
    cfg, d = _edge_inputs(**kw, bias=bias)
    g = upload(d)
    print(f"[fused edge] {edge} n_mover={n_mover}", flush=True)
    out, _, status = run_layer(cfg, g, n_mover=n_mover, gather=1)
    assert status == 0
    assert torch.equal(out, run_chain(cfg, g, gemm_ws=False)["out"])


@pytest.mark.parametrize("edge", SPLIT_EDGES)
def test_split_path_runs_and_is_deterministic(edge):
    """These shapes take the layer-1 split (a grid of one partial round, long
    F): its Y differs in rounding from the unsplit GEMM (so the split ran),
    stays within f32 regrouping error of it, and repeats bit for bit."""
    kw = dict(EDGE[edge])
    bias = kw.pop("bias", None)
    cfg, d = _edge_inputs(**kw, bias=bias)
    g = upload(d)
    a, b = run_chain(cfg, g), run_chain(cfg, g)
    un = run_chain(cfg, g, gemm_ws=False)
    assert torch.equal(a["y"], b["y"]) and torch.equal(a["out"], b["out"])
    assert torch.equal(a["hact"].view(torch.int16), un["hact"].view(torch.int16))  # layer 0 never splits
    assert not torch.equal(a["y"], un["y"])
    y0, y1 = un["y"].double(), a["y"].double()
    assert float((y1 - y0).norm() / y0.norm()) <= 1e-5


def test_local_holders_sum_to_full_layer():
    """Four calls holding 4 of 16 experts each: the counts are the full
    layer's, block by block, and the partial outputs add up to the full
    layer's output (f32 regrouping of the k-term sums only)."""
    kw = dict(M=256, H=128, F=192, E=16, k=4, S=2)
    cfg, d = _edge_inputs(**kw, seed=19)
    full = run_chain(cfg, upload(d))
    total = torch.zeros_like(full["out"])
    for b in range(0, 16, 4):
        pc, pd = _edge_inputs(**kw, seed=19, base=b, local=4)
        assert np.array_equal(pd["x"], d["x"]) and np.array_equal(pd["w_gate"], d["w_gate"][b:b + 4])
        part = run_chain(pc, upload(pd))
        for s_ in range(2):
            assert torch.equal(part["counts"][s_ * 4:(s_ + 1) * 4], full["counts"][s_ * 16 + b:s_ * 16 + b + 4])
        total += part["out"]
        fused, _, st = run_layer(pc, upload(pd), n_mover=0)
        ref = run_chain(pc, upload(pd), gemm_ws=False)
        assert st == 0 and torch.equal(fused, ref["out"])
    assert float((total - full["out"]).norm() / full["out"].norm()) <= 1e-6


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_combine_epilogue_is_exact_cast_of_sum(dtype):
    """moe_combine_ex: out = cast(acc + residual) with one f32 add, checked
    bit for bit against the plain combine's f32 result plus the residual,
    cast by torch (round to nearest even); and against the oracle's
    epilogue within one bf16 step."""
    import combine_topk_gate_amd as moe
    cfg, d = _edge_inputs(M=300, H=256, F=320, E=8, k=2, dtype=dtype, seed=23)
    g = upload(d)
    o = run_chain(cfg, g)
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, cfg.dtype)
    act = torch.bfloat16 if dtype == "bf16" else torch.float32
    res = (torch.randn(cfg.M, cfg.H, generator=torch.Generator().manual_seed(5)) * 3).to(act).cuda()
    acc = o["out"]
    for out_dtype, tdt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        for residual in (res, None):
            out = torch.empty(cfg.M, cfg.H, dtype=tdt, device="cuda")
            moe.moe_combine_ex(p, o["y"], o["topk_w"], o["flat_to_sorted"], moe.epilogue(residual, out_dtype), out)
            torch.cuda.synchronize()
            want = (acc + residual.float() if residual is not None else acc).to(tdt)
            assert torch.equal(out.view(torch.int16) if tdt == torch.bfloat16 else out,
                               want.view(torch.int16) if tdt == torch.bfloat16 else want), (out_dtype, residual is None)
    # against the oracle: bf16 out within one bf16 step of the oracle's cast
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, residual=host(res)
                         if dtype == "f32" else res.view(torch.int16).cpu().numpy().view(np.uint16), out_dtype="bf16")
    out = torch.empty(cfg.M, cfg.H, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_ex(p, o["y"], o["topk_w"], o["flat_to_sorted"], moe.epilogue(res, "bf16"), out)
    torch.cuda.synchronize()
    got = host(out)
    step = 2.0 ** -7 * np.maximum(np.abs(r["out"]), 2.0 ** -126)
    assert np.all(np.abs(got - r["out"]) <= step + 2e-2)
    assert rel_fro(got, r["out"]) <= 5e-3


def test_layer_ex_fused_equals_chain_with_epilogue():
    import combine_topk_gate_amd as moe
    cfg, d = _edge_inputs(M=512, H=256, F=512, E=8, k=2, seed=29)
    g = upload(d)
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k)
    res = torch.randn(cfg.M, cfg.H, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16).cuda()
    ws = torch.empty(moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER), dtype=torch.uint8, device="cuda")
    outs = []
    for fused, n_mover in ((1, 0), (1, 4), (0, -1)):
        out = torch.empty(cfg.M, cfg.H, dtype=torch.bfloat16, device="cuda")
        moe.moe_layer_ex(p, g["x"], g["logits"], None, g["w_gate"], g["w_up"], g["w_down"],
                         moe.epilogue(res, "bf16"), out, ws, n_mover=n_mover, fused=fused)
        torch.cuda.synchronize()
        outs.append(out.view(torch.int16).clone())
    # the chain's GEMM splits its last round, the fused kernel never does: compare
    # the fused schedules bitwise, and both against the plain combine + cast
    assert torch.equal(outs[0], outs[1])
    plain = run_chain(cfg, g, gemm_ws=False)
    want = (plain["out"] + res.float()).to(torch.bfloat16).view(torch.int16)
    assert torch.equal(outs[0], want)
    chain = run_chain(cfg, g)
    assert torch.equal(outs[2], (chain["out"] + res.float()).to(torch.bfloat16).view(torch.int16))


def test_zero_tokens_is_a_no_op():
    cfg, d = _edge_inputs(M=0, H=64, F=64, E=4, k=2)
    g = upload(d)
    out, _, status = run_layer(cfg, g, aux=False)
    assert status == 0 and out.numel() == 0


def test_route_crafted_ties():
    import combine_topk_gate_amd as moe
    M, E, k = 64, 16, 4
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((M, E)).astype(np.float32)
    lg[0, :] = 1.0
    lg[1, :] = -0.0
    lg[1, 1::2] = 0.0
    lg[2, 8:] = lg[2, :8]
    lg[3] = np.round(lg[3])
    p = moe.problem(M, 64, 64, E, k)
    idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    moe.moe_route(p, dev(lg), idx, w)
    torch.cuda.synchronize()
    ridx, rw = oracle.route(lg, k)
    assert np.array_equal(host(idx), ridx)
    assert list(host(idx)[0]) == [0, 1, 2, 3]
    assert np.max(np.abs(host(w) - rw)) <= 1e-6
