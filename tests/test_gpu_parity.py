"""GPU parity: every C-ABI call against the CPU oracle on the same seeded
inputs (needs an MI355X and the built library).

Routing indices, counts, offsets and the permutation are compared in full
and must be bit-exact; the dispatch copy must be bitwise; the top-k weights
within 1e-6 absolute; Hact within one bf16 rounding step of the oracle's
(both round the same f32/f64 value to bf16, so they differ only where the
value sits at a rounding boundary); Y and the layer output within relative
Frobenius 5e-3 and max abs 2e-2 (bf16 layers, f32 accumulation) or 1e-5
relative (f32 layer).  Large layers compare the FFN outputs on a seeded
sample of tokens (all k rows of each), spread over every source block.
"""
import gc

import numpy as np
import pytest
import torch

import moe_synth
import oracle
from moe_gpu_util import dev, host, rel_fro, run_chain, run_layer, tolerances, upload

pytestmark = pytest.mark.gpu

SAMPLE = {"tiny": None, "qwen2": 64, "mixtral": 24, "phi35": 24, "epshare": 16}

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
    ref = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                           src_block=d["src_block"], tokens=toks, want_rows=True)
    return dict(name=name, cfg=cfg, d=d, g=g, out=out, ref=ref, toks=toks)


def test_route_bit_exact(case):
    c = case
    assert np.array_equal(host(c["out"]["topk_idx"]), c["ref"]["topk_idx"])
    assert np.max(np.abs(host(c["out"]["topk_w"]) - c["ref"]["topk_w"])) <= 1e-6


def test_dispatch_bit_exact(case):
    c = case
    o, r, cfg = c["out"], c["ref"], c["cfg"]
    for key in ("counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    # X_perm[r] is token s2f[r] // k, bit for bit (checked on the device in full)
    src = c["g"]["x"][(o["sorted_to_flat"].long() // cfg.k)]
    assert torch.equal(o["x_perm"].view(torch.int16) if cfg.dtype == "bf16" else o["x_perm"],
                       src.view(torch.int16) if cfg.dtype == "bf16" else src)


def _sample_rows(c):
    cfg, r = c["cfg"], c["ref"]
    toks = np.arange(cfg.M) if c["toks"] is None else c["toks"]
    flat = (toks[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    return r["flat_to_sorted"][flat].astype(np.int64), toks


def test_layer0_swiglu(case):
    c = case
    rows, _ = _sample_rows(c)
    got = host(c["out"]["hact"][torch.from_numpy(rows).cuda()])
    ref = c["ref"]["hact"]
    if c["cfg"].dtype == "bf16":
        # Both sides round silu(g)*u to bf16: one rounding step (2^-8 relative,
        # 2^-7 across a binade edge) where the f32-accumulated g, u fall on the
        # other side of a rounding boundary, plus the f32 accumulation error
        # itself, which only shows where h is near zero (|dg| ~ 1e-6 for
        # K <= 7168 products of N(0,1) x N(0,0.02^2) terms; bound 5e-5).
        dev_ = np.abs(got - ref)
        excess = dev_ - 2.0 ** -7 * np.abs(ref)
        print(f"[parity] {c['name']}: hact max|d| {dev_.max():.3e}, max excess over 1 ulp {excess.max():.3e}, "
              f"relF {rel_fro(got, ref):.3e}")
        assert np.all(excess <= 5e-5)
        assert rel_fro(got, ref) <= 1e-3
    else:
        assert rel_fro(got, ref) <= 1e-5


def test_layer1_down(case):
    c = case
    rows, _ = _sample_rows(c)
    got = host(c["out"]["y"][torch.from_numpy(rows).cuda()])
    rel, mabs = tolerances(c["cfg"])
    assert rel_fro(got, c["ref"]["y"]) <= rel
    if mabs is not None:
        assert np.max(np.abs(got - c["ref"]["y"])) <= mabs


def test_combine_output(case):
    c = case
    _, toks = _sample_rows(c)
    got = host(c["out"]["out"][torch.from_numpy(toks).cuda()])
    rel, mabs = tolerances(c["cfg"])
    err = rel_fro(got, c["ref"]["out"])
    print(f"[parity] {c['name']}: out relF {err:.3e} maxabs {np.max(np.abs(got - c['ref']['out'])):.3e}")
    assert err <= rel
    if mabs is not None:
        assert np.max(np.abs(got - c["ref"]["out"])) <= mabs


def test_layer_equals_chain_bitwise(case):
    c = case
    out, _, status = run_layer(c["cfg"], c["g"])
    assert status == 0
    assert torch.equal(out, c["out"]["out"])


# ------------------------------------------------------------ edge cases --

def _edge_inputs(M, H, F, E, k, S=1, dtype="bf16", seed=7, bias=None):
    cfg = moe_synth.Config("edge", M, H, F, E, k, S, dtype, seed, 0.0, (M // S) if S > 1 else 0)
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
}


@pytest.mark.parametrize("edge", list(EDGE))
def test_edge_case_full_parity(edge):
    kw = dict(EDGE[edge])
    bias = kw.pop("bias", None)
    cfg, d = _edge_inputs(**kw, bias=bias)
    g = upload(d)
    o = run_chain(cfg, g)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                         src_block=d["src_block"])
    for key in ("topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), r[key]), key
    assert np.max(np.abs(host(o["topk_w"]) - r["topk_w"])) <= 1e-6
    rel, mabs = tolerances(cfg)
    assert rel_fro(host(o["out"]), r["out"]) <= rel
    if mabs is not None:
        assert np.max(np.abs(host(o["out"]) - r["out"])) <= mabs
    out, _, status = run_layer(cfg, g)
    assert status == 0 and torch.equal(out, o["out"])


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
