"""GPU parity of the MXFP8 activation path (dtype bf16_mxfp8): the MXFP8
quantiser bit for bit, and the layer with Hact and W_down in MXFP8 against
the oracle's MXFP8 path.

Tolerances.  The weights' codes are decided on the same bf16 values on both
sides, so they must match bit for bit.  Hact's codes are decided on the f32
value silu(g) * u, which the GPU accumulates in a different order from the
oracle's (f64, then rounded to f32): where that value sits at a rounding
boundary the two codes (or, where the block maximum sits at a power of two,
the two scales) differ by one step, so each dequantised element must lie
within one e4m3 step of the larger of the two block scales (2^-3 of the
magnitude, or 2^(X-9) in the subnormal range), and at least 99.9% of them
must be equal.  Rows covering every tile of both GEMMs (a row in every
128-row half of every 256-row tile of every segment, from the oracle's own
offsets) and every pair of a token sample are compared.  Y is checked
element by element: against the oracle's Y it may differ by the sum over f
of |Hact_gpu - Hact_oracle| |W_down| (the flipped codes, both dequantised)
plus 2^-13 of the sum of |terms| (the fp8 matrix cores' accumulation of
exact scaled products, a measured model: see parity_bounds.ACC_ULPS_FP8);
the combine then as in the bf16 path; and relative Frobenius 5e-3 on Y and out as a whole.  The distance
to the bf16 layer is printed: it is what MXFP8 costs, not a parity bound.
"""
import numpy as np
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
import oracle
import parity_bounds as pb
from moe_gpu_util import host, rel_fro, run_layer, upload

pytestmark = pytest.mark.gpu


def _bytes_to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def test_quantizer_bit_exact_against_oracle():
    rng = np.random.default_rng(201)
    rows, cols = 100, 256                        # a partial last group of 32 rows
    v = (rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-10, 10, (rows, 1)))).astype(np.float32)
    v[3] = 0.0                                   # all-zero rows
    v[5, :32] = 448.0                            # exact maximum
    v[7, :32] = 1e-40                            # below the smallest normal f32
    v[9, ::2] = -v[9, 1::2]                      # signs
    pos = np.array([oracle.e4m3_value(c) for c in range(127)])
    v[11, :126] = ((pos[:-1] + pos[1:]) / 2)[:126] * 2.0 ** -5  # ties after the block scale
    for src in (v, moe_synth.to_bf16_bits(v)):
        want = oracle.mx_quantize(src)
        t = torch.from_numpy(src.view(np.int16)).cuda().view(torch.bfloat16) if src.dtype == np.uint16 else \
            torch.from_numpy(src).cuda()
        dst = torch.empty(moe.mx_bytes(rows, cols), dtype=torch.uint8, device="cuda")
        moe.moe_quantize_mxfp8(t, dst)
        torch.cuda.synchronize()
        got = dst.cpu().numpy()
        assert np.array_equal(got, want), np.nonzero(got != want)[0][:10]


def run_chain_mx(cfg, g, wd_mx):
    """route -> dispatch -> layer 0 (Hact MXFP8) -> layer 1 (MXFP8) -> combine."""
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, "bf16_mxfp8", cfg.base, cfg.local)
    M, k, H, F, G, R = cfg.M, cfg.k, cfg.H, cfg.F, cfg.S * cfg.EL, cfg.M * cfg.k
    dev = "cuda"
    o = dict(topk_idx=torch.empty((M, k), dtype=torch.int32, device=dev),
             topk_w=torch.empty((M, k), dtype=torch.float32, device=dev),
             counts=torch.empty(G, dtype=torch.int32, device=dev),
             offsets=torch.empty(G + 1, dtype=torch.int32, device=dev),
             sorted_to_flat=torch.empty(R, dtype=torch.int32, device=dev),
             flat_to_sorted=torch.empty(R, dtype=torch.int32, device=dev),
             x_perm=torch.full((R, H), float("nan"), dtype=torch.bfloat16, device=dev),
             hact=torch.full((moe.mx_bytes(R, F),), 0x7F, dtype=torch.uint8, device=dev),  # e4m3 NaN codes
             y=torch.full((R, H), float("nan"), dtype=torch.float32, device=dev),
             out=torch.full((M, H), float("nan"), dtype=torch.float32, device=dev))
    ws = torch.empty(max(moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH), 4), dtype=torch.uint8, device=dev)
    assert moe.moe_workspace_bytes(p, moe.MOE_OP_GROUPED_GEMM) == 0
    moe.moe_route(p, g["logits"], o["topk_idx"], o["topk_w"])
    moe.moe_dispatch(p, g["x"], o["topk_idx"], g.get("src_block"), o["counts"], o["offsets"], o["sorted_to_flat"],
                     o["flat_to_sorted"], o["x_perm"], ws)
    moe.moe_grouped_gemm(p, 0, o["x_perm"], g["w_gate"], g["w_up"], o["offsets"], o["hact"])
    moe.moe_grouped_gemm(p, 1, o["hact"], wd_mx, None, o["offsets"], o["y"])
    moe.moe_combine(p, o["y"], o["topk_w"], o["flat_to_sorted"], o["out"])
    torch.cuda.synchronize()
    return p, o


E4M3 = np.array([oracle.e4m3_value(c) for c in range(256)])


def _values(codes, scales):
    """Values of MXFP8 codes [n, F] with their scale bytes [n, F/32]."""
    return E4M3[codes] * np.repeat(2.0 ** (scales.astype(np.int64) - 127), 32, axis=1)


def _hact_rows(buf, R, F, rows):
    """Dequantised values and block exponents of the given rows of an MXFP8
    Hact buffer (numpy uint8)."""
    codes = buf[:R * F].reshape(R, F)[rows]
    scales = oracle.mx_scales(buf, R, F)[rows]
    return _values(codes, scales), scales.astype(np.int64) - 127


CASES = {
    "small": (moe_synth.Config("mx_small", 300, 256, 384, 8, 2, 1, "bf16_mxfp8", 211), None),
    "qwen2": (moe_synth.config("qwen2", dtype="bf16_mxfp8"), 48),
    "mixtral": (moe_synth.config("mixtral", dtype="bf16_mxfp8"), 16),
    "held": (moe_synth.Config("mx_held", 256, 128, 256, 16, 4, 2, "bf16_mxfp8", 213, 0.0, 128, 4, 4), None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_mx_layer_parity(name):
    cfg, n_sample = CASES[name]
    _check_mx_layer(name, cfg, n_sample, 0.999)


def _random_mx_shape(i):
    rng = np.random.default_rng(9100 + i)
    E = int(rng.choice([2, 4, 8, 16, 32]))
    k = int(rng.integers(1, min(E, 6) + 1))
    S = int(rng.choice([1, 2, 4]))
    M = int(rng.integers(S, 700))
    H = 64 * int(rng.integers(1, 7))
    F = 128 * int(rng.integers(1, 5))
    block = -(-M // S) if S > 1 else 0
    base, local = 0, 0
    if i % 3 == 2:  # held experts: a middle group
        local = int(rng.integers(1, E)) if E > 1 else 0
        base = int(rng.integers(0, E - local + 1)) if local else 0
    return moe_synth.Config(f"mx_rand{i}", M, H, F, E, k, S, "bf16_mxfp8", 9300 + i, 0.0, block, base, local)


@pytest.mark.parametrize("i", range(6))
def test_mx_random_shape_parity(i):
    # small layers: a few elements at a rounding boundary are a larger share
    _check_mx_layer(f"random {i}", _random_mx_shape(i), None, 0.99)


def _check_mx_layer(name, cfg, n_sample, min_equal):
    print(f"[mx] {name} {cfg}", flush=True)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    EL, H, F = cfg.EL, cfg.H, cfg.F
    wd_mx_ref = oracle.mx_quantize(d["w_down"].reshape(EL * H, F))
    wd_mx = torch.empty(moe.mx_bytes(EL * H, F), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(g["w_down"], wd_mx)
    torch.cuda.synchronize()
    assert np.array_equal(wd_mx.cpu().numpy(), wd_mx_ref)
    print(f"[mx] {name}: W_down quantised, bit-exact", flush=True)
    p, o = run_chain_mx(cfg, g, wd_mx)
    toks = None if n_sample is None else moe_synth.token_sample(cfg, n_sample)
    ref = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                           src_block=d["src_block"], tokens=toks, want_rows=True, expert_base=cfg.base,
                           local_experts=cfg.local, w_down_mx=wd_mx_ref)
    for key in ("topk_idx", "counts", "offsets", "sorted_to_flat", "flat_to_sorted"):
        assert np.array_equal(host(o[key]), ref[key]), key
    R = cfg.M * cfg.k
    n = int(ref["offsets"][-1])
    assert bool(torch.isfinite(o["y"][:n]).all())
    # rows covering every tile (from the oracle's own offsets) and the token sample's rows
    cov_rows, tiles, halves = pb.covering_rows(ref["offsets"], cfg.seed + 77)
    hc, yc = oracle.ffn_rows(d["x"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, cfg.S, ref["sorted_to_flat"],
                             ref["offsets"], cov_rows, w_down_mx=wd_mx_ref)
    print(f"[mx] {name}: oracle done; {len(cov_rows)} covering rows over {tiles} row tiles ({halves} halves)",
          flush=True)
    tk = np.arange(cfg.M) if toks is None else toks
    flat = (tk[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    srows = ref["flat_to_sorted"][flat].astype(np.int64)
    kept = srows >= 0
    rows = np.concatenate([cov_rows, srows[kept]])
    rv = np.concatenate([hc, ref["hact"][kept]])
    ry = np.concatenate([yc, ref["y"][kept]])
    # Hact: within one e4m3 step of the larger block scale
    hv, hx = _hact_rows(o["hact"].cpu().numpy(), R, F, rows)
    rx = np.zeros_like(hx)
    for i in range(rv.shape[0]):
        q = oracle.mx_quantize(rv[i:i + 1])
        rx[i] = oracle.mx_scales(q, 1, F)[0].astype(np.int64) - 127
    X = np.repeat(np.maximum(hx, rx), 32, axis=1)
    step = np.maximum(np.maximum(np.abs(hv), np.abs(rv)) * 2.0 ** -3, 2.0 ** (X - 9))
    same = np.mean(hv == rv)
    print(f"[mx] {name}: Hact equal values {same:.5f}, max |d|/step {np.max(np.abs(hv - rv) / step):.3f}")
    assert np.all(np.abs(hv - rv) <= step * (1 + 1e-12))
    assert same >= min_equal
    # Y element by element: the GPU's own (dequantised) Hact against the
    # oracle's through the dequantised W_down, plus the f32 accumulation
    experts = pb.experts_of(ref["offsets"], rows, EL)
    w_scales = oracle.mx_scales(wd_mx_ref, EL * H, F)

    def w_of(e):
        return torch.from_numpy(_values(wd_mx_ref[e * H * F:(e + 1) * H * F].reshape(H, F),
                                        w_scales[e * H:(e + 1) * H])).cuda()

    y_allow = pb.y_allowance(torch.from_numpy(hv).cuda(), torch.from_numpy(rv).cuda(), experts, w_of, H,
                             acc_ulps=pb.ACC_ULPS_FP8)
    yg = host(o["y"][torch.from_numpy(rows).cuda()])
    pb.check_within(f"mx {name} Y", yg, ry, y_allow.cpu().numpy())
    ey = rel_fro(yg, ry)
    # the combine on the token sample, element by element
    n_t = len(tk)
    yb = np.zeros((n_t * cfg.k, H))
    ygs = np.zeros((n_t * cfg.k, H))
    ns = len(cov_rows)
    yb[kept] = y_allow[ns:].cpu().numpy()
    ygs[kept] = yg[ns:]
    tkd = torch.from_numpy(tk).cuda()
    og = host(o["out"][tkd])
    allow = pb.out_allowance(host(o["topk_w"][tkd]), ref["topk_w"][tk], ygs, ref["y"], yb, kept.reshape(n_t, cfg.k))
    pb.check_within(f"mx {name} out", og, ref["out"], allow)
    eo = rel_fro(og, ref["out"])
    bf = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                          src_block=d["src_block"], tokens=toks, expert_base=cfg.base, local_experts=cfg.local)
    print(f"[mx] {name}: Y relF {ey:.3e}, out relF {eo:.3e}; distance to the bf16 layer "
          f"{rel_fro(og, bf['out']):.3e}")
    assert ey <= 5e-3 and eo <= 5e-3
    assert rel_fro(og, bf["out"]) <= 0.1  # MXFP8's own error, a sanity bound only
    # moe_layer runs this dtype as the same chain
    out, _, st = run_layer(cfg, dict(g, w_down=wd_mx))
    assert st == 0 and torch.equal(out, o["out"])


def test_mx_combine_epilogue_reads_a_bf16_residual():
    """The residual of an MXFP8 layer is in x's dtype (bf16): the epilogue
    equals the f32 combine plus the residual, cast by torch, bit for bit."""
    cfg = moe_synth.Config("mx_epi", 256, 256, 256, 8, 2, 1, "bf16_mxfp8", 215)
    d = moe_synth.make_inputs(cfg)
    g = upload(d)
    wd_mx = torch.empty(moe.mx_bytes(cfg.E * cfg.H, cfg.F), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_mxfp8(g["w_down"], wd_mx)
    p, o = run_chain_mx(cfg, g, wd_mx)
    res = torch.randn(cfg.M, cfg.H, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16).cuda()
    out = torch.empty(cfg.M, cfg.H, dtype=torch.bfloat16, device="cuda")
    moe.moe_combine_ex(p, o["y"], o["topk_w"], o["flat_to_sorted"], moe.epilogue(res, "bf16"), out)
    torch.cuda.synchronize()
    want = (o["out"] + res.float()).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
