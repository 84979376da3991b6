"""Pins of the CPU oracle against things other than itself (CPU only).

Each test checks the oracle against a brute-force or closed-form construction
that does not share its code path: a Python sort for the routing, a numpy
stable ordering for the permutation, a dense evaluation of every expert on
every token for the layer, torch's bf16 conversion for the rounding, and
exact algebraic identities (scaling, zero input, token permutation, expert
relabelling).  A plausible slip in the oracle -- a dropped term, a flipped
tie rule, a transposed weight, a wrong index into the permutation -- breaks
at least one of these.
"""
import math

import numpy as np
import pytest
import torch

import moe_synth
import oracle

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


# ----------------------------------------------------------------- helpers --

def brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def small_inputs(M, H, F, E, k, dtype, seed, S=1):
    cfg = moe_synth.Config("pin", M, H, F, E, k, S, dtype, seed, 0.0, (M // S) if S > 1 else 0)
    d = moe_synth.make_inputs(cfg)
    return cfg, d


def widen(a):
    return moe_synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


def dense_layer(x, logits, wg, wu, wd, k, bf16, base=0):
    """Every expert on every token, then the top-k mask and weights.

    Independent of the oracle's routing / permutation / combine: experts are
    chosen by argsort, weights by the full softmax renormalised over the
    selected experts, and the FFN runs as dense numpy matmuls.  The weights
    may hold experts base .. base + len(wg) - 1 of the logits' experts only:
    then only those experts' terms are summed."""
    X = widen(x)
    L = logits.astype(np.float64)
    M, E = L.shape
    Wg, Wu, Wd = widen(wg), widen(wu), widen(wd)  # [EL,F,H], [EL,F,H], [EL,H,F]
    out = np.zeros((M, X.shape[1]))
    # selection: stable argsort of -logit gives ties to the lower index
    order = np.argsort(-L, axis=1, kind="stable")[:, :k]
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    for e in range(base, base + Wg.shape[0]):
        G = X @ Wg[e - base].T
        U = X @ Wu[e - base].T
        Hh = G / (1.0 + np.exp(-G)) * U
        if bf16:
            Hh = np.vectorize(oracle.round_to_bf16)(Hh)
        Y = Hh @ Wd[e - base].T
        sel = (order == e)
        mask = sel.any(axis=1)
        w = np.where(mask, p[:, e] / np.take_along_axis(p, order, axis=1).sum(axis=1), 0.0)
        # the combine consumes the stored f32 weights
        w = w.astype(np.float32).astype(np.float64)
        out += w[:, None] * Y
    return out, order


# -------------------------------------------------------------- bf16 pin --

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # exact halfway cases: bf16 value + half a bf16 ulp (representable in f32)
    base = moe_synth.bf16_bits_to_f32(rng.integers(0x0080, 0x7F00, size=2000, dtype=np.uint16))
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    vals = np.concatenate([vals, half, -half, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875])])
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_to_bf16(float(v)) for v in vals])
    assert np.array_equal(got, want)


# ------------------------------------------------------------- routing --

@pytest.mark.parametrize("E,k", [(1, 1), (2, 1), (2, 2), (8, 2), (16, 8), (64, 4), (64, 64), (512, 16)])
def test_route_matches_python_sort(E, k):
    rng = np.random.default_rng(E * 100 + k)
    M = 97
    logits = rng.standard_normal((M, E)).astype(np.float32)
    # plant ties: duplicated values, all-equal rows, signed zeros
    logits[3, :] = 0.5
    logits[5, : E // 2] = logits[5, E // 2 : 2 * (E // 2)]
    logits[7, :] = -0.0
    logits[7, ::2] = 0.0
    logits[11] = np.round(logits[11] * 2) / 2
    idx, w = oracle.route(logits, k)
    for t in range(M):
        assert list(idx[t]) == brute_topk(logits[t], k), t
    assert list(idx[3]) == list(range(k))  # all-equal row: lowest indices in order
    assert list(idx[7]) == list(range(k))  # +0.0 and -0.0 tie
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 4 * 2.0 ** -24 * k)


def test_route_weights_closed_form_k2():
    rng = np.random.default_rng(3)
    logits = (rng.standard_normal((500, 8)) * 3).astype(np.float32)
    idx, w = oracle.route(logits, 2)
    l0 = np.take_along_axis(logits, idx[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, idx[:, 1:2], 1)[:, 0].astype(np.float64)
    w0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.all(np.abs(w[:, 0] - w0) <= 2.0 ** -24)
    assert np.all(np.abs(w[:, 1] - (1.0 - w0)) <= 2.0 ** -24)


def test_route_weights_full_softmax_renormalised():
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((300, 64)).astype(np.float32)
    idx, w = oracle.route(logits, 4)
    p = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    ps = np.take_along_axis(p, idx.astype(np.int64), 1)
    want = ps / ps.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - want)) <= 1e-7


def test_route_k1_weight_is_exactly_one():
    logits = np.random.default_rng(5).standard_normal((64, 16)).astype(np.float32)
    idx, w = oracle.route(logits, 1)
    assert np.all(w == 1.0)
    assert np.array_equal(idx[:, 0], np.argmax(logits, axis=1))


# ---------------------------------------------- counts / offsets / permute --

@pytest.mark.parametrize("M,E,k,S", [(1, 1, 1, 1), (37, 8, 2, 1), (200, 64, 4, 1), (96, 16, 8, 8), (50, 4, 4, 2),
                                     (0, 8, 2, 1)])
def test_segments_and_permutation_brute_force(M, E, k, S):
    rng = np.random.default_rng(M * 7 + E)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    if M > 4:
        logits[: M // 3, 0] += 10.0  # crowd expert 0, leave others light / empty
    idx, _ = oracle.route(logits, k)
    src = None if S == 1 else (np.arange(M) * S // max(M, 1)).astype(np.int32)
    counts, offsets = oracle.counts_offsets(idx, E, S, src)
    s2f, f2s = oracle.permutation(idx, E, S, src)
    R = M * k
    seg = [(0 if src is None else int(src[f // k])) * E + int(idx.reshape(-1)[f]) for f in range(R)]
    # brute force: python stable sort of the flat indices by segment
    want = sorted(range(R), key=lambda f: (seg[f], f))
    assert list(s2f) == want
    assert counts.sum() == R
    assert np.array_equal(counts, np.bincount(np.array(seg, dtype=np.int64), minlength=S * E)[: S * E])
    assert offsets[0] == 0 and offsets[-1] == R and np.all(np.diff(offsets) == counts)
    assert sorted(s2f.tolist()) == list(range(R))  # bijection
    assert np.array_equal(f2s[s2f], np.arange(R))
    for g in range(S * E):  # stable inside every segment, and in the right segment
        part = s2f[offsets[g]:offsets[g + 1]]
        assert np.all(np.diff(part) > 0)
        assert all(seg[f] == g for f in part)


def test_dispatch_is_bitwise_row_copy():
    cfg, d = small_inputs(40, 64, 64, 8, 2, "bf16", 11)
    idx, _ = oracle.route(d["logits"], cfg.k)
    s2f, _ = oracle.permutation(idx, cfg.E)
    xp = oracle.dispatch(d["x"], cfg.k, s2f)
    assert np.array_equal(xp, d["x"][s2f // cfg.k])


@pytest.mark.parametrize("dtype,base,EL,S", [("bf16", 4, 4, 1), ("f32", 0, 1, 2), ("bf16", 6, 2, 4)])
def test_dispatch_with_held_experts_zero_fills_past_kept_pairs(dtype, base, EL, S):
    """With held experts the sorted positions past the kept pairs hold no
    pair (-1): their X_perm rows are zero, every kept row is its token's row
    bit for bit (numpy fancy indexing, not the oracle's loop)."""
    cfg, d = small_inputs(48, 64, 64, 8, 2, dtype, 17 + base, S=S)
    idx, _ = oracle.route(d["logits"], cfg.k)
    s2f, _ = oracle.permutation(idx, cfg.E, S, d["src_block"], base, EL)
    kept = int(np.isin(idx, np.arange(base, base + EL)).sum())
    assert 0 < kept < cfg.M * cfg.k
    assert np.all(s2f[:kept] >= 0) and np.all(s2f[kept:] == -1)
    # a stale buffer (all bits set) must come back with zero rows past the kept pairs
    stale = np.empty((cfg.M * cfg.k, cfg.H), dtype=d["x"].dtype)
    stale.view(np.uint8)[:] = 0xFF
    xp = oracle.dispatch(d["x"], cfg.k, s2f, out=stale)
    assert xp is stale
    assert np.array_equal(xp[:kept], d["x"][s2f[:kept] // cfg.k])
    assert not np.any(xp[kept:])


def test_route_rejects_more_experts_than_its_selection_arrays():
    with pytest.raises(ValueError):
        oracle.route(np.zeros((2, 1025), np.float32), 2)
    idx, w = oracle.route(np.zeros((2, 1024), np.float32), 3)
    assert idx.tolist() == [[0, 1, 2], [0, 1, 2]]


# ------------------------------------------------------------------ layer --

@pytest.mark.parametrize("dtype,E,k", [("f32", 4, 2), ("f32", 8, 8), ("bf16", 4, 2), ("bf16", 6, 3), ("f32", 1, 1)])
def test_layer_matches_dense_brute_force(dtype, E, k):
    cfg, d = small_inputs(48, 64, 96, E, k, dtype, 21 + E + k)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], k)
    dense, order = dense_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], k, dtype == "bf16")
    assert np.array_equal(r["topk_idx"], order)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-9, atol=1e-12)


def test_layer_with_source_blocks_matches_dense():
    cfg, d = small_inputs(64, 64, 64, 4, 2, "bf16", 33, S=4)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, S=4, src_block=d["src_block"])
    dense, _ = dense_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, True)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-9, atol=1e-12)
    assert r["counts"].sum() == 128 and r["offsets"][-1] == 128


def test_top1_single_expert_is_one_dense_swiglu_ffn():
    cfg, d = small_inputs(32, 64, 128, 1, 1, "f32", 41)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 1)
    assert np.all(r["topk_w"] == 1.0)
    X = torch.from_numpy(d["x"]).double()
    g = torch.matmul(X, torch.from_numpy(d["w_gate"][0]).double().T)
    u = torch.matmul(X, torch.from_numpy(d["w_up"][0]).double().T)
    y = torch.matmul(torch.nn.functional.silu(g) * u, torch.from_numpy(d["w_down"][0]).double().T)
    np.testing.assert_allclose(r["out"], y.numpy(), rtol=1e-10, atol=1e-13)


def test_token_subset_equals_full_layer_rows():
    cfg, d = small_inputs(64, 64, 64, 8, 2, "bf16", 51)
    full = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, want_rows=True)
    toks = np.array([0, 5, 17, 63])
    sub = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, tokens=toks, want_rows=True)
    assert np.array_equal(sub["out"], full["out"][toks])
    rows = (toks[:, None] * 2 + np.arange(2)).reshape(-1)
    assert np.array_equal(sub["y"], full["y"][rows])


# ----------------------------------------------------------- equivariances --

def _layer(d, k, **kw):
    return oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], k, **kw)["out"]


def test_scaling_w_down_by_two_doubles_output_exactly():
    cfg, d = small_inputs(32, 64, 64, 4, 2, "f32", 61)
    base = _layer(d, 2)
    d2 = dict(d, w_down=d["w_down"] * np.float32(2.0))
    assert np.array_equal(_layer(d2, 2), 2.0 * base)


def test_zero_input_gives_zero_output():
    cfg, d = small_inputs(16, 64, 64, 4, 2, "bf16", 62)
    d0 = dict(d, x=np.zeros_like(d["x"]))
    assert np.all(_layer(d0, 2) == 0.0)


def test_permuting_tokens_permutes_outputs():
    cfg, d = small_inputs(40, 64, 64, 8, 2, "bf16", 63)
    base = _layer(d, 2)
    perm = np.random.default_rng(1).permutation(40)
    dp = dict(d, x=d["x"][perm], logits=d["logits"][perm])
    assert np.array_equal(_layer(dp, 2), base[perm])


def test_relabelling_experts_leaves_output_unchanged():
    cfg, d = small_inputs(40, 64, 64, 8, 2, "f32", 64)
    base = _layer(d, 2)
    perm = np.random.default_rng(2).permutation(8)
    dp = dict(d, logits=d["logits"][:, perm], w_gate=d["w_gate"][perm], w_up=d["w_up"][perm],
              w_down=d["w_down"][perm])
    # N(0,1) f32 logits: ties have probability ~0, so the selected experts map one to one
    assert np.array_equal(_layer(dp, 2), base)


# ---------------------------------------------------------------- inputs --

@pytest.mark.parametrize("name", ["mixtral", "phi35"])
def test_stored_skew_scale_reproduces_target_std(name):
    cfg = moe_synth.CONFIGS[name]
    logits = moe_synth.make_logits(cfg)
    idx, _ = oracle.route(logits, cfg.k)
    counts, _ = oracle.counts_offsets(idx, cfg.E)
    frac = counts / float(cfg.M * cfg.k)
    assert abs(frac.std() - cfg.skew) <= 5e-4
    if name == "phi35":
        assert counts.min() < 500  # the lightest expert gets only a few hundred rows


def test_unskewed_configs_are_near_uniform():
    cfg = moe_synth.CONFIGS["qwen2"]
    idx, _ = oracle.route(moe_synth.make_logits(cfg), cfg.k)
    counts, _ = oracle.counts_offsets(idx, cfg.E)
    frac = counts / float(cfg.R)
    assert frac.std() < 0.25 / cfg.E


# ------------------------------------------------- local experts (EP share) --
# A call that holds experts [base, base + EL) of E keeps only the pairs routed
# to them (COMET review §4.1.2 dispatch by source and expert; the PTO MoE
# article's 16 local experts per card), and its combine is that holder's
# share of each token's sum.

@pytest.mark.parametrize("M,E,k,S,base,EL", [(60, 16, 4, 1, 4, 4), (96, 32, 8, 4, 0, 8), (50, 8, 2, 2, 6, 2),
                                             (40, 8, 2, 1, 0, 8), (33, 16, 2, 1, 15, 1), (0, 8, 2, 1, 2, 3)])
def test_local_segments_brute_force(M, E, k, S, base, EL):
    rng = np.random.default_rng(M * 13 + E + base)
    logits = rng.standard_normal((M, E)).astype(np.float32)
    idx, _ = oracle.route(logits, k)
    src = None if S == 1 else (np.arange(M) * S // max(M, 1)).astype(np.int32)
    counts, offsets = oracle.counts_offsets(idx, E, S, src, base, EL)
    s2f, f2s = oracle.permutation(idx, E, S, src, base, EL)
    R = M * k
    flat_e = idx.reshape(-1)
    kept = [f for f in range(R) if base <= flat_e[f] < base + EL]
    seg = {f: (0 if src is None else int(src[f // k])) * EL + int(flat_e[f]) - base for f in kept}
    want = sorted(kept, key=lambda f: (seg[f], f))
    n = len(want)
    assert counts.shape == (S * EL,) and offsets.shape == (S * EL + 1,)
    assert list(s2f[:n]) == want and np.all(s2f[n:] == -1)
    assert offsets[0] == 0 and offsets[-1] == n and np.all(np.diff(offsets) == counts)
    for f in range(R):
        assert f2s[f] == (want.index(f) if f in seg else -1)


def test_local_full_range_is_the_plain_layer():
    cfg, d = small_inputs(40, 64, 64, 8, 2, "bf16", 51, S=2)
    a = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, S=2, src_block=d["src_block"])
    b = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, S=2, src_block=d["src_block"],
                         expert_base=0, local_experts=8)
    for key in a:
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("dtype,E,k,base,EL", [("f32", 8, 2, 2, 3), ("bf16", 16, 4, 12, 4), ("bf16", 8, 8, 0, 1)])
def test_local_layer_matches_dense_partial(dtype, E, k, base, EL):
    cfg, d = small_inputs(48, 64, 96, E, k, dtype, 61 + E + base)
    sl = slice(base, base + EL)
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"][sl], d["w_up"][sl], d["w_down"][sl], k,
                         expert_base=base, local_experts=EL)
    dense, order = dense_layer(d["x"], d["logits"], d["w_gate"][sl], d["w_up"][sl], d["w_down"][sl], k,
                               dtype == "bf16", base=base)
    assert np.array_equal(r["topk_idx"], order)
    np.testing.assert_allclose(r["out"], dense, rtol=1e-9, atol=1e-12)


def test_local_partition_sums_to_full_layer():
    """Four holders of 4 experts each: their counts are the full counts,
    source block by source block, and their partial outputs add up to the
    full layer's output."""
    cfg, d = small_inputs(64, 64, 64, 16, 4, "bf16", 71, S=2)
    full = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 4, S=2,
                            src_block=d["src_block"])
    total = np.zeros_like(full["out"])
    for b in range(0, 16, 4):
        sl = slice(b, b + 4)
        part = oracle.moe_layer(d["x"], d["logits"], d["w_gate"][sl], d["w_up"][sl], d["w_down"][sl], 4, S=2,
                                src_block=d["src_block"], expert_base=b, local_experts=4)
        for s in range(2):
            assert np.array_equal(part["counts"][s * 4:(s + 1) * 4], full["counts"][s * 16 + b:s * 16 + b + 4])
        total += part["out"]
    np.testing.assert_allclose(total, full["out"], rtol=1e-12, atol=1e-13)


# -------------------------------------------------------------- epilogue --
# cast(acc + residual) (grouped-GEMM article, fused GemmAdd epilogue).

def test_epilogue_hand_values():
    b = lambda v: moe_synth.to_bf16_bits(np.float32([v]))  # noqa: E731  exact bf16 residuals
    # 1 + 2^-8 lies halfway between the bf16 values 1 and 1 + 2^-7: to even (1)
    assert oracle.epilogue(np.array([1.0]), b(2.0 ** -8), "bf16")[0] == 1.0
    # a little above halfway rounds up
    assert oracle.epilogue(np.array([1.0 + 2.0 ** -12]), b(2.0 ** -8), "bf16")[0] == 1.0 + 2.0 ** -7
    # 257 lies halfway between 256 and 258: to even (256); 259 -> 260
    assert oracle.epilogue(np.array([256.0]), b(1.0), "bf16")[0] == 256.0
    assert oracle.epilogue(np.array([256.0]), b(3.0), "bf16")[0] == 260.0
    # negative, f32 residual, f32 output: the plain sum
    assert oracle.epilogue(np.array([-2.5]), np.float32([0.25]), "f32")[0] == -2.25
    assert oracle.epilogue(np.array([0.1]), None, "f32")[0] == 0.1
    # 1 + 3 * 2^-9 is above halfway between 1 and 1 + 2^-7 -> up; -(that) -> down
    assert oracle.epilogue(np.array([1.0, -1.0]), np.float32([3 * 2.0 ** -9, -3 * 2.0 ** -9]), "bf16").tolist() == \
        [1.0 + 2.0 ** -7, -1.0 - 2.0 ** -7]


def test_epilogue_bf16_matches_torch_rounding_of_f32_sums():
    rng = np.random.default_rng(81)
    # both operands on the grid of 2^-12 with magnitude below 8: every sum
    # is a multiple of 2^-12 below 16, exact in f32, so torch rounds it once
    grid = lambda v: np.clip(np.round(v * 4096.0), -32000, 32000) / 4096.0  # noqa: E731
    acc = grid(rng.standard_normal(5000) * 2.0)
    res = moe_synth.to_bf16_bits(grid(rng.standard_normal(5000) * 2.0).astype(np.float32))
    res_v = moe_synth.bf16_bits_to_f32(res).astype(np.float64)
    got = oracle.epilogue(acc, res, "bf16")
    exact = acc + res_v
    assert np.array_equal(exact.astype(np.float32).astype(np.float64), exact)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)


def test_layer_epilogue_is_applied_to_the_combined_output():
    cfg, d = small_inputs(24, 64, 64, 4, 2, "bf16", 91)
    res = moe_synth.to_bf16_bits(np.random.default_rng(92).standard_normal((24, 64)).astype(np.float32))
    toks = np.array([3, 0, 17, 23])
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, tokens=toks, residual=res,
                         out_dtype="bf16")
    plain = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, tokens=toks)
    assert np.array_equal(r["acc"], plain["out"])
    want = torch.from_numpy((plain["out"] + widen(res)[toks]).astype(np.float32)).to(torch.bfloat16).double()
    # the f32 rounding of the sum is within half an f32 ulp: the bf16 results agree except at exact ties
    assert np.mean(r["out"] == want.numpy()) > 0.999


# ----------------------------------------------------------- MXFP8 (NEXT) --
# The activation quantised as SwiGLU produces it (PTO MoE article, two-stage
# SwiGLU) in the open OCP microscaling format MXFP8: e4m3 elements, one
# power-of-two scale per 32 values.

def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([oracle.e4m3_value(c) for c in codes])
    nan = (codes & 0x7F) == 0x7F
    assert np.all(np.isnan(got[nan])) and np.array_equal(got[~nan], want[~nan])


def test_e4m3_rounding_matches_torch_below_448():
    rng = np.random.default_rng(101)
    vals = np.concatenate([rng.standard_normal(4000) * 40, rng.standard_normal(2000) * 0.01,
                           rng.uniform(-448, 448, 2000)])
    # every midpoint between neighbouring codes (exact ties) and the codes themselves
    pos = np.array([oracle.e4m3_value(c) for c in range(127)])
    mids = (pos[:-1] + pos[1:]) / 2
    vals = np.concatenate([vals, mids, -mids, pos, -pos]).astype(np.float32)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_round(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_rounding_clamps_to_448():
    for v, c in [(448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (480.0, 0x7E), (1e9, 0x7E), (-500.0, 0xFE),
                 (0.0, 0x00), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02)]:
        assert oracle.e4m3_round(v) == c, (v, c)


def test_mx_block_hand_values():
    def q(block):
        # one row of 128 values: the block under test, then three zero blocks
        buf = oracle.mx_quantize(np.concatenate([np.asarray(block, np.float64), np.zeros(96)]).reshape(1, 128))
        assert np.all(buf[32:128] == 0) and buf.size == 128 + 32 * 4 and np.all(buf[129:] == 0)
        return buf[:32], int(buf[128])
    codes, s = q([1.0] * 32)            # floor(log2 1) - 8 = -8: 1 / 2^-8 = 256 = code 0x78
    assert s == 127 - 8 and np.all(codes == 0x78)
    codes, s = q([448.0] + [0.0] * 31)  # X = 0, 448 exact
    assert s == 127 and codes[0] == 0x7E and np.all(codes[1:] == 0)
    codes, s = q([500.0, -1.0] + [0.0] * 30)  # X = 0 (floor log2 500 = 8): 500 clamps to 448
    assert s == 127 and codes[0] == 0x7E and codes[1] == 0xB8
    codes, s = q([0.0] * 32)            # all zero: the smallest scale, zero codes
    assert s == 0 and np.all(codes == 0)
    codes, s = q([0.75] + [0.1] * 31)   # X = -1 - 8: 0.75 * 512 = 384 = 1.5 * 2^8 = 0x7C
    assert s == 127 - 9 and codes[0] == 0x7C
    assert abs(oracle.e4m3_value(codes[1]) * 2.0 ** -9 - 0.1) <= 0.1 * 2.0 ** -4


def test_mx_round_trip_within_half_a_step():
    rng = np.random.default_rng(103)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    buf = oracle.mx_quantize(v)
    d = oracle.mx_dequantize(buf, 64, 256)
    scales = oracle.mx_scales(buf, 64, 256).astype(np.int64)
    X = np.repeat(scales - 127, 32, axis=1)
    t = np.abs(v) / 2.0 ** X                      # magnitude in units of the block scale
    assert np.all(t.reshape(64, 8, 32).max(axis=2) >= 256) and np.all(t < 512)
    half = np.where(t >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(t, 2.0 ** -6))) - 4), 2.0 ** -10)
    err = np.abs(d - v) / 2.0 ** X
    clamped = t > 448
    assert np.all(err[~clamped] <= half[~clamped] * (1 + 1e-12))
    assert np.all(np.abs(d[clamped]) == 448 * 2.0 ** X[clamped])
    # values already on the grid come back exactly
    assert np.array_equal(oracle.mx_dequantize(oracle.mx_quantize(d), 64, 256), d)


def test_mx_scale_storage_layout():
    """The buffer format (a storage convention of the library, not of the
    format): codes row-major, then for each group of 32 rows (the last one
    padded with zero bytes) and each 128-column quad, the 4 scale bytes of
    each row in turn.  Every block here gets its own power of two, so its
    scale byte names it: block (r, b) holds 2^(r + 2b - 40) * 256."""
    rows, cols = 40, 256
    r_, b_ = np.meshgrid(np.arange(rows), np.arange(cols // 32), indexing="ij")
    X = r_ + 2 * b_ - 40
    v = np.repeat(2.0 ** X * 256, 32, axis=1)
    buf = oracle.mx_quantize(v)
    assert buf.size == rows * cols + 64 * 8        # two groups of 32 rows, 8 blocks each
    assert np.all(buf[:rows * cols] == 0x78)        # 256 in units of the scale = 1.0 * 2^8
    sc = buf[rows * cols:]
    for r in range(rows):
        for b in range(cols // 32):
            g, q = divmod(r, 32)[0], b // 4
            pos = (g * 2 + q) * 128 + (r % 32) * 4 + b % 4
            assert sc[pos] == 127 + X[r, b], (r, b)
    # padding rows 40..63 of the second group
    for q in range(2):
        blk = sc[(2 + q) * 128:(3 + q) * 128].reshape(32, 4)
        assert np.all(blk[8:] == 0)
    assert np.array_equal(oracle.mx_scales(buf, rows, cols), (127 + X).astype(np.uint8))


def test_mx_layer_matches_dense_quantised_evaluation():
    """The fp8-activation layer against a dense evaluation: every expert on
    every token in numpy, the activation rounded to f32 and quantised by
    blocks of 32 along F, the down product on the dequantised values."""
    cfg, d = small_inputs(40, 64, 128, 4, 2, "bf16", 111)
    wd_mx = oracle.mx_quantize(d["w_down"].reshape(4 * 64, 128))
    r = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], 2, w_down_mx=wd_mx)
    X, L = widen(d["x"]), d["logits"].astype(np.float64)
    Wg, Wu = widen(d["w_gate"]), widen(d["w_up"])
    Wd = oracle.mx_dequantize(wd_mx, 4 * 64, 128).reshape(4, 64, 128)
    order = np.argsort(-L, axis=1, kind="stable")[:, :2]
    p = np.exp(L - L.max(axis=1, keepdims=True))
    p = p / p.sum(axis=1, keepdims=True)
    out = np.zeros((40, 64))
    for e in range(4):
        G, U = X @ Wg[e].T, X @ Wu[e].T
        h = (G / (1.0 + np.exp(-G)) * U).astype(np.float32).astype(np.float64)
        hq = oracle.mx_dequantize(oracle.mx_quantize(h), 40, 128)
        mask = (order == e).any(axis=1)
        w = np.where(mask, p[:, e] / np.take_along_axis(p, order, axis=1).sum(axis=1), 0.0)
        out += w.astype(np.float32).astype(np.float64)[:, None] * (hq @ Wd[e].T)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12)
