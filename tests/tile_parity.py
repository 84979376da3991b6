"""Tile-covering, element-wise comparison of a GPU layer run against the
CPU oracle, shared by the parity tests (see parity_bounds for the rows and
the bounds)."""
import numpy as np
import torch

import oracle
import parity_bounds as pb
from moe_gpu_util import host, rel_fro, tolerances


def oracle_case(name, cfg, d, g, out, toks, seed):
    """The oracle's own routing and offsets (in full), the rows covering
    every tile with the oracle's Hact and Y for them, and the oracle's layer
    for the token sample toks (None: every token)."""
    cov = _oracle_rows(cfg, d, seed)
    print(f"[parity] {name}: {len(cov['rows'])} covering rows over {cov['tiles']} row tiles "
          f"({cov['halves']} halves)", flush=True)
    ref = oracle.moe_layer(d["x"], d["logits"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, S=cfg.S,
                           src_block=d["src_block"], tokens=toks, want_rows=True, expert_base=cfg.base,
                           local_experts=cfg.local)
    return dict(name=name, cfg=cfg, d=d, g=g, out=out, ref=ref, toks=toks, cov=cov)


def _oracle_rows(cfg, d, seed):
    """The oracle's own routing and offsets (in full), the rows covering
    every tile, and the oracle's Hact and Y for those rows."""
    idx, _ = oracle.route(d["logits"], cfg.k)
    held = dict(expert_base=cfg.base, local_experts=cfg.local)
    _, offs = oracle.counts_offsets(idx, cfg.E, cfg.S, d["src_block"], **held)
    s2f, _ = oracle.permutation(idx, cfg.E, cfg.S, d["src_block"], **held)
    rows, tiles, halves = pb.covering_rows(offs, seed)
    hr, yr = oracle.ffn_rows(d["x"], d["w_gate"], d["w_up"], d["w_down"], cfg.k, cfg.S, s2f, offs, rows)
    return dict(rows=rows, tiles=tiles, halves=halves, hact=hr, y=yr, offsets=offs, s2f=s2f)


def sample_rows(c):
    """Sorted rows of the sampled tokens' kept pairs, the tokens, and which of
    the oracle's per-pair rows (token-major, all k slots) they are."""
    cfg, r = c["cfg"], c["ref"]
    toks = np.arange(cfg.M) if c["toks"] is None else c["toks"]
    flat = (toks[:, None] * cfg.k + np.arange(cfg.k)[None, :]).reshape(-1)
    rows = r["flat_to_sorted"][flat].astype(np.int64)
    kept = rows >= 0
    return rows[kept], toks, kept


def compared_rows(c):
    """Covering rows and the token sample's rows, with the oracle's Hact and Y."""
    rows_s, _, kept = sample_rows(c)
    rows = np.concatenate([c["cov"]["rows"], rows_s])
    hr = np.concatenate([c["cov"]["hact"], c["ref"]["hact"][kept]])
    yr = np.concatenate([c["cov"]["y"], c["ref"]["y"][kept]])
    return rows, hr, yr


def bounds(c, o, rows, hr):
    """Per-element bounds of Hact and Y on the given rows, for the GPU
    outputs o (chain or fused layer with its intermediates)."""
    cfg, g = c["cfg"], c["g"]
    experts = pb.experts_of(c["ref"]["offsets"], rows, cfg.EL)
    tok = torch.from_numpy(c["cov"]["s2f"][rows] // cfg.k).cuda()
    sums = pb.gate_up_sums(g["x"][tok], g["w_gate"], g["w_up"], experts)
    h_allow = pb.hact_allowance(sums, cfg.dtype == "bf16")
    hg = o["hact"][torch.from_numpy(rows).cuda()].double()
    y_allow = pb.y_allowance(hg, torch.from_numpy(hr).cuda(), experts, lambda e: g["w_down"][e].double(), cfg.H)
    return hg, h_allow, y_allow


def check_ffn(c, o, what):
    rows, hr, yr = compared_rows(c)
    hg, h_allow, y_allow = bounds(c, o, rows, hr)
    print(f"[parity] {c['name']} {what}: {len(rows)} rows compared, covering {c['cov']['tiles']} row tiles",
          flush=True)
    pb.check_within(f"{c['name']} {what} Hact", hg.cpu().numpy(), hr, h_allow.cpu().numpy())
    yg = host(o["y"][torch.from_numpy(rows).cuda()])
    pb.check_within(f"{c['name']} {what} Y", yg, yr, y_allow.cpu().numpy())
    if len(rows) == 0:
        return
    rel, mabs = tolerances(c["cfg"])
    assert rel_fro(yg, yr) <= rel
    if mabs is not None:
        assert np.max(np.abs(yg - yr)) <= mabs
    if c["cfg"].dtype != "bf16":
        assert rel_fro(hg.cpu().numpy(), hr) <= 1e-5


def check_out(c, o, out, what):
    cfg, r = c["cfg"], c["ref"]
    rows, toks, kept = sample_rows(c)
    n_t = len(toks)
    # Y bounds for every pair of the sampled tokens (dropped pairs: zero)
    _, _, y_allow = bounds(c, o, rows, r["hact"][kept])
    yb = np.zeros((n_t * cfg.k, cfg.H))
    yb[kept] = y_allow.cpu().numpy()
    yg = np.zeros((n_t * cfg.k, cfg.H))
    yg[kept] = host(o["y"][torch.from_numpy(rows).cuda()])
    tk = torch.from_numpy(toks).cuda()
    wg = host(o["topk_w"][tk])
    allow = pb.out_allowance(wg, r["topk_w"][toks], yg, r["y"], yb, kept.reshape(n_t, cfg.k))
    got = host(out[tk])
    pb.check_within(f"{c['name']} {what} out", got, r["out"], allow)
    rel, mabs = tolerances(cfg)
    err = rel_fro(got, r["out"])
    print(f"[parity] {c['name']} {what}: out relF {err:.3e} maxabs {np.max(np.abs(got - r['out'])):.3e}")
    assert err <= rel
    if mabs is not None:
        assert np.max(np.abs(got - r["out"])) <= mabs
