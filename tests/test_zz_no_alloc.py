"""The allocation-free dispatch (moe_dispatch_noalloc, static device
scratch) against moe_dispatch with a caller workspace: bit-exact counts,
offsets, permutation and X_perm, on two calls in a row, the second with a
smaller input (the scratch keeps the first call's contents)."""
import pytest
import torch

import combine_topk_gate_amd as moe
import moe_synth
from moe_gpu_util import upload

pytestmark = pytest.mark.gpu


def _dispatch(cfg, g, noalloc):
    p = moe.problem(cfg.M, cfg.H, cfg.F, cfg.E, cfg.k, cfg.S, cfg.dtype, cfg.base, cfg.local)
    M, k, H, G, R = cfg.M, cfg.k, cfg.H, cfg.S * cfg.EL, cfg.M * cfg.k
    act = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
    w = torch.empty((M, k), dtype=torch.float32, device="cuda")
    moe.moe_route(p, g["logits"], idx, w)
    # outputs start as all-ones bits, so a position the call fails to write shows
    o = dict(counts=torch.full((G,), -7, dtype=torch.int32, device="cuda"),
             offsets=torch.full((G + 1,), -7, dtype=torch.int32, device="cuda"),
             s2f=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
             f2s=torch.full((R,), -7, dtype=torch.int32, device="cuda"),
             xp=torch.zeros((R, H), dtype=act, device="cuda"))
    args = (p, g["x"], idx, g.get("src_block"), o["counts"], o["offsets"], o["s2f"], o["f2s"], o["xp"])
    if noalloc:
        moe.moe_dispatch_noalloc(*args)
    else:
        ws = torch.empty(max(4, moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH)), dtype=torch.uint8, device="cuda")
        moe.moe_dispatch(*args, ws)
    torch.cuda.synchronize()
    return o


CASES = [
    # (first call, second smaller call)
    (dict(M=3000, H=256, F=256, E=8, k=2), dict(M=700, H=256, F=256, E=8, k=2)),
    (dict(M=2048, H=128, F=128, E=16, k=4, S=4), dict(M=300, H=128, F=128, E=16, k=4, S=2)),
    (dict(M=1500, H=128, F=128, E=32, k=4, base=8, local=8), dict(M=90, H=128, F=128, E=32, k=4, base=8, local=8)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_noalloc_dispatch_equals_workspace_dispatch(first, second):
    for i, kw in enumerate((first, second)):
        kw = dict(kw)
        S = kw.pop("S", 1)
        base, local = kw.pop("base", 0), kw.pop("local", 0)
        cfg = moe_synth.Config("noalloc", kw["M"], kw["H"], kw["F"], kw["E"], kw["k"], S, "bf16", 40 + i, 0.0,
                               (kw["M"] // S) if S > 1 else 0, base, local)
        print(f"[noalloc] call {i}: {cfg}", flush=True)
        g = upload(moe_synth.make_inputs(cfg))
        a = _dispatch(cfg, g, noalloc=True)
        b = _dispatch(cfg, g, noalloc=False)
        for key in ("counts", "offsets", "s2f", "f2s"):
            assert torch.equal(a[key], b[key]), (i, key)
        n = int(b["offsets"][-1])
        assert torch.equal(a["xp"][:n].view(torch.int16), b["xp"][:n].view(torch.int16)), i
        assert int(b["counts"].sum()) == n


def test_noalloc_rejects_problems_past_its_scratch():
    # 16 source blocks x 64 experts = 1024 segments over 2^17 pairs: the
    # bookkeeping needs more than the static scratch holds
    p = moe.problem(1 << 16, 64, 64, 64, 4, 16)
    assert moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH) > moe.MOE_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moe.MoeError) as ex:
        t = torch.empty(16, dtype=torch.int32, device="cuda")
        moe.moe_dispatch_noalloc(p, t, t, t, t, t, t, t, t)
    assert ex.value.status == moe.MOE_ERR_UNSUPPORTED
