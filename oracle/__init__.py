"""CPU oracle for the MoE layer hot path -- TEST INFRASTRUCTURE ONLY.

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and the two share no code.

The arithmetic lives in ``moe_oracle.c`` (plain C, fp64); this module only
builds/loads it and marshals numpy arrays through ctypes.  The function
docstrings say which step of the layer each call is; the C file's header
cites the passages of the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE double, no contraction, OpenMP)."""
    if force or not os.path.exists(_LIB):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-shared", "-fPIC", _SRC, "-o", _LIB + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _configure(lib):
    P = ctypes.c_void_p
    I64, I32 = ctypes.c_int64, ctypes.c_int
    lib.orc_round_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_round_to_bf16.restype = ctypes.c_double
    lib.orc_route.argtypes = [I64, I32, I32, P, P, P]
    lib.orc_counts_offsets.argtypes = [I64, I32, I32, I32, I32, I32, P, P, P, P]
    lib.orc_permutation.argtypes = [I64, I32, I32, I32, I32, I32, P, P, P, P]
    lib.orc_dispatch.argtypes = [I64, I32, I32, I32, P, P, P]
    lib.orc_ffn_rows.argtypes = [I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, I64, P, P, P]
    lib.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_round.argtypes = [ctypes.c_double]
    lib.orc_e4m3_round.restype = ctypes.c_uint8
    lib.orc_mx_quantize.argtypes = [I64, I32, I32, P, P]
    lib.orc_mx_dequantize.argtypes = [I64, I32, P, P]
    lib.orc_mx_scales.argtypes = [I64, I32, P, P]
    lib.orc_combine_tokens.argtypes = [I32, I32, I64, P, P, P, P]
    lib.orc_epilogue.argtypes = [I64, P, P, I32, I32, P]
    lib.orc_moe_layer.argtypes = [I64, I32, I32, I32, I32, I32, I32, I32, I32, I32, P, P, P, P, P, P, I64, P,
                                  P, P, P, P, P, P, P, P, P]
    lib.orc_num_threads.argtypes = []
    for name in ("orc_route", "orc_counts_offsets", "orc_permutation", "orc_dispatch",
                 "orc_ffn_rows", "orc_combine_tokens", "orc_epilogue", "orc_moe_layer", "orc_num_threads",
                 "orc_mx_quantize", "orc_mx_dequantize", "orc_mx_scales"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = _configure(ctypes.CDLL(_LIB))
    return _lib


def build_variant(source_text: str, path: str) -> str:
    """Compile another copy of the oracle source (the mutation tests plant
    mistakes in such copies to show the pins catch them)."""
    src = path + ".c"
    with open(src, "w") as fh:
        fh.write(source_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared",
                    "-fPIC", src, "-o", path, "-lm"], check=True)
    return path


class use_library:
    """Context manager: route every call of this module to another build."""

    def __init__(self, path: str):
        self.lib = _configure(ctypes.CDLL(path))

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = self.lib
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def source_text() -> str:
    with open(_SRC) as fh:
        return fh.read()


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _dtype_code(arr):
    if arr.dtype == np.float32:
        return F32
    if arr.dtype == np.uint16:
        return BF16
    raise TypeError("oracle takes float32 arrays or bf16 bit patterns as uint16")


def round_to_bf16(v: float) -> float:
    """The oracle's own double -> bf16 (round to nearest even) rounding."""
    return _load().orc_round_to_bf16(float(v))


def num_threads() -> int:
    return _load().orc_num_threads()


def route(logits, k):
    """Step 1: top-k indices (descending, ties to the lower index) and weights."""
    logits = _c(logits, np.float32)
    M, E = logits.shape
    idx = np.empty((M, k), np.int32)
    w = np.empty((M, k), np.float32)
    _check(_load().orc_route(M, E, k, _p(logits), _p(idx), _p(w)), "route")
    return idx, w


def _local(E, expert_base, local_experts):
    return local_experts if local_experts else E


def counts_offsets(topk_idx, E, S=1, src_block=None, expert_base=0, local_experts=0):
    """Step 2: per-(source block, expert) counts and the exclusive prefix sum.
    With local_experts = EL > 0 only pairs routed to experts
    [expert_base, expert_base + EL) are counted, as segment src*EL + (e - base)."""
    topk_idx = _c(topk_idx, np.int32)
    src_block = _c(src_block, np.int32)
    M, k = topk_idx.shape
    G = S * _local(E, expert_base, local_experts)
    counts = np.empty(G, np.int32)
    offsets = np.empty(G + 1, np.int32)
    _check(_load().orc_counts_offsets(M, E, k, S, expert_base, local_experts, _p(topk_idx), _p(src_block),
                                      _p(counts), _p(offsets)), "counts_offsets")
    return counts, offsets


def permutation(topk_idx, E, S=1, src_block=None, expert_base=0, local_experts=0):
    """Step 3: the stable permutation and its inverse (-1 for dropped pairs
    and for sorted positions past the kept pairs)."""
    topk_idx = _c(topk_idx, np.int32)
    src_block = _c(src_block, np.int32)
    M, k = topk_idx.shape
    s2f = np.empty(M * k, np.int32)
    f2s = np.empty(M * k, np.int32)
    _check(_load().orc_permutation(M, E, k, S, expert_base, local_experts, _p(topk_idx), _p(src_block), _p(s2f),
                                   _p(f2s)), "permutation")
    return s2f, f2s


def dispatch(x, k, sorted_to_flat, out=None):
    """Step 4: X_perm rows, a byte copy of the token rows (rows of sorted
    positions that hold no pair are written as zeros).  out: an optional
    [M*k, H] buffer of x's dtype to write into."""
    x = np.ascontiguousarray(x)
    M, H = x.shape
    s2f = _c(sorted_to_flat, np.int32)
    xp = np.empty((M * k, H), x.dtype) if out is None else out
    assert xp.shape == (M * k, H) and xp.dtype == x.dtype and xp.flags.c_contiguous
    _check(_load().orc_dispatch(M, H, k, x.dtype.itemsize, _p(x), _p(s2f), _p(xp)), "dispatch")
    return xp


def e4m3_value(code: int) -> float:
    """Value of an e4m3 code (OCP 8-bit "fn" variant)."""
    return _load().orc_e4m3_value(int(code))


def e4m3_round(v: float) -> int:
    """Nearest e4m3 code (ties to the even code, clamped to +-448)."""
    return int(_load().orc_e4m3_round(float(v)))


def mx_bytes(rows, cols):
    """Bytes of an MX buffer: the codes, then the scales in groups of 32 rows."""
    return rows * cols + (rows + 31) // 32 * 32 * (cols // 32)


def mx_quantize(values):
    """MXFP8 quantisation of a [rows, cols] array (f32, bf16 bits or f64;
    cols a multiple of 128) in blocks of 32 along a row: one uint8 buffer of
    rows*cols e4m3 codes followed by the scale bytes (groups of 32 rows, per
    128-column quad the 4 bytes of each row)."""
    v = np.ascontiguousarray(values)
    rows, cols = v.shape[0], int(np.prod(v.shape[1:]))
    dt = -1 if v.dtype == np.float64 else _dtype_code(v)
    out = np.empty(mx_bytes(rows, cols), np.uint8)
    _check(_load().orc_mx_quantize(rows, cols, dt, _p(v), _p(out)), "mx_quantize")
    return out


def mx_dequantize(buf, rows, cols):
    """Values of an MXFP8 buffer as float64 [rows, cols]."""
    b = _c(buf, np.uint8)
    out = np.empty((rows, cols), np.float64)
    _check(_load().orc_mx_dequantize(rows, cols, _p(b), _p(out)), "mx_dequantize")
    return out


def mx_scales(buf, rows, cols):
    """Scale bytes of an MXFP8 buffer as a [rows, cols/32] uint8 array."""
    b = _c(buf, np.uint8)
    out = np.empty((rows, cols // 32), np.uint8)
    _check(_load().orc_mx_scales(rows, cols, _p(b), _p(out)), "mx_scales")
    return out


def ffn_rows(x, w_gate, w_up, w_down, k, S, sorted_to_flat, offsets, rows, w_down_mx=None):
    """Steps 5-6 for the listed sorted rows: (hact [n,F], y [n,H]) in float64.
    w_down_mx (an mx_quantize buffer of W_down) selects the MXFP8 activation
    path, as in moe_layer."""
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x)
    E, F, H = w_gate.shape
    wg, wu, wd = (np.ascontiguousarray(a, dtype=x.dtype) for a in (w_gate, w_up, w_down))
    act_fp8 = 0
    if w_down_mx is not None:
        act_fp8 = 1
        wd = _c(w_down_mx, np.uint8)
        assert wd.size == mx_bytes(E * H, F)
    rows = _c(rows, np.int64)
    n = rows.shape[0]
    hact = np.empty((n, F), np.float64)
    y = np.empty((n, H), np.float64)
    _check(_load().orc_ffn_rows(H, F, E, S, k, dt, act_fp8, _p(x), _p(wg), _p(wu), _p(wd),
                                _p(_c(sorted_to_flat, np.int32)), _p(_c(offsets, np.int32)), n, _p(rows),
                                _p(hact), _p(y)), "ffn_rows")
    return hact, y


def combine_tokens(topk_w_sub, y_rows, kept=None):
    """Step 7: out[i] = sum over kept j of w[i,j] * y_rows[i*k+j] in float64
    (kept [n,k] bool, None: every pair)."""
    w = _c(topk_w_sub, np.float32)
    n, k = w.shape
    y_rows = _c(y_rows, np.float64)
    H = y_rows.shape[1]
    kp = None if kept is None else _c(np.asarray(kept, bool).astype(np.uint8), np.uint8)
    out = np.empty((n, H), np.float64)
    _check(_load().orc_combine_tokens(H, k, n, _p(w), _p(y_rows), _p(kp), _p(out)), "combine_tokens")
    return out


def epilogue(acc, residual=None, out_dtype="f32"):
    """cast(acc + residual): the residual (f32 array, or uint16 bf16 bits)
    widened exactly, the sum in float64, rounded to bf16 (nearest even) when
    out_dtype is "bf16".  Returns float64 values."""
    acc = _c(acc, np.float64)
    res = None if residual is None else np.ascontiguousarray(residual)
    if res is not None:
        assert res.shape == acc.shape
    rdt = F32 if res is None else _dtype_code(res)
    odt = {"f32": F32, "bf16": BF16}[out_dtype]
    out = np.empty(acc.shape, np.float64)
    _check(_load().orc_epilogue(acc.size, _p(acc), _p(res), rdt, odt, _p(out)), "epilogue")
    return out


def moe_layer(x, logits, w_gate, w_up, w_down, k, S=1, src_block=None, tokens=None, want_rows=False,
              expert_base=0, local_experts=0, residual=None, out_dtype="f32", w_down_mx=None):
    """The whole layer.  Routing, counts, offsets and the permutation are
    computed for every token; the FFN and the combine for ``tokens`` only
    (all tokens if None).  Routing chooses among logits.shape[1] experts;
    with local_experts = EL > 0 the weights hold experts
    [expert_base, expert_base + EL) only and out is the partial combine over
    the pairs routed to them.  residual [M,H] and out_dtype select the
    epilogue cast(acc + residual) ("out" then holds its values; "acc" the
    plain combine).  w_down_mx (an mx_quantize buffer of W_down) selects
    the MXFP8 activation path: Hact quantised in blocks of 32 along F and the
    down product on the quantised values.  Returns a dict of numpy arrays."""
    x = np.ascontiguousarray(x)
    dt = _dtype_code(x)
    logits = _c(logits, np.float32)
    M, H = x.shape
    EL, F, H2 = w_gate.shape
    E = logits.shape[1]
    assert H2 == H and logits.shape == (M, E)
    assert EL == _local(E, expert_base, local_experts)
    wg, wu, wd = (np.ascontiguousarray(a, dtype=x.dtype) for a in (w_gate, w_up, w_down))
    act_fp8 = 0
    if w_down_mx is not None:
        act_fp8 = 1
        wd = _c(w_down_mx, np.uint8)
        assert wd.size == mx_bytes(EL * H, F)
    src_block = _c(src_block, np.int32)
    tok = None if tokens is None else _c(tokens, np.int64)
    n_tok = M if tok is None else tok.shape[0]
    r = dict(
        topk_idx=np.empty((M, k), np.int32), topk_w=np.empty((M, k), np.float32),
        counts=np.empty(S * EL, np.int32), offsets=np.empty(S * EL + 1, np.int32),
        sorted_to_flat=np.empty(M * k, np.int32), flat_to_sorted=np.empty(M * k, np.int32),
        out=np.empty((n_tok, H), np.float64))
    hact = np.empty((n_tok * k, F), np.float64) if want_rows else None
    y = np.empty((n_tok * k, H), np.float64) if want_rows else None
    _check(_load().orc_moe_layer(M, H, F, E, k, S, expert_base, local_experts, dt, act_fp8, _p(x), _p(logits),
                                 _p(src_block), _p(wg), _p(wu), _p(wd), n_tok, _p(tok), _p(r["topk_idx"]),
                                 _p(r["topk_w"]), _p(r["counts"]), _p(r["offsets"]), _p(r["sorted_to_flat"]),
                                 _p(r["flat_to_sorted"]), _p(r["out"]), _p(hact), _p(y)), "moe_layer")
    if want_rows:
        r["hact"] = hact
        r["y"] = y
    if residual is not None or out_dtype != "f32":
        r["acc"] = r["out"]
        res = None
        if residual is not None:
            res = np.ascontiguousarray(residual)
            res = res if tokens is None else res[tok]
        r["out"] = epilogue(r["acc"], res, out_dtype)
    return r
