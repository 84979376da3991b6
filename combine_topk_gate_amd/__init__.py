"""Python binding of the MoE layer library (``lib/libmoe.so``, C ABI in
``include/moe.h``).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  Tensors are torch device tensors (row-major, contiguous); the
binding passes their data pointers and the current HIP stream of torch (or
the stream given) straight through.  There is no fallback: if the library is
missing, loading it raises.

The entry points keep the C names: ``moe_route``, ``moe_dispatch``,
``moe_dispatch_noalloc``, ``moe_grouped_gemm``, ``moe_combine``, ``moe_combine_ex``, ``moe_layer``,
``moe_layer_ex`` (plus
``moe_workspace_bytes``, ``moe_layer_default_movers``,
``moe_debug_device_status``, ``moe_status_string``, ``moe_abi_version``).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4
MOE_ERR_DEVICE_TIMEOUT = 5

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_DTYPE_BF16_MXFP8 = 2

MOE_OP_DISPATCH = 0
MOE_OP_GROUPED_GEMM = 1
MOE_OP_LAYER = 2

MOE_NOALLOC_SCRATCH_BYTES = 1 << 20

EXPORTED = ("moe_workspace_bytes", "moe_route", "moe_dispatch", "moe_dispatch_noalloc", "moe_grouped_gemm", "moe_combine", "moe_combine_ex",
            "moe_layer", "moe_layer_ex", "moe_quantize_mxfp8", "moe_transpose_weights", "moe_layer_default_movers",
            "moe_debug_device_status",
            "moe_status_string", "moe_abi_version")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_name(status)} ({status})")
        self.status = status


class Problem(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int64), ("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("topk", ctypes.c_int32), ("num_src_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("expert_base", ctypes.c_int32), ("local_experts", ctypes.c_int32)]


class Epilogue(ctypes.Structure):
    _fields_ = [("residual", ctypes.c_void_p), ("out_dtype", ctypes.c_int32)]


class LayerAux(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "counts", "offsets", "sorted_to_flat",
                                              "flat_to_sorted", "x_perm", "hact", "y")]


class LayerOpts(ctypes.Structure):
    _fields_ = [("n_mover", ctypes.c_int32), ("grid", ctypes.c_int32), ("fused", ctypes.c_int32),
                ("spin_limit", ctypes.c_int32), ("gather", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"MoE HIP library not built: {path} missing "
                           "(run python -m combine_topk_gate_amd.build)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    PP = ctypes.POINTER(Problem)
    sig = {
        "moe_workspace_bytes": ([PP, I32], SZ),
        "moe_route": ([PP, P, P, P, P], I32),
        "moe_dispatch": ([PP, P, P, P, P, P, P, P, P, P, SZ, P], I32),
        "moe_dispatch_noalloc": ([PP, P, P, P, P, P, P, P, P, P], I32),
        "moe_grouped_gemm": ([PP, I32, P, P, P, P, P, P, SZ, P], I32),
        "moe_combine": ([PP, P, P, P, P, P], I32),
        "moe_combine_ex": ([PP, P, P, P, ctypes.POINTER(Epilogue), P, P], I32),
        "moe_layer": ([PP, P, P, P, P, P, P, P, ctypes.POINTER(LayerAux), ctypes.POINTER(LayerOpts), P, SZ, P], I32),
        "moe_layer_ex": ([PP, P, P, P, P, P, P, ctypes.POINTER(Epilogue), P, ctypes.POINTER(LayerAux),
                          ctypes.POINTER(LayerOpts), P, SZ, P], I32),
        "moe_quantize_mxfp8": ([ctypes.c_int64, I32, I32, P, P, P], I32),
        "moe_transpose_weights": ([ctypes.c_int64, I32, I32, I32, P, P, P], I32),
        "moe_layer_default_movers": ([PP], I32),
        "moe_debug_device_status": ([PP, P, SZ, P], I32),
        "moe_status_string": ([I32], ctypes.c_char_p),
        "moe_abi_version": ([], I32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def status_name(status: int) -> str:
    try:
        return load_library().moe_status_string(status).decode()
    except Exception:  # library not loadable: plain number
        return str(status)


_DTYPES = {"bf16": MOE_DTYPE_BF16, "f32": MOE_DTYPE_F32, "bf16_mxfp8": MOE_DTYPE_BF16_MXFP8,
           MOE_DTYPE_BF16: MOE_DTYPE_BF16, MOE_DTYPE_F32: MOE_DTYPE_F32, MOE_DTYPE_BF16_MXFP8: MOE_DTYPE_BF16_MXFP8}


def mx_bytes(rows: int, cols: int) -> int:
    """Bytes of an MXFP8 buffer of rows x cols (cols a multiple of 128): the
    codes, then one scale byte per 32 values with rows padded to a multiple
    of 32."""
    return rows * cols + (rows + 31) // 32 * 32 * (cols // 32)


def problem(M, H, F, E, k, S=1, dtype="bf16", expert_base=0, local_experts=0) -> Problem:
    return Problem(int(M), int(H), int(F), int(E), int(k), int(S), _DTYPES[dtype], int(expert_base),
                   int(local_experts))


def epilogue(residual=None, out_dtype="f32") -> Epilogue:
    """The combine's output epilogue: out = cast(acc + residual)."""
    return Epilogue(None if residual is None else residual.data_ptr(), _DTYPES[out_dtype])


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(status, what)


def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_status_string(status: int) -> str:
    return load_library().moe_status_string(status).decode()


def moe_workspace_bytes(p: Problem, op: int) -> int:
    return load_library().moe_workspace_bytes(ctypes.byref(p), op)


def moe_layer_default_movers(p: Problem) -> int:
    return load_library().moe_layer_default_movers(ctypes.byref(p))


def moe_route(p, logits, topk_idx, topk_w, stream=None):
    _check(load_library().moe_route(ctypes.byref(p), _ptr(logits), _ptr(topk_idx), _ptr(topk_w), _stream(stream)),
           "moe_route")


def moe_dispatch(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm, ws,
                 stream=None):
    _check(load_library().moe_dispatch(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(src_block), _ptr(counts),
                                       _ptr(offsets), _ptr(sorted_to_flat), _ptr(flat_to_sorted), _ptr(x_perm),
                                       _ptr(ws), _nbytes(ws), _stream(stream)), "moe_dispatch")


def moe_dispatch_noalloc(p, x, topk_idx, src_block, counts, offsets, sorted_to_flat, flat_to_sorted, x_perm,
                         stream=None):
    _check(load_library().moe_dispatch_noalloc(ctypes.byref(p), _ptr(x), _ptr(topk_idx), _ptr(src_block),
                                               _ptr(counts), _ptr(offsets), _ptr(sorted_to_flat),
                                               _ptr(flat_to_sorted), _ptr(x_perm), _stream(stream)),
           "moe_dispatch_noalloc")


def moe_grouped_gemm(p, layer, a, w0, w1, offsets, c, ws=None, stream=None):
    _check(load_library().moe_grouped_gemm(ctypes.byref(p), int(layer), _ptr(a), _ptr(w0), _ptr(w1), _ptr(offsets),
                                           _ptr(c), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_grouped_gemm")


def moe_combine(p, y, topk_w, flat_to_sorted, out, stream=None):
    _check(load_library().moe_combine(ctypes.byref(p), _ptr(y), _ptr(topk_w), _ptr(flat_to_sorted), _ptr(out),
                                      _stream(stream)), "moe_combine")


def moe_combine_ex(p, y, topk_w, flat_to_sorted, epi, out, stream=None):
    _check(load_library().moe_combine_ex(ctypes.byref(p), _ptr(y), _ptr(topk_w), _ptr(flat_to_sorted),
                                         ctypes.byref(epi) if epi is not None else None, _ptr(out),
                                         _stream(stream)), "moe_combine_ex")


def moe_quantize_mxfp8(src, dst, stream=None):
    """MXFP8 quantisation of a 2-D (or stacked) bf16/f32 tensor along its last
    dimension into dst (uint8, mx_bytes(rows, cols) bytes)."""
    import torch
    cols = src.shape[-1]
    rows = src.numel() // cols
    dt = MOE_DTYPE_BF16 if src.dtype == torch.bfloat16 else MOE_DTYPE_F32
    _check(load_library().moe_quantize_mxfp8(rows, cols, dt, _ptr(src), _ptr(dst), _stream(stream)),
           "moe_quantize_mxfp8")


def moe_transpose_weights(src, dst, stream=None):
    """dst[b] = src[b].T for a [batch, rows, cols] bf16/f32 tensor src and a
    [batch, cols, rows] tensor dst of the same dtype (weights given as the
    math writes them -> the storage the layer reads)."""
    import torch
    batch, rows, cols = (1,) * (3 - src.dim()) + tuple(src.shape)
    dt = MOE_DTYPE_BF16 if src.dtype == torch.bfloat16 else MOE_DTYPE_F32
    _check(load_library().moe_transpose_weights(batch, rows, cols, dt, _ptr(src), _ptr(dst), _stream(stream)),
           "moe_transpose_weights")


def moe_layer(p, x, logits, src_block, w_gate, w_up, w_down, out, ws, aux: dict | None = None,
              n_mover: int = -1, grid: int = 0, fused: int = 1, spin_limit: int = 0,
              gather: int = -1, stream=None):
    a = None
    if aux:
        a = LayerAux(**{k: (v.data_ptr() if v is not None else None) for k, v in aux.items()})
    o = LayerOpts(int(n_mover), int(grid), int(fused), int(spin_limit), int(gather))
    _check(load_library().moe_layer(ctypes.byref(p), _ptr(x), _ptr(logits), _ptr(src_block), _ptr(w_gate),
                                    _ptr(w_up), _ptr(w_down), _ptr(out), ctypes.byref(a) if a else None,
                                    ctypes.byref(o), _ptr(ws), _nbytes(ws), _stream(stream)), "moe_layer")


def moe_layer_ex(p, x, logits, src_block, w_gate, w_up, w_down, epi, out, ws, aux: dict | None = None,
                 n_mover: int = -1, grid: int = 0, fused: int = 1, spin_limit: int = 0,
                 gather: int = -1, stream=None):
    a = None
    if aux:
        a = LayerAux(**{k: (v.data_ptr() if v is not None else None) for k, v in aux.items()})
    o = LayerOpts(int(n_mover), int(grid), int(fused), int(spin_limit), int(gather))
    _check(load_library().moe_layer_ex(ctypes.byref(p), _ptr(x), _ptr(logits), _ptr(src_block), _ptr(w_gate),
                                       _ptr(w_up), _ptr(w_down), ctypes.byref(epi) if epi is not None else None,
                                       _ptr(out), ctypes.byref(a) if a else None, ctypes.byref(o), _ptr(ws),
                                       _nbytes(ws), _stream(stream)), "moe_layer_ex")


def moe_debug_device_status(p, ws, stream=None) -> int:
    return load_library().moe_debug_device_status(ctypes.byref(p), _ptr(ws), _nbytes(ws), _stream(stream))
