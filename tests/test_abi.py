"""The C-ABI library loads and exports every symbol include/moe.h declares,
and rejects bad arguments on the host (CPU only: no call here reaches a
kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_topk_gate_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.LIB_PATH):
        from combine_topk_gate_amd import build
        build.build()
    return moe.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert "moe_layer" in names and "moe_route" in names and len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", moe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (moe_\w+)", out))
    for n in names:
        assert n in exported, n
        getattr(lib, n)
    assert set(moe.EXPORTED) == set(names)


def test_no_torch_types_in_header():
    text = open(HEADER).read()
    assert "torch" not in text.lower().replace("torch", "", 0) or "at::" not in text
    assert "at::Tensor" not in text and "c10" not in text


def test_version_and_status_strings(lib):
    assert moe.moe_abi_version() >> 16 == 2
    assert moe.moe_status_string(moe.MOE_OK) == "MOE_OK"
    assert moe.moe_status_string(moe.MOE_ERR_DEVICE_TIMEOUT) == "MOE_ERR_DEVICE_TIMEOUT"


BAD = [
    dict(M=-1), dict(H=100), dict(H=0), dict(F=32), dict(E=0), dict(E=513), dict(k=0), dict(k=17),
    dict(E=4, k=5), dict(S=0), dict(S=3, E=512), dict(dtype=7),
    # held experts: negative, base without a count, past E, too many segments with the dropped one
    dict(EL=-1), dict(base=-1, EL=2), dict(base=3, EL=0), dict(base=6, EL=3), dict(E=512, S=4, EL=256),
    dict(E=512, S=3, EL=512),
]


@pytest.mark.parametrize("bad", BAD)
def test_invalid_problem_is_rejected_without_launch(lib, bad):
    shape = dict(M=16, H=64, F=64, E=8, k=2, S=1, dtype=moe.MOE_DTYPE_BF16, base=0, EL=0)
    shape.update(bad)
    p = moe.Problem(shape["M"], shape["H"], shape["F"], shape["E"], shape["k"], shape["S"], shape["dtype"],
                    shape["base"], shape["EL"])
    assert lib.moe_route(ctypes.byref(p), None, None, None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_workspace_bytes(ctypes.byref(p), moe.MOE_OP_LAYER) == 0
    assert lib.moe_layer_default_movers(ctypes.byref(p)) == -1


def test_null_and_misaligned_pointers_are_rejected(lib):
    p = moe.problem(16, 64, 64, 8, 2)
    assert lib.moe_route(None, None, None, None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_route(ctypes.byref(p), None, None, None, None) == moe.MOE_ERR_INVALID_ARGUMENT
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1002)
    # misaligned x in dispatch
    ws = ctypes.c_void_p(0x100000)
    r = lib.moe_dispatch(ctypes.byref(p), odd, fake, None, fake, fake, fake, fake, fake, ws, 1 << 20, None)
    assert r == moe.MOE_ERR_INVALID_ARGUMENT
    # too-small workspace
    r = lib.moe_dispatch(ctypes.byref(p), fake, fake, None, fake, fake, fake, fake, fake, ws, 0, None)
    assert r == moe.MOE_ERR_WORKSPACE_TOO_SMALL
    # source blocks without src_block
    p8 = moe.problem(16, 64, 64, 8, 2, S=2)
    r = lib.moe_dispatch(ctypes.byref(p8), fake, fake, None, fake, fake, fake, fake, fake, ws, 1 << 20, None)
    assert r == moe.MOE_ERR_INVALID_ARGUMENT
    # grouped gemm: bad layer, missing up weights
    assert lib.moe_grouped_gemm(ctypes.byref(p), 2, fake, fake, fake, fake, fake, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_grouped_gemm(ctypes.byref(p), 0, fake, fake, None, fake, fake, None, 0, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    # layer: workspace too small
    opts = moe.LayerOpts(-1, 0, 1, 0)
    r = lib.moe_layer(ctypes.byref(p), fake, fake, None, fake, fake, fake, fake, None, ctypes.byref(opts), ws, 16,
                      None)
    assert r == moe.MOE_ERR_WORKSPACE_TOO_SMALL


def test_held_experts_limits(lib):
    # S * EL = 1024 is fine when every expert is held; with one not held the
    # dropped pairs need one more segment
    assert lib.moe_workspace_bytes(ctypes.byref(moe.problem(16, 64, 64, 512, 2, S=2)), moe.MOE_OP_LAYER) > 0
    assert lib.moe_workspace_bytes(ctypes.byref(moe.problem(16, 64, 64, 512, 2, S=4, local_experts=256)),
                                   moe.MOE_OP_LAYER) == 0
    assert lib.moe_workspace_bytes(ctypes.byref(moe.problem(16, 64, 64, 512, 2, S=4, expert_base=1,
                                                            local_experts=255)), moe.MOE_OP_LAYER) > 0
    # EL = E with base 0 is the plain problem: same workspace
    a = moe.problem(300, 128, 256, 16, 4, S=2)
    b = moe.problem(300, 128, 256, 16, 4, S=2, local_experts=16)
    for op in (moe.MOE_OP_DISPATCH, moe.MOE_OP_GROUPED_GEMM, moe.MOE_OP_LAYER):
        assert lib.moe_workspace_bytes(ctypes.byref(a), op) == lib.moe_workspace_bytes(ctypes.byref(b), op)


def test_bad_epilogue_is_rejected(lib):
    p = moe.problem(16, 64, 64, 8, 2)
    fake, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)
    bad_type = moe.Epilogue(None, 7)
    assert lib.moe_combine_ex(ctypes.byref(p), fake, fake, fake, ctypes.byref(bad_type), fake, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    odd_res = moe.Epilogue(odd, moe.MOE_DTYPE_BF16)
    assert lib.moe_combine_ex(ctypes.byref(p), fake, fake, fake, ctypes.byref(odd_res), fake, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    ok = moe.Epilogue(None, moe.MOE_DTYPE_BF16)
    assert lib.moe_combine_ex(ctypes.byref(p), fake, fake, fake, ctypes.byref(ok), odd, None) == \
        moe.MOE_ERR_INVALID_ARGUMENT
    opts = moe.LayerOpts(-1, 0, 1, 0)
    ws = ctypes.c_void_p(0x100000)
    r = lib.moe_layer_ex(ctypes.byref(p), fake, fake, None, fake, fake, fake, ctypes.byref(bad_type), fake, None,
                         ctypes.byref(opts), ws, 1 << 30, None)
    assert r == moe.MOE_ERR_INVALID_ARGUMENT


def test_unsupported_sizes(lib):
    # 32-bit element offsets: R * H must stay below 2^31
    p = moe.problem(1 << 20, 4096, 64, 8, 2)
    assert lib.moe_route(ctypes.byref(p), None, None, None, None) == moe.MOE_ERR_UNSUPPORTED
    # a token count whose product with topk would wrap
    p = moe.problem((1 << 62) + 3, 4096, 64, 8, 2)
    assert lib.moe_route(ctypes.byref(p), None, None, None, None) == moe.MOE_ERR_UNSUPPORTED


def test_workspace_sizes_cover_intermediates(lib):
    for (M, H, F, E, k, S) in [(8192, 4096, 14336, 8, 2, 1), (16384, 7168, 4096, 16, 8, 8), (1, 64, 64, 1, 1, 1)]:
        p = moe.problem(M, H, F, E, k, S)
        R = M * k
        need = R * H * 2 + R * F * 2 + R * H * 4 + 4 * R * 4
        gemm = moe.moe_workspace_bytes(p, moe.MOE_OP_GROUPED_GEMM)
        # bf16: the split last round needs at least one 256 x 256 f32 partial
        assert gemm >= 256 * 256 * 4
        assert moe.moe_workspace_bytes(p, moe.MOE_OP_LAYER) >= need + gemm
        assert moe.moe_workspace_bytes(p, moe.MOE_OP_DISPATCH) >= 4 * S * E
    p32 = moe.problem(256, 256, 512, 8, 2, 1, "f32")
    assert moe.moe_workspace_bytes(p32, moe.MOE_OP_GROUPED_GEMM) == 0


def test_mxfp8_quantiser_rejects_bad_arguments(lib):
    fake = ctypes.c_void_p(1 << 20)
    lib.moe_quantize_mxfp8.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    inval = moe.MOE_ERR_INVALID_ARGUMENT
    # columns must be a whole number of 128-column quads (the scale layout's unit)
    for cols in (0, 32, 96, 200, 384 + 32):
        assert lib.moe_quantize_mxfp8(4, cols, moe.MOE_DTYPE_BF16, fake, fake, None) == inval, cols
    assert lib.moe_quantize_mxfp8(-1, 128, moe.MOE_DTYPE_BF16, fake, fake, None) == inval
    assert lib.moe_quantize_mxfp8(4, 128, moe.MOE_DTYPE_BF16_MXFP8, fake, fake, None) == inval  # src dtype
    assert lib.moe_quantize_mxfp8(4, 128, moe.MOE_DTYPE_BF16, None, fake, None) == inval
    assert lib.moe_quantize_mxfp8(4, 128, moe.MOE_DTYPE_F32, fake, ctypes.c_void_p((1 << 20) + 8), None) == inval
    assert lib.moe_quantize_mxfp8(0, 128, moe.MOE_DTYPE_BF16, None, None, None) == moe.MOE_OK  # nothing to do
    # a row count whose product with cols would wrap
    assert lib.moe_quantize_mxfp8((1 << 62) + 5, 1 << 20, moe.MOE_DTYPE_BF16, fake, fake, None) == \
        moe.MOE_ERR_UNSUPPORTED


def test_mx_buffer_size_matches_the_layout():
    # codes, then one scale byte per 32 values with rows padded to 32
    assert moe.mx_bytes(1, 128) == 128 + 32 * 4
    assert moe.mx_bytes(32, 256) == 32 * 256 + 32 * 8
    assert moe.mx_bytes(33, 256) == 33 * 256 + 64 * 8
    assert moe.mx_bytes(0, 128) == 0


def test_noalloc_dispatch_checks_arguments_and_size_on_the_host(lib):
    """moe_dispatch_noalloc rejects bad arguments and problems whose
    bookkeeping exceeds its static scratch before touching the device."""
    text = open(HEADER).read()
    m = re.search(r"#define MOE_NOALLOC_SCRATCH_BYTES \(1u << (\d+)\)", text)
    assert m and moe.MOE_NOALLOC_SCRATCH_BYTES == 1 << int(m.group(1))
    fake, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1002)
    p = moe.problem(16, 64, 64, 8, 2)
    f = lib.moe_dispatch_noalloc
    assert f(ctypes.byref(p), fake, fake, None, None, fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID_ARGUMENT
    assert f(ctypes.byref(p), odd, fake, None, fake, fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID_ARGUMENT
    p2 = moe.problem(16, 64, 64, 8, 2, S=2)
    assert f(ctypes.byref(p2), fake, fake, None, fake, fake, fake, fake, fake, None) == moe.MOE_ERR_INVALID_ARGUMENT
    big = moe.problem(1 << 16, 64, 64, 64, 4, S=16)  # 512 chunks x 1024 segments
    assert lib.moe_workspace_bytes(ctypes.byref(big), moe.MOE_OP_DISPATCH) > moe.MOE_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), fake, fake, fake, fake, fake, fake, fake, fake, None) == moe.MOE_ERR_UNSUPPORTED
    # the workloads of the benchmark fit
    for (M, H, F, E, k, S) in [(8192, 4096, 14336, 8, 2, 1), (16384, 7168, 4096, 16, 8, 8), (4096, 2048, 1408, 64, 4, 1),
                               (16384, 4096, 6400, 16, 2, 1)]:
        q = moe.problem(M, H, F, E, k, S)
        assert lib.moe_workspace_bytes(ctypes.byref(q), moe.MOE_OP_DISPATCH) <= moe.MOE_NOALLOC_SCRATCH_BYTES


def test_weight_transpose_rejects_bad_arguments(lib):
    # host checks only: nothing here reaches a launch
    P = ctypes.c_void_p
    bf16, f32 = moe.MOE_DTYPE_BF16, moe.MOE_DTYPE_F32
    a, b = P(1 << 32), P((1 << 32) + (1 << 30))
    INV = moe.MOE_ERR_INVALID_ARGUMENT
    assert lib.moe_transpose_weights(2, 96, 128, bf16, a, b, None) == INV  # rows not a multiple of 64
    assert lib.moe_transpose_weights(2, 128, 100, bf16, a, b, None) == INV  # cols not a multiple of 64
    assert lib.moe_transpose_weights(2, 128, 128, 7, a, b, None) == INV  # dtype
    assert lib.moe_transpose_weights(-1, 128, 128, bf16, a, b, None) == INV
    assert lib.moe_transpose_weights(2, 128, 128, bf16, None, b, None) == INV
    assert lib.moe_transpose_weights(2, 128, 128, bf16, P((1 << 32) + 8), b, None) == INV  # misaligned
    # overlapping source and destination (2 x 128 x 128 f32 = 128 KiB)
    assert lib.moe_transpose_weights(2, 128, 128, f32, a, P((1 << 32) + (64 << 10)), None) == INV
    assert lib.moe_transpose_weights(2, 128, 128, f32, P((1 << 32) + (64 << 10)), a, None) == INV
    assert lib.moe_transpose_weights(0, 128, 128, bf16, a, b, None) == moe.MOE_OK  # nothing to do
    # sizes past 2^40 elements, including ones whose products would wrap
    UNS = moe.MOE_ERR_UNSUPPORTED
    assert lib.moe_transpose_weights(1 << 40, 64, 64, bf16, a, b, None) == UNS
    assert lib.moe_transpose_weights((1 << 62) + 1, 1 << 30, 1 << 30, bf16, a, b, None) == UNS
    assert lib.moe_transpose_weights(1 << 20, 1 << 14, 1 << 14, f32, a, b, None) == UNS
