"""The C ABI (no GPU needed): the library loads, exports every function that
include/moe.h declares, and rejects bad arguments with the documented status
before touching the GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "routing_grouped_gemm_router_amd", "libmoe.so")


def declared():
    src = open(HDR).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted({n for n in names if n.startswith(("moe_", "mxfp8_"))})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        # load the build script by path (importing the package needs the library)
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_moe_build", os.path.join(ROOT, "routing_grouped_gemm_router_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return ctypes.CDLL(LIB)


def test_header_declares_the_boundary():
    names = declared()
    for n in ("moe_route", "moe_permute", "moe_grouped_gemm", "moe_combine", "moe_backward",
              "mxfp8_quantize"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    for s in range(7):
        assert lib.moe_status_str(s).startswith(b"MOE_")
    lib.moe_version.restype = ctypes.c_int32
    assert lib.moe_version() == 102


def test_validation_without_gpu(lib):
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.moe_route.argtypes = [P, I64, I32, I32, I32] + [P] * 9 + [SZ, P]
    fake = ctypes.c_void_p(0x100000)      # never dereferenced: validation fails first
    nul = ctypes.c_void_p(0)
    args = lambda T, E, k, ws=1 << 20, logits=fake, counts=fake: (
        logits, T, E, k, 128, fake, fake, counts, fake, fake, fake, fake, fake, fake, ws, nul)
    assert lib.moe_route(*args(16, 8, 9)) == 2          # k > E
    assert lib.moe_route(*args(16, 300, 2)) == 2        # E > 256
    assert lib.moe_route(*args(1 << 30, 8, 4)) == 2     # T*k >= 2^31
    assert lib.moe_route(*args(16, 8, 2, logits=nul)) == 1
    assert lib.moe_route(*args(16, 8, 2, counts=nul)) == 1
    assert lib.moe_route(*args(16, 8, 2, ws=3)) == 5    # workspace too small
    unaligned = ctypes.c_void_p(0x100004)
    assert lib.moe_route(*args(16, 8, 2, logits=unaligned)) == 4
    lib.moe_route_workspace_size.argtypes = [I64, I32, I32]
    lib.moe_route_workspace_size.restype = SZ
    assert lib.moe_route_workspace_size(16384, 128, 4) == 4 * 128 * 256
    lib.moe_permute.argtypes = [P, P, I32, I64, I32, I32, P, P, P, P]
    assert lib.moe_permute(fake, nul, 1, 16, 48, 2, fake, fake, nul, nul) == 2   # d % 32
    assert lib.moe_permute(fake, nul, 7, 16, 64, 2, fake, fake, nul, nul) == 3   # dtype
    assert lib.moe_permute(fake, nul, 2, 16, 64, 2, fake, fake, nul, nul) == 1   # MXFP8 scales
    assert lib.moe_permute(nul, nul, 1, 0, 64, 2, nul, nul, nul, nul) == 0       # T = 0: no-op
    lib.moe_combine.argtypes = [P, I32, P, P, I64, I32, I32, P, P]
    assert lib.moe_combine(fake, 2, fake, fake, 16, 64, 2, fake, nul) == 3       # no MXFP8 combine
    lib.mxfp8_quantize.argtypes = [P, I32, I64, I64, I32, P, I32, P, P, P, P]
    assert lib.mxfp8_quantize(fake, 1, 64, 40, 1, nul, 0, nul, fake, fake, nul) == 2
    assert lib.mxfp8_quantize(fake, 1, 64, 64, 2, nul, 0, nul, fake, fake, nul) == 2


def test_gemm_descriptor_validation(lib):
    import sys
    sys.path.insert(0, ROOT)
    # the binding needs torch only for device buffers; the descriptor layout is plain ctypes
    from routing_grouped_gemm_router_amd import GemmDesc, BwdDesc
    lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_void_p]
    g = GemmDesc()
    g.mode, g.dtype, g.epilogue, g.n_groups, g.rows = 0, 1, 0, 8, 64
    g.N, g.K = 64, 64
    g.offsets = g.A = g.B = g.C = 0x100000
    bad = GemmDesc.from_buffer_copy(g)
    bad.mode = 7
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 3
    bad = GemmDesc.from_buffer_copy(g)
    bad.epilogue = 2                          # SwiGLU backward needs DGRAD
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 3
    bad = GemmDesc.from_buffer_copy(g)
    bad.n_groups = 0
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 2
    bad = GemmDesc.from_buffer_copy(g)
    bad.K = 48
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 2
    bad = GemmDesc.from_buffer_copy(g)
    bad.A = 0
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 1
    bad = GemmDesc.from_buffer_copy(g)
    bad.epilogue = 1                          # SwiGLU forward needs aux_out
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 1
    lib.moe_backward.argtypes = [ctypes.POINTER(BwdDesc), ctypes.c_void_p]
    b = BwdDesc()
    b.dtype, b.d, b.h, b.E, b.k, b.T = 1, 64, 64, 8, 2, 16
    assert lib.moe_backward(ctypes.byref(b), None) == 1
    b.dtype = 7
    assert lib.moe_backward(ctypes.byref(b), None) == 3
    b.dtype = 2                               # MXFP8 needs d % 128 == 0
    assert lib.moe_backward(ctypes.byref(b), None) == 2
    b.d = b.h = 128
    assert lib.moe_backward(ctypes.byref(b), None) == 1       # missing weights / workspace


def test_mxfp8_gemm_validation(lib):
    import sys
    sys.path.insert(0, ROOT)
    from routing_grouped_gemm_router_amd import GemmDesc
    lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_void_p]
    g = GemmDesc()
    g.mode, g.dtype, g.epilogue, g.n_groups, g.rows = 0, 2, 0, 8, 64
    g.N, g.K = 64, 128
    g.offsets = g.A = g.B = g.C = 0x100000
    assert lib.moe_grouped_gemm(ctypes.byref(g), None) == 1          # scales missing
    g.a_scale = g.b_scale = 0x100000
    bad = GemmDesc.from_buffer_copy(g)
    bad.K = 96                                                       # K % 128
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 2
    bad = GemmDesc.from_buffer_copy(g)
    bad.a_scale = 0x100002                                           # scale words 4-byte aligned
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 4
    bad = GemmDesc.from_buffer_copy(g)
    bad.aux_out_scale = 0x100000                     # H' quantised: SwiGLU forward only
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 3
    sw = GemmDesc.from_buffer_copy(g)
    sw.epilogue, sw.aux_out, sw.aux_out_scale = 1, 0x100000, 0x100000
    assert lib.moe_grouped_gemm(ctypes.byref(sw), None) == 1         # column layout missing
    sw.aux_out_cols = 0x100000
    assert lib.moe_grouped_gemm(ctypes.byref(sw), None) == 1         # ... and its scales
    sw.aux_out_cols_scale = 0x100002
    assert lib.moe_grouped_gemm(ctypes.byref(sw), None) == 4         # 4-byte aligned
    sw.dtype = 1
    assert lib.moe_grouped_gemm(ctypes.byref(sw), None) == 3         # bf16 stores bf16 H'
    bad = GemmDesc.from_buffer_copy(g)
    bad.mode, bad.M, bad.N, bad.rows = 2, 64, 64, (1 << 24) + 1      # WGRAD column blocks:
    assert lib.moe_grouped_gemm(ctypes.byref(bad), None) == 2        # 32-bit row offsets
    lib.mxfp8_col_blocks.argtypes = [ctypes.c_int64, ctypes.c_int32]
    lib.mxfp8_col_blocks.restype = ctypes.c_size_t
    assert lib.mxfp8_col_blocks(65536, 128) == 65536 // 32 + 4 * 128 + 4


def test_capacity_validation(lib):
    """Host-side checks of the padded-capacity calls (nothing is launched)."""
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.moe_capacity_pad.argtypes = [P, P, P, I64, I32, I32, I32, P, P, P]
    lib.moe_capacity_zero_rows.argtypes = [P, I32, P, I32, I32, I32, P]
    buf = ctypes.create_string_buffer(4096)
    a = ctypes.addressof(buf)
    a16 = (a + 15) // 16 * 16
    assert lib.moe_capacity_pad(a, a, a, 16, 300, 2, 8, a, a, None) == 2        # E > 256
    assert lib.moe_capacity_pad(a, a, a, 16, 8, 2, -1, a, a, None) == 2         # capacity < 0
    assert lib.moe_capacity_pad(a, a, a, 16, 256, 2, 1 << 24, a, a, None) == 2  # E*C >= 2^31
    assert lib.moe_capacity_pad(a, a, a, 16, 8, 2, 8, a, None, None) == 1       # offsets_pad
    assert lib.moe_capacity_pad(None, a, a, 16, 8, 2, 8, a, a, None) == 1       # topk_idx
    assert lib.moe_capacity_zero_rows(a16, 2, a, 8, 8, 64, None) == 3           # MXFP8 buffer
    assert lib.moe_capacity_zero_rows(a16, 1, a, 8, 8, 33, None) == 2           # cols % 32
    assert lib.moe_capacity_zero_rows(a16, 1, a, 0, 8, 64, None) == 2           # E < 1
    assert lib.moe_capacity_zero_rows(None, 1, a, 8, 8, 64, None) == 1
    assert lib.moe_capacity_zero_rows(a16 + 4, 1, a, 8, 8, 64, None) == 4       # alignment
    assert lib.moe_capacity_zero_rows(None, 1, None, 8, 0, 64, None) == 0       # nothing to do


def test_load_balance_validation(lib):
    """Host-side checks of moe_load_balance (nothing is launched)."""
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.moe_load_balance.argtypes = [P, P, I64, I32, I32, ctypes.c_float, P, P, P, SZ, P]
    lib.moe_load_balance_workspace_size.argtypes = [I64, I32]
    lib.moe_load_balance_workspace_size.restype = SZ
    assert lib.moe_load_balance_workspace_size(16384, 128) == 256 * 128 * 4 + 128 * 8
    fake = 0x100000
    big = 1 << 30
    assert lib.moe_load_balance(fake, fake, 16, 300, 2, 1.0, fake, None, fake, big, None) == 2  # E
    assert lib.moe_load_balance(fake, fake, 16, 8, 9, 1.0, fake, None, fake, big, None) == 2    # k > E
    assert lib.moe_load_balance(fake, fake, 16, 8, 2, 1.0, None, None, fake, big, None) == 1    # stats
    assert lib.moe_load_balance(None, fake, 16, 8, 2, 1.0, fake, None, fake, big, None) == 1    # logits
    assert lib.moe_load_balance(fake, fake, 16, 8, 2, 1.0, fake, None, None, big, None) == 1    # ws
    assert lib.moe_load_balance(fake, fake, 16, 8, 2, 1.0, fake + 2, None, fake, big, None) == 4
    assert lib.moe_load_balance(fake, fake, 16, 8, 2, 1.0, fake, fake + 1, fake, big, None) == 4
    assert lib.moe_load_balance(fake, fake, 16, 8, 2, 1.0, fake, None, fake + 4, big, None) == 4
    assert lib.moe_load_balance(fake, fake, 100, 8, 2, 1.0, fake, None, fake, 4, None) == 5     # ws size


def test_accumulate_and_quantize_both_validation(lib):
    import sys
    sys.path.insert(0, ROOT)
    from routing_grouped_gemm_router_amd import GemmDesc, BwdDesc
    lib.moe_grouped_gemm.argtypes = [ctypes.POINTER(GemmDesc), ctypes.c_void_p]
    g = GemmDesc()
    g.mode, g.dtype, g.epilogue, g.n_groups, g.rows = 0, 1, 0, 8, 64
    g.N, g.K = 64, 64
    g.offsets = g.A = g.B = g.C = 0x100000
    g.accumulate = 1                               # accumulate is for WGRAD only
    assert lib.moe_grouped_gemm(ctypes.byref(g), None) == 3
    g.mode, g.M, g.N, g.accumulate = 2, 64, 64, 2  # and takes 0 or 1
    assert lib.moe_grouped_gemm(ctypes.byref(g), None) == 3
    lib.moe_backward.argtypes = [ctypes.POINTER(BwdDesc), ctypes.c_void_p]
    b = BwdDesc()
    b.dtype, b.d, b.h, b.E, b.k, b.T, b.accumulate_dw = 1, 64, 64, 8, 2, 16, 3
    assert lib.moe_backward(ctypes.byref(b), None) == 3
    b.dtype, b.d, b.h, b.accumulate_dw = 2, 128, 128, 0          # MXFP8: T*k <= 2^24
    b.T = (1 << 23) + 1
    assert lib.moe_backward(ctypes.byref(b), None) == 2
    b.T = 16
    for dt in (0, 1, 2):                                         # h <= 8192: GEMM1 is 2h wide
        b.dtype, b.h = dt, 8192 + 128
        assert lib.moe_backward(ctypes.byref(b), None) == 2
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.mxfp8_quantize_both.argtypes = [P, I32, I64, I64, P, I32, P, P, P, P, P]
    f = 0x100000
    assert lib.mxfp8_quantize_both(f, 2, 64, 64, None, 0, f, f, f, f, None) == 3     # dtype
    assert lib.mxfp8_quantize_both(f, 0, 64, 48, None, 0, f, f, f, f, None) == 2     # cols % 32
    assert lib.mxfp8_quantize_both(f, 0, 64, 64, f, 0, f, f, f, f, None) == 2        # n_groups
    assert lib.mxfp8_quantize_both(f, 0, 64, 64, None, 0, f, None, f, f, None) == 1
    assert lib.mxfp8_quantize_both(f + 4, 0, 64, 64, None, 0, f, f, f, f, None) == 4
    assert lib.mxfp8_quantize_both(None, 0, 0, 64, None, 0, None, None, None, None, None) == 0
