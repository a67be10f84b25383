"""Host-only checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/mxq.h declares, and rejects invalid arguments with the
documented status before anything is launched.  Pointers here are fake
device addresses: validation never dereferences them.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel", Numerics and tests: every launcher error path is
exercised (bounds, pointer alignment, geometry guards).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def m():
    import swiglu_mxfp8_quant_amd as mod
    return mod


def header_functions():
    src = open(os.path.join(ROOT, "include", "mxq.h")).read()
    return sorted(set(re.findall(r"^(?:mxq_status|const char \*)\s*(mxq_\w+)\(", src, re.M)))


def test_header_symbols_exported(m):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(m.lib, n), n
    assert sorted(m.EXPORTS) == names


def test_version_and_status_strings(m):
    assert m.version().startswith("mxq")
    for s, name in m.STATUS.items():
        assert m.lib.mxq_status_string(s).decode() == name


BASE = 0x7F0000000000  # a 256-byte aligned fake device address


def fake(off=0):
    return ctypes.c_void_p(BASE + off)


def mxout(codes_off, ld, scales_off, lds):
    return m_mod().mxq_mx_out(BASE + codes_off, ld, BASE + scales_off, lds)


def m_mod():
    import swiglu_mxfp8_quant_amd as mod
    return mod


def fwd(m, M=64, K=64, gate=0, ldg=128, up=64 * 2, ldu=128, scale=None, groups=None, dirs=1,
        row=None, col=None, act=None):
    mb = 1 << 24
    if row is None and dirs & 1:
        row = m.mxq_mx_out(BASE + 4 * mb, K, BASE + 5 * mb, K // 32)
    if col is None and dirs & 2:
        col = m.mxq_mx_out(BASE + 6 * mb, K, BASE + 7 * mb, K)
    return m.lib.mxq_swiglu_quantize_fwd(
        None if act is None else ctypes.byref(act), M, K, fake(gate), ldg, fake(up), ldu,
        None if scale is None else fake(scale), None if groups is None else ctypes.byref(groups), dirs,
        None if row is None else ctypes.byref(row), None if col is None else ctypes.byref(col), None)


def test_fwd_validation(m):
    assert fwd(m, K=48) == 2                       # K % 32
    assert fwd(m, M=-1) == 2
    assert fwd(m, dirs=0) == 2
    assert fwd(m, dirs=4) == 2
    assert fwd(m, ldg=32) == 2                     # ld < K
    assert fwd(m, gate=8) == 3                     # misaligned pointer
    assert fwd(m, ldg=132) == 3                    # pitch not 16 bytes
    row = m.mxq_mx_out(0, 64, BASE + (5 << 24), 2)
    assert fwd(m, row=row) == 1                    # enabled output missing
    row = m.mxq_mx_out(BASE + (4 << 24), 32, BASE + (5 << 24), 2)
    assert fwd(m, row=row) == 2                    # ld_codes < K
    row = m.mxq_mx_out(BASE + 0, 64, BASE + (5 << 24), 2)
    assert fwd(m, row=row) == 5                    # codes overlap gate
    col = m.mxq_mx_out(BASE + (6 << 24), 64, BASE + (7 << 24) + 4, 64)
    assert fwd(m, dirs=2, col=col) == 3            # colwise scales must be 8-aligned
    act = m.mxq_act(1, 0.0)
    assert fwd(m, act=act) == 2                    # clamp limit must be > 0
    act = m.mxq_act(9, 7.0)
    assert fwd(m, act=act) == 6                    # unknown activation
    g = m.mxq_groups(0, BASE + (9 << 24), BASE + (10 << 24))
    assert fwd(m, dirs=2, groups=g) == 2           # G < 1
    g = m.mxq_groups(4, None, None)
    assert fwd(m, dirs=2, groups=g) == 1           # offsets missing
    assert fwd(m, M=0) == 0                        # empty: success, nothing launched
    assert "K" in m.last_error() or m.last_error() == ""


def test_bwd_validation(m):
    lib = m.lib
    K, M = 64, 64
    none = None

    def call(dirs=1, dgate=fake(1 << 28), dup=fake((1 << 28) + 128), dscale=None, ws=None, wsb=0, ldd=128,
             grad=fake(3 << 24)):
        row = m.mxq_mx_out(BASE + (4 << 24), 2 * K, BASE + (5 << 24), 2 * K // 32)
        col = m.mxq_mx_out(BASE + (6 << 24), 2 * K, BASE + (7 << 24), 2 * K)
        return lib.mxq_swiglu_quantize_bwd(none, M, K, grad, K, fake(0), 2 * K, fake(128), 2 * K, none, none,
                                           dgate, ldd, dup, ldd, dscale, dirs,
                                           ctypes.byref(row) if dirs & 1 else None,
                                           ctypes.byref(col) if dirs & 2 else None, ws, wsb, None)
    assert call(dgate=None) == 1                   # dgate without dup
    assert call(dirs=0, dgate=None, dup=None) == 2  # nothing requested
    assert call(ldd=32) == 2
    assert call(dgate=fake((1 << 28) + 2)) == 3
    assert call(grad=fake(1)) == 3
    # a shape whose dscale needs partial sums: the missing workspace is caught
    n = ctypes.c_size_t(0)
    K2 = 7168
    assert lib.mxq_swiglu_quantize_bwd_workspace(M, K2, 3, ctypes.byref(n)) == 0
    assert n.value > 0
    row = m.mxq_mx_out(BASE + (4 << 24), 2 * K2, BASE + (5 << 24), 2 * K2 // 32)
    st = lib.mxq_swiglu_quantize_bwd(none, M, K2, fake(3 << 26), K2, fake(0), 2 * K2, fake(2 * K2), 2 * K2,
                                     none, none, none, 0, none, 0, fake(1 << 30), 1, ctypes.byref(row), None,
                                     None, 0, None)
    assert st == 8, m.last_error()


def test_offsets_validation(m):
    lib = m.lib
    assert lib.mxq_splits_to_offsets(None, 4, fake(64), None, None, None) == 1
    assert lib.mxq_splits_to_offsets(fake(0), 0, fake(64), None, None, None) == 2
    assert lib.mxq_splits_to_offsets(fake(4), 4, fake(64), None, None, None) == 3
    assert lib.mxq_splits_to_offsets(fake(0), 4, fake(16), None, None, None) == 5   # row_off overlaps splits


def test_quantize_validation(m):
    lib = m.lib
    row = m.mxq_mx_out(BASE + (4 << 24), 64, BASE + (5 << 24), 2)
    assert lib.mxq_quantize(64, 64, fake(0), 60, None, 1, ctypes.byref(row), None, None) == 2
    assert lib.mxq_quantize(64, 33, fake(0), 64, None, 1, ctypes.byref(row), None, None) == 2
    assert lib.mxq_quantize(64, 64, fake(0), 64, None, 3, ctypes.byref(row), None, None) == 1


def gemm_args(m, mode, M=256, N=256, K=256, G=4, max_wg=0):
    """MXFP8 grouped-GEMM arguments over fake, disjoint, aligned device ranges."""
    f8 = m.DTYPE_MXFP8
    if mode == m.GEMM_TN:
        A = m.mxq_operand(f8, BASE + (1 << 28), M, 0, BASE + (2 << 28), M, 0)
        B = m.mxq_operand(f8, BASE + (3 << 28), N, 0, BASE + (4 << 28), N, 0)
        return m.mxq_gemm_args(mode, G, BASE, BASE + 4096, M, N, 0, 1024, A, B, m.DTYPE_BF16,
                               BASE + (5 << 28), N, M * N, 0, max_wg)
    A = m.mxq_operand(f8, BASE + (1 << 28), K, 0, BASE + (2 << 28), K // 32, 0)
    B = m.mxq_operand(f8, BASE + (3 << 28), K, N * K, BASE + (4 << 28), K // 32, N * (K // 32))
    return m.mxq_gemm_args(mode, G, BASE, None, M, N, K, M, A, B, m.DTYPE_BF16, BASE + (5 << 28), N, 0, 0,
                           max_wg)


def test_gemm_workspace_and_validation(m):
    """The K-grouped GEMM keeps its dynamic tile counter in the caller's
    workspace: the query asks for it, and a call without it (or misaligned)
    is refused before anything is launched; the other modes need none.  A
    negative workgroup cap is a shape error."""
    lib = m.lib
    tn, nt = gemm_args(m, m.GEMM_TN), gemm_args(m, m.GEMM_NT)
    assert m.mxq_grouped_gemm_workspace(tn) == 256
    assert m.mxq_grouped_gemm_workspace(nt) == 0
    assert lib.mxq_grouped_gemm(ctypes.byref(tn), None, 0, None) == 8            # MXQ_ERR_WORKSPACE
    assert lib.mxq_grouped_gemm(ctypes.byref(tn), fake(6 << 28), 255, None) == 8
    assert lib.mxq_grouped_gemm(ctypes.byref(tn), fake((6 << 28) + 2), 256, None) == 3   # MXQ_ERR_ALIGN
    assert lib.mxq_grouped_gemm(ctypes.byref(gemm_args(m, m.GEMM_TN, max_wg=-1)), fake(6 << 28), 256, None) == 2
    assert lib.mxq_grouped_gemm(ctypes.byref(gemm_args(m, m.GEMM_NT, max_wg=-8)), None, 0, None) == 2
    assert lib.mxq_grouped_gemm(ctypes.byref(gemm_args(m, m.GEMM_NT, K=48)), None, 0, None) == 2
