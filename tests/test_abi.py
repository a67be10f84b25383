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


def test_activation_variant_validation(m):
    """SReLU is unary (no up, no dup); the GLU interleave block must be a
    positive multiple of 32 dividing K, applies to the SwiGLU kinds only, and
    makes the backward's dense gradient interleaved (dup = dgate + B)."""
    lib = m.lib
    assert fwd(m, act=m.mxq_act(2, 7.0, 0)) == 2                  # SReLU with an up pointer
    assert fwd(m, act=m.mxq_act(0, 7.0, 48)) == 2                 # block not a multiple of 32
    assert fwd(m, act=m.mxq_act(0, 7.0, -32)) == 2
    assert fwd(m, K=96, ldg=256, ldu=256, up=96 * 2, act=m.mxq_act(0, 7.0, 64)) == 2   # 96 % 64
    # interleaved gate / up views span 2K - B columns: a pitch of K is too small
    assert fwd(m, K=64, ldg=64, ldu=64, up=32 * 2, act=m.mxq_act(0, 7.0, 32)) == 2
    K, M = 64, 64
    row = m.mxq_mx_out(BASE + (4 << 24), 2 * K, BASE + (5 << 24), 2 * K // 32)

    def bwd(act, dgate, dup, up=fake(64), ldd=128):
        return lib.mxq_swiglu_quantize_bwd(ctypes.byref(act), M, K, fake(3 << 24), K, fake(0), 2 * K, up, 2 * K,
                                           None, None, dgate, ldd, dup, ldd, None, 1, ctypes.byref(row), None,
                                           None, 0, None)
    il = m.mxq_act(0, 7.0, 32)
    assert bwd(il, fake(1 << 28), fake((1 << 28) + 128)) == 2     # dup must be dgate + B elements
    srelu = m.mxq_act(2, 7.0, 0)
    assert bwd(srelu, fake(1 << 28), fake((1 << 28) + 128), up=None) == 2   # SReLU has no dup
    assert bwd(srelu, fake(1 << 28), None, up=fake(64)) == 2                # nor an up input
    assert bwd(m.mxq_act(2, 7.0, 32), fake(1 << 28), None, up=None) == 2    # nor an interleave


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


def test_quantize_noop_validation(m):
    """The no-op flag must be 4-byte aligned and must not overlap an output
    (it is an input); the rest is validated as mxq_quantize does."""
    lib = m.lib
    row = m.mxq_mx_out(BASE + (4 << 24), 64, BASE + (5 << 24), 2)
    assert lib.mxq_quantize_noop(64, 64, fake(0), 64, None, 1, ctypes.byref(row), None, fake((6 << 24) + 2),
                                 None) == 3
    assert lib.mxq_quantize_noop(64, 64, fake(0), 64, None, 1, ctypes.byref(row), None, fake((4 << 24) + 64),
                                 None) == 5
    assert lib.mxq_quantize_noop(64, 64, fake(0), 64, None, 1, ctypes.byref(row), None, fake((5 << 24) + 4),
                                 None) == 5
    assert lib.mxq_quantize_noop(64, 33, fake(0), 64, None, 1, ctypes.byref(row), None, fake(6 << 24), None) == 2


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


def test_gemm_output_alias_rejected(m):
    """An output overlapping an operand, an operand's scales or the offsets is
    refused with MXQ_ERR_ALIAS before anything is launched, in every mode (a
    persistent kernel would otherwise read tiles other workgroups overwrite)."""
    lib = m.lib
    for mode in (m.GEMM_NT, m.GEMM_NN, m.GEMM_TN):
        for target in (1 << 28, 2 << 28, 3 << 28, 4 << 28, 0):   # A, A scales, B, B scales, row_off
            a = gemm_args(m, mode)
            if mode == m.GEMM_NN:   # B per group (K x N), colwise scales (K/32 x N)
                a.B.ld, a.B.ld_scales, a.B.scale_gstride = 256, 256, 8 * 256
            a.out = BASE + target + (64 if target else 0)
            ws = fake(6 << 28) if mode == m.GEMM_TN else None
            assert lib.mxq_grouped_gemm(ctypes.byref(a), ws, 256 if ws else 0, None) == 5, (mode, target)
            assert "overlaps" in m.last_error()
    # the last group of a stacked B: out just inside its end, then just past it
    a = gemm_args(m, m.GEMM_NT)
    endB = (3 << 28) + (4 - 1) * 256 * 256 + (256 - 1) * 256 + 256
    a.out = BASE + endB - 16
    assert lib.mxq_grouped_gemm(ctypes.byref(a), None, 0, None) == 5


def test_fused_fc1_validation(m):
    """The fused FC1 epilogue takes bf16 NT launches with a bf16 output, N a
    multiple of 256, the weight's gate / up rows interleaved in blocks of 128,
    a SwiGLU kind, and block_off for colwise output; its activation outputs
    must not overlap the inputs or the bf16 product."""
    lib = m.lib

    def args(mode=None, N=256, dtype=None):
        a = gemm_args(m, m.GEMM_NT if mode is None else mode, N=N)
        a.A.dtype = a.B.dtype = m.DTYPE_BF16 if dtype is None else dtype
        a.A.scales = a.B.scales = None
        a.A.ld, a.B.ld, a.B.gstride = 256, 256, N * 256
        a.ld_out = N
        return a
    row = m.mxq_mx_out(BASE + (6 << 28), 128, BASE + (7 << 28), 4)
    il = m.mxq_act(0, 7.0, 128)

    def call(a, act=il, dirs=1, r=row):
        return lib.mxq_grouped_gemm_swiglu(ctypes.byref(a), ctypes.byref(act), None, dirs, ctypes.byref(r), None,
                                           None)
    assert call(args(), act=m.mxq_act(0, 7.0, 64)) == 2            # interleave block must be 128
    assert call(args(), act=m.mxq_act(2, 7.0, 128)) == 6           # SReLU: not a fused kind
    assert call(args(N=384)) == 2                                   # N % 256
    assert call(args(), dirs=2) == 1                                # colwise needs block_off
    assert call(args(), dirs=0) == 2
    bad = m.mxq_mx_out(BASE + (1 << 28) + 64, 128, BASE + (7 << 28), 4)
    assert call(args(), r=bad) == 5                                 # codes overlap A
    bad = m.mxq_mx_out(BASE + (5 << 28) + 64, 128, BASE + (7 << 28), 4)
    assert call(args(), r=bad) == 5                                 # codes overlap the bf16 product


def test_noalloc_backward_refuses_beyond_its_scratch(m):
    """The allocation-free backward checks its scratch size before it touches
    the device: 2^20 rows at K = 8192 need 64 MiB of dscale partials, more than
    the 16 MiB the library holds."""
    f = fake(0)
    st = m.lib.mxq_swiglu_quantize_bwd_noalloc(None, 1 << 20, 8192, f, 16384, f, 16384, f, 16384, None, None,
                                               None, 0, None, 0, fake(1 << 30), 1, None, None, None)
    assert st == 8 and "scratch" in m.last_error()


def fwd_dense(m, M=64, K=64, dirs=0, h=8 << 24, ldh=64, act=None, row=None):
    return m.lib.mxq_swiglu_fwd_bf16(
        None if act is None else ctypes.byref(act), M, K, fake(0), 128, fake(128), 128, None, None, dirs,
        None if row is None else ctypes.byref(row), None, None if h is None else fake(h), ldh, None)


def test_dense_forward_validation(m):
    """mxq_swiglu_fwd_bf16 (the activation recomputed as dense bf16): dirs may
    be 0 there (and only there), h is required, aligned, at least K wide and
    may not overlap an input; an empty call succeeds without h."""
    assert fwd(m, dirs=0) == 2                              # the quantizing forward needs a direction
    assert fwd_dense(m, dirs=4) == 2
    assert fwd_dense(m, h=None) == 1
    assert fwd_dense(m, h=(8 << 24) + 8) == 3               # misaligned h
    assert fwd_dense(m, ldh=68) == 3                        # pitch not 16 bytes
    assert fwd_dense(m, ldh=32) == 2                        # ld_h < K
    assert fwd_dense(m, h=64) == 5                          # h overlaps gate
    row = m.mxq_mx_out(BASE + (8 << 24) + 64, 64, BASE + (5 << 24), 2)
    assert fwd_dense(m, dirs=1, row=row) == 5               # codes overlap h
    assert fwd_dense(m, M=0, h=None) == 0
    act = m.mxq_act(m.ACT_SRELU, 0.0, 0)
    assert m.lib.mxq_swiglu_fwd_bf16(ctypes.byref(act), 64, 64, fake(0), 128, fake(128), 128, None, None, 0, None,
                                     None, fake(8 << 24), 64, None) == 2   # SReLU is unary: up must be NULL


def test_gemm_bf16_every_mode_validates(m):
    """bf16 operands are accepted in every mode (NN and TN read them strided
    along the contraction); bf16 TN needs no block_off.  Only validation runs
    here: the calls stop at an alias before anything is launched."""
    lib = m.lib
    bf = m.DTYPE_BF16
    for mode in (m.GEMM_NN, m.GEMM_TN):
        a = gemm_args(m, mode)
        a.A.dtype = a.B.dtype = bf
        a.A.scales = a.B.scales = None
        a.block_off = None
        if mode == m.GEMM_NN:
            a.B.ld, a.B.gstride = 256, 256 * 256
        a.out = BASE + (1 << 28) + 64                       # on top of A
        ws = fake(6 << 28) if mode == m.GEMM_TN else None
        assert lib.mxq_grouped_gemm(ctypes.byref(a), ws, 256 if ws else 0, None) == 5, mode
        assert "overlaps" in m.last_error()


def test_kblock_gemm_validation(m):
    """K-blocked operands (kblock_plane > 0): only the operands read along
    the contraction (A of NT / NN, B of NT), with 64-byte plane rows (ld 64
    codes or 32 bf16), K a multiple of 64 bytes, the plane a multiple of 16
    holding every row; their footprint (planes x plane) counts in the overlap
    check."""
    lib = m.lib

    def args(mode=m.GEMM_NT, ka=True, kb=False, K=256):
        a = gemm_args(m, mode, K=K)
        if mode == m.GEMM_NN:
            a.B.ld, a.B.ld_scales, a.B.scale_gstride = 256, 256, 8 * 256
        if ka:
            a.A.ld, a.A.kblock_plane = 64, 256 * 64
        if kb:
            a.B.ld, a.B.gstride, a.B.kblock_plane = 64, 256 * 64, 4 * 256 * 64
        return a

    def call(a):
        return lib.mxq_grouped_gemm(ctypes.byref(a), None, 0, None)
    bad = args()
    bad.A.ld = 256                      # a K-blocked operand has ld 64
    assert call(bad) == 2
    bad = args(K=96)                    # K a multiple of 64
    bad.A.ld_scales = bad.B.ld_scales = 3
    assert call(bad) == 2
    bad = args()
    bad.A.kblock_plane = 255 * 64       # the plane must hold all M rows
    assert call(bad) == 2
    bad = args()
    bad.A.kblock_plane = 256 * 64 + 8   # 16-byte multiple
    assert call(bad) == 3
    bad = args(kb=True)
    bad.B.kblock_plane = 4 * 256 * 64 - 16   # the plane must hold all G x N rows
    assert call(bad) == 2
    bad = args(kb=True)
    bad.B.gstride = 255 * 64            # groups of N rows do not overlap
    assert call(bad) == 2
    nn = args(m.GEMM_NN, ka=False)
    nn.B.kblock_plane = 1 << 20         # B of NN runs along N: not K-blocked
    assert call(nn) == 6
    tn = gemm_args(m, m.GEMM_TN)
    tn.A.kblock_plane = 1 << 20
    assert lib.mxq_grouped_gemm(ctypes.byref(tn), fake(6 << 28), 256, None) == 6
    bf = args()
    bf.A.dtype = bf.B.dtype = m.DTYPE_BF16
    bf.A.scales = bf.B.scales = None
    bf.A.ld = 64                        # a bf16 plane row is 32 elements (64 bytes)
    assert call(bf) == 2
    # the output just inside the last plane of A (plane 3 starts at 3 x 16384)
    a = args()
    a.out = BASE + (1 << 28) + 3 * 256 * 64 + 256 * 64 - 16
    assert call(a) == 5


def test_kblock_mx_out_validation(m):
    """K-blocked rowwise codes (mxq_mx_out.kblock_plane): ld_codes 64, a
    multiple of 64 columns, the plane a 16-byte multiple holding every row,
    under 2^31 bytes in all; colwise codes and the fused FC1 epilogue stay
    row-major; the blocked footprint counts in the overlap check."""
    lib = m.lib

    def q(M=64, K=128, ld_codes=64, plane=64 * 64, dirs=1, col_plane=0, x=0):
        row = m.mxq_mx_out(BASE + (4 << 24), ld_codes, BASE + (5 << 24), K // 32, plane)
        col = m.mxq_mx_out(BASE + (6 << 24), K, BASE + (7 << 24), K, col_plane)
        return lib.mxq_quantize(M, K, fake(x), K, None, dirs, ctypes.byref(row) if dirs & 1 else None,
                                ctypes.byref(col) if dirs & 2 else None, None)
    assert q(ld_codes=128) == 2              # blocked codes have ld_codes 64
    assert q(K=96) == 2                      # a multiple of 64 columns
    assert q(plane=63 * 64) == 2             # the plane holds all M rows
    assert q(plane=64 * 64 + 4) == 3         # 16-byte multiple
    assert q(M=1 << 22, K=1 << 13, plane=(1 << 22) * 64) == 4   # 128 planes of 256 MiB: past 2^31 bytes
    assert q(dirs=2, col_plane=64 * 64) == 6  # colwise codes are row-major
    # an input inside the last plane of the blocked codes (plane 1 of 2)
    assert q(x=(4 << 24) + 64 * 64 + 32) == 5
    # the fused FC1 epilogue writes row-major codes
    a = gemm_args(m, m.GEMM_NT, N=256)
    a.A.dtype = a.B.dtype = m.DTYPE_BF16
    a.A.scales = a.B.scales = None
    a.A.ld, a.B.ld, a.B.gstride, a.ld_out = 256, 256, 256 * 256, 256
    row = m.mxq_mx_out(BASE + (6 << 28), 64, BASE + (7 << 28), 4, 64 * 256)
    assert lib.mxq_grouped_gemm_swiglu(ctypes.byref(a), ctypes.byref(m.mxq_act(0, 7.0, 128)), None, 1,
                                       ctypes.byref(row), None, None) == 6
