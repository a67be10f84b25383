"""Python view of the CPU oracle (mxq_oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never does, and the oracle shares no code
with it.  Every function takes and returns plain numpy arrays:
bf16 values travel as uint16 bit patterns, E4M3 codes and E8M0 scales as uint8.

Function map (the C file cites the page passage each one follows):
  e8m0_from_amax, double_to_e4m3, e4m3_to_double, double_to_bf16,
  bf16_to_double              -- number formats and the RCEIL scale rule
  near_bf16_tie               -- boundary closeness of an exact value
  splits_to_offsets           -- exclusive prefix sums of split sizes
  mx_quantize                 -- the standalone 1x32 / 32x1 block quantizer
  swiglu_fwd / swiglu_bwd     -- the row-scaled (clamped) SwiGLU and its gradient
  swiglu_quantize_fwd/_bwd    -- activation followed by the block quantizer
  srelu_fwd / srelu_bwd       -- the row-scaled SReLU (squared ReLU) and its gradient
  srelu_quantize_fwd/_bwd     -- SReLU followed by the block quantizer
  glu_split / glu_join        -- gate/up interleaved in blocks of B columns
  swiglu_quantize_bwd_interleaved -- the backward in the interleaved layout
  grouped_gemm                -- brute-force per-group GEMM, fp32 accumulation
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxq_oracle.so")
_lib = None

ROW = 1
COL = 2
SWIGLU = 0
CLAMPED_SWIGLU = 1


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


class _Operand(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("data", ctypes.c_void_p),
                ("gstride", ctypes.c_int64), ("ld_i", ctypes.c_int64),
                ("ld_k", ctypes.c_int64), ("scales", ctypes.c_void_p),
                ("sgstride", ctypes.c_int64), ("sld_i", ctypes.c_int64),
                ("sld_k", ctypes.c_int64)]


def _declare(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = ctypes.c_double
    lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_e4m3_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_to_double.restype = ctypes.c_double
    lib.oracle_double_to_e4m3.argtypes = [ctypes.c_double]
    lib.oracle_double_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_e8m0_to_double.argtypes = [ctypes.c_uint8]
    lib.oracle_e8m0_to_double.restype = ctypes.c_double
    lib.oracle_e8m0_from_amax.argtypes = [ctypes.c_double]
    lib.oracle_e8m0_from_amax.restype = ctypes.c_uint8
    lib.oracle_near_bf16_tie.argtypes = [ctypes.c_double]
    lib.oracle_near_bf16_tie.restype = ctypes.c_int
    lib.oracle_splits_to_offsets.argtypes = [P, I64, P, P]
    lib.oracle_splits_to_offsets.restype = None
    lib.oracle_mx_quantize.argtypes = [I64, I64, P, I64, I64, P, ctypes.c_uint32, P, P, P, P]
    lib.oracle_mx_quantize.restype = None
    lib.oracle_swiglu_fwd.argtypes = [ctypes.c_int, ctypes.c_double, I64, I64, P, I64, P, I64,
                                      P, P, P]
    lib.oracle_swiglu_fwd.restype = None
    lib.oracle_swiglu_bwd.argtypes = [ctypes.c_int, ctypes.c_double, I64, I64, P, I64, P, I64,
                                      P, I64, P, P, I64, P, I64, P, P, P]
    lib.oracle_swiglu_bwd.restype = None
    lib.oracle_srelu_fwd.argtypes = [I64, I64, P, I64, P, P, P]
    lib.oracle_srelu_fwd.restype = None
    lib.oracle_srelu_bwd.argtypes = [I64, I64, P, I64, P, I64, P, P, I64, P, P, P]
    lib.oracle_srelu_bwd.restype = None
    lib.oracle_grouped_gemm.argtypes = [ctypes.c_int, I64, P, I64, I64, I64,
                                        ctypes.POINTER(_Operand), ctypes.POINTER(_Operand),
                                        P, ctypes.c_int, I64, I64, ctypes.c_int]
    lib.oracle_grouped_gemm.restype = None


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats ---

def bf16_to_double(bits):
    lib = _load()
    bits = np.asarray(bits, dtype=np.uint16)
    return np.array([lib.oracle_bf16_to_double(int(b)) for b in bits.ravel()]).reshape(bits.shape)


def double_to_bf16(x):
    lib = _load()
    x = np.asarray(x, dtype=np.float64)
    return np.array([lib.oracle_double_to_bf16(float(v)) for v in x.ravel()],
                    dtype=np.uint16).reshape(x.shape)


def e4m3_to_double(codes):
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    return np.array([lib.oracle_e4m3_to_double(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def double_to_e4m3(y):
    lib = _load()
    y = np.asarray(y, dtype=np.float64)
    return np.array([lib.oracle_double_to_e4m3(float(v)) for v in y.ravel()],
                    dtype=np.uint8).reshape(y.shape)


def e8m0_to_double(e):
    lib = _load()
    e = np.asarray(e, dtype=np.uint8)
    return np.array([lib.oracle_e8m0_to_double(int(v)) for v in e.ravel()]).reshape(e.shape)


def e8m0_from_amax(amax):
    lib = _load()
    amax = np.asarray(amax, dtype=np.float64)
    return np.array([lib.oracle_e8m0_from_amax(float(v)) for v in amax.ravel()],
                    dtype=np.uint8).reshape(amax.shape)


def near_bf16_tie(t):
    """1 where the exact value t lies within 2 binary32 ulps (of t) of a bf16
    rounding tie (the boundary-closeness flag of the parity rules)."""
    lib = _load()
    t = np.asarray(t, dtype=np.float64)
    return np.array([lib.oracle_near_bf16_tie(float(v)) for v in t.ravel()],
                    dtype=np.uint8).reshape(t.shape)


# ---------------------------------------------------------------- offsets ---

def splits_to_offsets(splits):
    lib = _load()
    s = _c(splits, np.int64)
    G = s.shape[0]
    row_off = np.zeros(G + 1, np.int64)
    block_off = np.zeros(G + 1, np.int64)
    lib.oracle_splits_to_offsets(_ptr(s), G, _ptr(row_off), _ptr(block_off))
    return row_off, block_off


# -------------------------------------------------------------- quantizer ---

def colwise_scale_rows(M, row_off=None):
    if row_off is None:
        return (M + 31) // 32
    splits = np.diff(np.asarray(row_off, np.int64))
    return int(((splits + 31) // 32).sum())


def mx_quantize(x, dirs=ROW | COL, row_off=None):
    """Block-quantize an (M, K) bf16 matrix (uint16 bits, any row stride).

    Returns (row_codes, col_codes, row_scales, col_scales); a disabled
    direction comes back zero-sized.
    """
    lib = _load()
    x = np.asarray(x, dtype=np.uint16)
    M, K = x.shape
    if x.strides[1] != 2:
        x = np.ascontiguousarray(x)
    ldx = x.strides[0] // 2 if M > 0 else K
    rc = np.zeros((M, K) if dirs & ROW else (0, 0), np.uint8)
    rs = np.zeros((M, K // 32) if dirs & ROW else (0, 0), np.uint8)
    nsr = colwise_scale_rows(M, row_off)
    cc = np.zeros((M, K) if dirs & COL else (0, 0), np.uint8)
    cs = np.zeros((nsr, K) if dirs & COL else (0, 0), np.uint8)
    ro = None if row_off is None else _c(row_off, np.int64)
    G = 1 if ro is None else ro.shape[0] - 1
    lib.oracle_mx_quantize(M, K, _ptr(x), ldx, G, _ptr(ro), dirs,
                           _ptr(rc), _ptr(rs), _ptr(cc), _ptr(cs))
    return rc, cc, rs, cs


# ------------------------------------------------------------- activation ---

def _ld(a):
    return a.strides[0] // a.itemsize if a.shape[0] > 0 else a.shape[1]


def _rowview(a, dtype):
    a = np.asarray(a)
    assert a.dtype == dtype
    if a.ndim != 2 or a.strides[1] != a.itemsize:
        a = np.ascontiguousarray(a)
    return a


def swiglu_fwd(gate, up, scale=None, kind=SWIGLU, limit=7.0, want_close=False):
    """h = bf16(bf16(silu(g)) * u * s); returns h (uint16) and, optionally,
    the boundary-closeness flags (uint8, bit0 silu, bit1 h)."""
    lib = _load()
    g = _rowview(gate, np.uint16)
    u = _rowview(up, np.uint16)
    M, K = g.shape
    sc = None if scale is None else _c(scale, np.float32)
    h = np.zeros((M, K), np.uint16)
    close = np.zeros((M, K), np.uint8) if want_close else None
    lib.oracle_swiglu_fwd(kind, limit, M, K, _ptr(g), _ld(g), _ptr(u), _ld(u),
                          _ptr(sc), _ptr(h), _ptr(close))
    return (h, close) if want_close else h


def swiglu_bwd(grad, gate, up, scale=None, kind=SWIGLU, limit=7.0, want_close=False):
    """Returns (dgate, dup, dscale[, close, dscale_tol])."""
    lib = _load()
    dh = _rowview(grad, np.uint16)
    g = _rowview(gate, np.uint16)
    u = _rowview(up, np.uint16)
    M, K = g.shape
    sc = None if scale is None else _c(scale, np.float32)
    dg = np.zeros((M, K), np.uint16)
    du = np.zeros((M, K), np.uint16)
    ds = np.zeros(M, np.float32)
    close = np.zeros((M, 2 * K), np.uint8) if want_close else None
    tol = np.zeros(M, np.float64) if want_close else None
    lib.oracle_swiglu_bwd(kind, limit, M, K, _ptr(dh), _ld(dh), _ptr(g), _ld(g),
                          _ptr(u), _ld(u), _ptr(sc), _ptr(dg), K, _ptr(du), K,
                          _ptr(ds), _ptr(close), _ptr(tol))
    if want_close:
        return dg, du, ds, close, tol
    return dg, du, ds


def swiglu_quantize_fwd(gate, up, scale=None, dirs=ROW | COL, row_off=None,
                        kind=SWIGLU, limit=7.0, want_close=False):
    """The unfused definition: activation, then the standalone quantizer.
    Returns (row_codes, col_codes, row_scales, col_scales, h[, close])."""
    r = swiglu_fwd(gate, up, scale, kind, limit, want_close)
    h, close = r if want_close else (r, None)
    q = mx_quantize(h, dirs, row_off)
    return (*q, h, close) if want_close else (*q, h)


def swiglu_quantize_bwd(grad, gate, up, scale=None, dirs=ROW | COL, row_off=None,
                        kind=SWIGLU, limit=7.0, want_close=False):
    """Returns (row_codes, col_codes, row_scales, col_scales, dgate, dup, dscale
    [, close, dscale_tol]); the codes cover the (M, 2K) matrix [dgate | dup]."""
    r = swiglu_bwd(grad, gate, up, scale, kind, limit, want_close)
    dg, du, ds = r[:3]
    q = mx_quantize(np.concatenate([dg, du], axis=1), dirs, row_off)
    out = (*q, dg, du, ds)
    return (*out, r[3], r[4]) if want_close else out


def srelu_fwd(x, scale=None, want_close=False):
    """h = bf16(bf16(max(x, 0)^2) * s); returns h (uint16) and, optionally, the
    boundary-closeness flags (uint8, bit0 the square, bit1 h)."""
    lib = _load()
    xv = _rowview(x, np.uint16)
    M, K = xv.shape
    sc = None if scale is None else _c(scale, np.float32)
    h = np.zeros((M, K), np.uint16)
    close = np.zeros((M, K), np.uint8) if want_close else None
    lib.oracle_srelu_fwd(M, K, _ptr(xv), _ld(xv), _ptr(sc), _ptr(h), _ptr(close))
    return (h, close) if want_close else h


def srelu_bwd(grad, x, scale=None, want_close=False):
    """Returns (dx, dscale[, close, dscale_tol]) with dx = bf16(dh*s*2*max(x,0))
    and dscale = fp32(sum_j dh * bf16(max(x,0)^2))."""
    lib = _load()
    dh = _rowview(grad, np.uint16)
    xv = _rowview(x, np.uint16)
    M, K = xv.shape
    sc = None if scale is None else _c(scale, np.float32)
    dx = np.zeros((M, K), np.uint16)
    ds = np.zeros(M, np.float32)
    close = np.zeros((M, K), np.uint8) if want_close else None
    tol = np.zeros(M, np.float64) if want_close else None
    lib.oracle_srelu_bwd(M, K, _ptr(dh), _ld(dh), _ptr(xv), _ld(xv), _ptr(sc), _ptr(dx), K, _ptr(ds),
                         _ptr(close), _ptr(tol))
    return (dx, ds, close, tol) if want_close else (dx, ds)


def srelu_quantize_fwd(x, scale=None, dirs=ROW | COL, row_off=None, want_close=False):
    """Row-scaled SReLU, then the standalone quantizer.
    Returns (row_codes, col_codes, row_scales, col_scales, h[, close])."""
    r = srelu_fwd(x, scale, want_close)
    h, close = r if want_close else (r, None)
    q = mx_quantize(h, dirs, row_off)
    return (*q, h, close) if want_close else (*q, h)


def srelu_quantize_bwd(grad, x, scale=None, dirs=ROW | COL, row_off=None, want_close=False):
    """Returns (row_codes, col_codes, row_scales, col_scales, dx, dscale
    [, close, dscale_tol]); the codes cover the (M, K) matrix dx."""
    r = srelu_bwd(grad, x, scale, want_close)
    q = mx_quantize(r[0], dirs, row_off)
    return (*q, *r)


# ------------------------------------------------------- GLU interleaving ---
# A gated input may hold gate and up interleaved in blocks of B columns:
# columns [2Bi, 2Bi + B) are gate columns [Bi, Bi + B) and [2Bi + B, 2Bi + 2B)
# are the matching up columns (page "Activation + GroupedLinear Fusion for MOE
# and other MOE optimizations", Important Files Changed: the GLU interleave
# reshaping moves into the scaled SwiGLU kernels; the pages give no block
# size, so it is a parameter).  B = K is the plain packed [gate | up].

def glu_split(packed, B):
    """(M, 2K) interleaved with block B -> (gate, up), each (M, K)."""
    p = np.asarray(packed)
    M, K2 = p.shape
    K = K2 // 2
    assert K % B == 0
    blocks = p.reshape(M, K // B, 2, B)
    return (np.ascontiguousarray(blocks[:, :, 0, :].reshape(M, K)),
            np.ascontiguousarray(blocks[:, :, 1, :].reshape(M, K)))


def glu_join(gate, up, B):
    """(gate, up) (M, K) -> the (M, 2K) layout interleaved with block B."""
    g, u = np.asarray(gate), np.asarray(up)
    M, K = g.shape
    assert K % B == 0 and u.shape == g.shape
    out = np.empty((M, K // B, 2, B), g.dtype)
    out[:, :, 0, :] = g.reshape(M, K // B, B)
    out[:, :, 1, :] = u.reshape(M, K // B, B)
    return out.reshape(M, 2 * K)


def swiglu_quantize_bwd_interleaved(grad, packed, B, scale=None, dirs=ROW | COL, row_off=None,
                                    kind=SWIGLU, limit=7.0, want_close=False):
    """The backward on a gated input interleaved with block B: the gradient
    [dgate | dup] and its MXFP8 form take the input's interleaved layout.
    Returns (row_codes, col_codes, row_scales, col_scales, d_packed, dscale
    [, close, dscale_tol]) with d_packed (M, 2K) interleaved."""
    g, u = glu_split(packed, B)
    r = swiglu_bwd(grad, g, u, scale, kind, limit, want_close)
    dg, du, ds = r[:3]
    d = glu_join(dg, du, B)
    q = mx_quantize(d, dirs, row_off)
    out = (*q, d, ds)
    if want_close:
        cg, cu = r[3][:, :dg.shape[1]], r[3][:, dg.shape[1]:]
        out = (*out, glu_join(cg, cu, B), r[4])
    return out


# ----------------------------------------------------------- grouped GEMM ---

class Operand:
    """A GEMM operand for the oracle.

    dtype 'bf16' (data uint16) or 'mxfp8' (data uint8 codes + uint8 scales).
    Element (i, k) of group g is data.flat[g*gstride + i*ld_i + k*ld_k]; its
    scale is scales.flat[g*sgstride + sblock*sld_k + i*sld_i].
    """

    def __init__(self, dtype, data, gstride, ld_i, ld_k, scales=None,
                 sgstride=0, sld_i=0, sld_k=0):
        self.dtype = dtype
        self.data = np.ascontiguousarray(data)
        self.scales = None if scales is None else np.ascontiguousarray(scales, np.uint8)
        self.s = _Operand(0 if dtype == "bf16" else 1, self.data.ctypes.data,
                          gstride, ld_i, ld_k,
                          None if self.scales is None else self.scales.ctypes.data,
                          sgstride, sld_i, sld_k)


def grouped_gemm(mode, row_off, Mdim, N, Kdim, A, B, out_dtype="bf16", out=None,
                 accumulate=False):
    """mode 'm' (M-grouped): C (R, N), C[r,n] = sum_k A(r,k) B_g(n,k).
    mode 'k' (K-grouped): C (G, Mdim, N), C_g[m,n] = sum_{r in g} A(m,r) B(n,r).
    Returns C as uint16 bf16 bits or float32."""
    lib = _load()
    ro = _c(row_off, np.int64)
    G = ro.shape[0] - 1
    dt = np.uint16 if out_dtype == "bf16" else np.float32
    if mode == "m":
        shape = (int(ro[-1]), N)
        ldc, ogs = N, 0
    else:
        shape = (G, Mdim, N)
        ldc, ogs = N, Mdim * N
    if out is None:
        out = np.zeros(shape, dt)
    else:
        assert out.shape == shape and out.dtype == dt and out.flags.c_contiguous
    lib.oracle_grouped_gemm(0 if mode == "m" else 1, G, _ptr(ro), Mdim, N, Kdim,
                            ctypes.byref(A.s), ctypes.byref(B.s), _ptr(out),
                            0 if out_dtype == "bf16" else 1, ldc, ogs, int(accumulate))
    return out
