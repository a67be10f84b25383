"""Python binding of libmxq, the MI355X (gfx950) library for the fused
row-scaled SwiGLU + MXFP8 quantization path and the grouped GEMM over experts.

The functions named mxq_* mirror the C ABI in include/mxq.h one to one: they
only marshal torch tensors (device memory) into pointers, leading dimensions
and descriptor structs, and return the mxq_status.  Every computation runs in
the HIP kernels of libmxq.so; nothing here computes on the host.

The friendlier helpers (splits_to_offsets, swiglu_quantize_fwd, ...) allocate
the outputs with torch and call the mxq_* functions; they raise MxqError on a
non-zero status.

Importing this package loads libmxq.so and fails loudly if it is missing (run
`python -m swiglu_mxfp8_quant_amd.build`).  There is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmxq.so")

MXQ_OK = 0
STATUS = {0: "MXQ_OK", 1: "MXQ_ERR_NULL", 2: "MXQ_ERR_SHAPE", 3: "MXQ_ERR_ALIGN",
          4: "MXQ_ERR_OVERFLOW", 5: "MXQ_ERR_ALIAS", 6: "MXQ_ERR_UNSUPPORTED",
          7: "MXQ_ERR_HIP", 8: "MXQ_ERR_WORKSPACE"}
ROWWISE = 1
COLWISE = 2
ACT_SWIGLU = 0
ACT_CLAMPED_SWIGLU = 1
ACT_SRELU = 2
DTYPE_BF16 = 0
DTYPE_MXFP8 = 1
DTYPE_F32 = 2
GEMM_NT = 0
GEMM_NN = 1
GEMM_TN = 2

# every symbol include/mxq.h declares
EXPORTS = [
    "mxq_splits_to_offsets", "mxq_swiglu_quantize_fwd", "mxq_swiglu_fwd_bf16", "mxq_swiglu_quantize_bwd_workspace",
    "mxq_swiglu_quantize_bwd", "mxq_swiglu_quantize_bwd_noalloc", "mxq_quantize", "mxq_quantize_noop",
    "mxq_grouped_gemm_workspace",
    "mxq_grouped_gemm", "mxq_grouped_gemm_swiglu",
    "mxq_status_string", "mxq_last_error_message", "mxq_version",
]


class MxqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class mxq_act(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("limit", ctypes.c_float), ("glu_interleave", ctypes.c_int32)]


class mxq_groups(ctypes.Structure):
    _fields_ = [("G", ctypes.c_int64), ("row_off", ctypes.c_void_p), ("block_off", ctypes.c_void_p)]


class mxq_mx_out(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("ld_codes", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("ld_scales", ctypes.c_int64),
                ("kblock_plane", ctypes.c_int64)]


class mxq_operand(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("data", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("gstride", ctypes.c_int64), ("scales", ctypes.c_void_p),
                ("ld_scales", ctypes.c_int64), ("scale_gstride", ctypes.c_int64),
                ("kblock_plane", ctypes.c_int64)]


class mxq_gemm_args(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("G", ctypes.c_int64), ("row_off", ctypes.c_void_p),
                ("block_off", ctypes.c_void_p), ("M", ctypes.c_int64), ("N", ctypes.c_int64),
                ("K", ctypes.c_int64), ("rows", ctypes.c_int64), ("A", mxq_operand),
                ("B", mxq_operand), ("out_dtype", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("ld_out", ctypes.c_int64), ("out_gstride", ctypes.c_int64),
                ("accumulate", ctypes.c_int32), ("max_workgroups", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmxq.so not built at {LIB_PATH}; run python -m swiglu_mxfp8_quant_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    P, I64, U32, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32
    sig = {
        "mxq_splits_to_offsets": [P, I64, P, P, P, P],
        "mxq_swiglu_quantize_fwd": [ctypes.POINTER(mxq_act), I64, I64, P, I64, P, I64, P,
                                    ctypes.POINTER(mxq_groups), U32, ctypes.POINTER(mxq_mx_out),
                                    ctypes.POINTER(mxq_mx_out), P],
        "mxq_swiglu_fwd_bf16": [ctypes.POINTER(mxq_act), I64, I64, P, I64, P, I64, P,
                                ctypes.POINTER(mxq_groups), U32, ctypes.POINTER(mxq_mx_out),
                                ctypes.POINTER(mxq_mx_out), P, I64, P],
        "mxq_swiglu_quantize_bwd_workspace": [I64, I64, U32, ctypes.POINTER(ctypes.c_size_t)],
        "mxq_swiglu_quantize_bwd": [ctypes.POINTER(mxq_act), I64, I64, P, I64, P, I64, P, I64, P,
                                    ctypes.POINTER(mxq_groups), P, I64, P, I64, P, U32,
                                    ctypes.POINTER(mxq_mx_out), ctypes.POINTER(mxq_mx_out), P,
                                    ctypes.c_size_t, P],
        "mxq_swiglu_quantize_bwd_noalloc": [ctypes.POINTER(mxq_act), I64, I64, P, I64, P, I64, P, I64, P,
                                            ctypes.POINTER(mxq_groups), P, I64, P, I64, P, U32,
                                            ctypes.POINTER(mxq_mx_out), ctypes.POINTER(mxq_mx_out), P],
        "mxq_quantize": [I64, I64, P, I64, ctypes.POINTER(mxq_groups), U32,
                         ctypes.POINTER(mxq_mx_out), ctypes.POINTER(mxq_mx_out), P],
        "mxq_quantize_noop": [I64, I64, P, I64, ctypes.POINTER(mxq_groups), U32,
                              ctypes.POINTER(mxq_mx_out), ctypes.POINTER(mxq_mx_out), P, P],
        "mxq_grouped_gemm_workspace": [ctypes.POINTER(mxq_gemm_args), ctypes.POINTER(ctypes.c_size_t)],
        "mxq_grouped_gemm": [ctypes.POINTER(mxq_gemm_args), P, ctypes.c_size_t, P],
        "mxq_grouped_gemm_swiglu": [ctypes.POINTER(mxq_gemm_args), ctypes.POINTER(mxq_act), P, U32,
                                    ctypes.POINTER(mxq_mx_out), ctypes.POINTER(mxq_mx_out), P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = I32
    lib.mxq_status_string.argtypes = [I32]
    lib.mxq_status_string.restype = ctypes.c_char_p
    lib.mxq_last_error_message.argtypes = []
    lib.mxq_last_error_message.restype = ctypes.c_char_p
    lib.mxq_version.argtypes = []
    lib.mxq_version.restype = ctypes.c_char_p
    return lib


lib = _load()


def version() -> str:
    return lib.mxq_version().decode()


def last_error() -> str:
    return lib.mxq_last_error_message().decode()


def check(status: int) -> None:
    if status != MXQ_OK:
        raise MxqError(status, last_error())


# ------------------------------------------------------------- marshalling ---

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t):
    """Row pitch (elements) of a 2-D view with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D view with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else t.shape[1] if t.stride(0) < t.shape[1] else t.stride(0)


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)


def _hold(t, stream):
    """Keep a temporary device buffer (a workspace) from being handed out again
    before the work queued on `stream` has used it (torch frees it on return;
    its caching allocator only orders reuse on the current stream).  With a raw
    stream handle the caller must keep the current stream ordered with it."""
    if t is not None and stream is not None and not isinstance(stream, int):
        t.record_stream(stream)


def make_act(kind=ACT_SWIGLU, limit=7.0, interleave=0):
    return mxq_act(kind, limit, interleave)


def make_groups(row_off=None, block_off=None):
    if row_off is None:
        return None
    return mxq_groups(row_off.numel() - 1, row_off.data_ptr(),
                      None if block_off is None else block_off.data_ptr())


def make_mx_out(codes, scales):
    if codes is None:
        return None
    if isinstance(codes, KBlocked):
        return mxq_mx_out(codes.data.data_ptr(), 64, scales.data_ptr(), _ld(scales), codes.plane)
    return mxq_mx_out(codes.data_ptr(), _ld(codes), scales.data_ptr(), _ld(scales), 0)


def _byref(x):
    return None if x is None else ctypes.byref(x)


# ------------------------------------------------------------ C-ABI mirror ---

def mxq_splits_to_offsets(splits, row_off, block_off=None, err_flag=None, stream=None):
    return lib.mxq_splits_to_offsets(_ptr(splits), splits.numel(), _ptr(row_off), _ptr(block_off),
                                     _ptr(err_flag), _stream(stream))


def mxq_swiglu_quantize_fwd(act, gate, up, row_scale, groups, dirs, row_out, col_out, stream=None):
    M, K = gate.shape
    return lib.mxq_swiglu_quantize_fwd(_byref(act), M, K, _ptr(gate), _ld(gate), _ptr(up),
                                       _ld(up) if up is not None else 0,
                                       _ptr(row_scale), _byref(groups), dirs, _byref(row_out),
                                       _byref(col_out), _stream(stream))


def mxq_swiglu_fwd_bf16(act, gate, up, row_scale, groups, dirs, row_out, col_out, h, stream=None):
    M, K = gate.shape
    return lib.mxq_swiglu_fwd_bf16(_byref(act), M, K, _ptr(gate), _ld(gate), _ptr(up),
                                   _ld(up) if up is not None else 0,
                                   _ptr(row_scale), _byref(groups), dirs, _byref(row_out),
                                   _byref(col_out), _ptr(h), _ld(h) if h is not None else 0, _stream(stream))


def mxq_swiglu_quantize_bwd_workspace(M, K, dirs):
    n = ctypes.c_size_t(0)
    check(lib.mxq_swiglu_quantize_bwd_workspace(M, K, dirs, ctypes.byref(n)))
    return n.value


def mxq_swiglu_quantize_bwd(act, grad, gate, up, row_scale, groups, dgate, dup, dscale, dirs,
                            row_out, col_out, ws, stream=None):
    M, K = gate.shape
    return lib.mxq_swiglu_quantize_bwd(
        _byref(act), M, K, _ptr(grad), _ld(grad), _ptr(gate), _ld(gate), _ptr(up),
        _ld(up) if up is not None else 0, _ptr(row_scale), _byref(groups), _ptr(dgate),
        _ld(dgate) if dgate is not None else 0, _ptr(dup), _ld(dup) if dup is not None else 0, _ptr(dscale),
        dirs, _byref(row_out), _byref(col_out), _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))


def mxq_swiglu_quantize_bwd_noalloc(act, grad, gate, up, row_scale, groups, dgate, dup, dscale, dirs,
                                    row_out, col_out, stream=None):
    M, K = gate.shape
    return lib.mxq_swiglu_quantize_bwd_noalloc(
        _byref(act), M, K, _ptr(grad), _ld(grad), _ptr(gate), _ld(gate), _ptr(up), _ld(up) if up is not None else 0,
        _ptr(row_scale), _byref(groups), _ptr(dgate), _ld(dgate) if dgate is not None else 0,
        _ptr(dup), _ld(dup) if dup is not None else 0, _ptr(dscale), dirs, _byref(row_out),
        _byref(col_out), _stream(stream))


def mxq_quantize(x, groups, dirs, row_out, col_out, stream=None):
    M, K = x.shape
    return lib.mxq_quantize(M, K, _ptr(x), _ld(x), _byref(groups), dirs, _byref(row_out),
                            _byref(col_out), _stream(stream))


def mxq_quantize_noop(x, groups, dirs, row_out, col_out, noop_flag, stream=None):
    M, K = x.shape
    return lib.mxq_quantize_noop(M, K, _ptr(x), _ld(x), _byref(groups), dirs, _byref(row_out),
                                 _byref(col_out), _ptr(noop_flag), _stream(stream))


def mxq_grouped_gemm_workspace(args):
    n = ctypes.c_size_t(0)
    check(lib.mxq_grouped_gemm_workspace(ctypes.byref(args), ctypes.byref(n)))
    return n.value


def mxq_grouped_gemm_swiglu(args, act, row_scale, dirs, row_out, col_out, stream=None):
    return lib.mxq_grouped_gemm_swiglu(ctypes.byref(args), _byref(act), _ptr(row_scale), dirs, _byref(row_out),
                                       _byref(col_out), _stream(stream))


def mxq_grouped_gemm(args, ws=None, stream=None):
    return lib.mxq_grouped_gemm(ctypes.byref(args), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))


# ---------------------------------------------------------------- helpers ---

def colwise_scale_rows_bound(M, G=0):
    return (M + 31) // 32 + (G if G else 0)


def splits_to_offsets(splits, stream=None):
    """(row_off, block_off, err_flag) int64 / int32 device tensors."""
    import torch
    G = splits.numel()
    row_off = torch.empty(G + 1, dtype=torch.int64, device=splits.device)
    block_off = torch.empty(G + 1, dtype=torch.int64, device=splits.device)
    err = torch.zeros(1, dtype=torch.int32, device=splits.device)
    check(mxq_splits_to_offsets(splits, row_off, block_off, err, stream))
    return row_off, block_off, err


def _alloc_mx(M, K, dirs, n_col_blocks, device, kblock=False):
    import torch
    if kblock and dirs & ROWWISE:
        rc = KBlocked.empty((M, K), device)
    else:
        rc = torch.empty((M, K) if dirs & ROWWISE else (0, 0), dtype=torch.uint8, device=device)
    rs = torch.empty((M, K // 32) if dirs & ROWWISE else (0, 0), dtype=torch.uint8, device=device)
    cc = torch.empty((M, K) if dirs & COLWISE else (0, 0), dtype=torch.uint8, device=device)
    cs = torch.empty((n_col_blocks, K) if dirs & COLWISE else (0, 0), dtype=torch.uint8, device=device)
    return rc, cc, rs, cs


def _outs(rc, cc, rs, cs, dirs):
    return (make_mx_out(rc, rs) if dirs & ROWWISE else None,
            make_mx_out(cc, cs) if dirs & COLWISE else None)


def swiglu_quantize_fwd(gate, up, scale=None, rowwise=True, colwise=False, row_off=None,
                        block_off=None, n_col_blocks=None, clamped=False, limit=7.0, interleave=0,
                        kblock=False, stream=None):
    """Returns (codes_row, codes_col, scales_row, scales_col); a disabled
    direction comes back zero-sized.  With groups, n_col_blocks must be the
    number of colwise scale rows (sum of ceil(split/32)).  With interleave = B,
    gate and up are (M, K) views p[:, :K] and p[:, B:B + K] of a packed (M, 2K)
    buffer p holding gate and up interleaved in blocks of B columns.  With
    kblock the rowwise codes come back K-blocked (a KBlocked)."""
    M, K = gate.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, K, dirs, n_col_blocks, gate.device, kblock)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    act = make_act(ACT_CLAMPED_SWIGLU if clamped else ACT_SWIGLU, limit, interleave)
    check(mxq_swiglu_quantize_fwd(act, gate, up, scale, make_groups(row_off, block_off), dirs, ro, co, stream))
    return rc, cc, rs, cs


def swiglu_bf16(gate, up, scale=None, rowwise=False, colwise=False, row_off=None, block_off=None,
                n_col_blocks=None, clamped=False, limit=7.0, interleave=0, srelu=False, out=None, stream=None):
    """The activation as dense bf16 h (M, K) (up None with srelu), and its
    MXFP8 forms from the same pass when asked: returns (h, codes_row,
    codes_col, scales_row, scales_col), a disabled direction zero-sized."""
    import torch
    M, K = gate.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, K, dirs, n_col_blocks, gate.device)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    h = out if out is not None else torch.empty((M, K), dtype=torch.bfloat16, device=gate.device)
    act = make_act(ACT_SRELU if srelu else (ACT_CLAMPED_SWIGLU if clamped else ACT_SWIGLU), limit, interleave)
    groups = make_groups(row_off, block_off) if row_off is not None else None
    check(mxq_swiglu_fwd_bf16(act, gate, up, scale, groups, dirs, ro, co, h, stream))
    return h, rc, cc, rs, cs


def srelu_quantize_fwd(x, scale=None, rowwise=True, colwise=False, row_off=None, block_off=None,
                       n_col_blocks=None, kblock=False, stream=None):
    """The row-scaled SReLU forward, MXFP8 out: (codes_row, codes_col,
    scales_row, scales_col) as swiglu_quantize_fwd."""
    M, K = x.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, K, dirs, n_col_blocks, x.device, kblock)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    check(mxq_swiglu_quantize_fwd(make_act(ACT_SRELU), x, None, scale, make_groups(row_off, block_off), dirs, ro,
                                  co, stream))
    return rc, cc, rs, cs


def quantize(x, rowwise=True, colwise=False, row_off=None, block_off=None, n_col_blocks=None, kblock=False,
             stream=None):
    M, K = x.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, K, dirs, n_col_blocks, x.device, kblock)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    check(mxq_quantize(x, make_groups(row_off, block_off), dirs, ro, co, stream))
    return rc, cc, rs, cs


def quantize_into(x, codes_row, codes_col, scales_row, scales_col, noop_flag=None, row_off=None,
                  block_off=None, stream=None):
    """Quantize x into caller-owned outputs (a direction is enabled when its
    codes tensor is given); with noop_flag (a device int32 tensor) the launch
    does nothing while the flag holds a non-zero value."""
    dirs = (ROWWISE if codes_row is not None else 0) | (COLWISE if codes_col is not None else 0)
    ro = make_mx_out(codes_row, scales_row) if codes_row is not None else None
    co = make_mx_out(codes_col, scales_col) if codes_col is not None else None
    check(mxq_quantize_noop(x, make_groups(row_off, block_off), dirs, ro, co, noop_flag, stream))


def swiglu_quantize_bwd(grad, gate, up, scale=None, rowwise=True, colwise=False, row_off=None,
                        block_off=None, n_col_blocks=None, clamped=False, limit=7.0, dense=True,
                        want_dscale=True, interleave=0, kblock=False, stream=None):
    """Returns (codes_row, codes_col, scales_row, scales_col, dgate_dup, dscale)
    where the codes cover the (M, 2K) [dgate | dup] matrix and dgate_dup is the
    packed (M, 2K) bf16 gradient (None when dense=False); with interleave = B
    (gate, up as in swiglu_quantize_fwd) both take the interleaved layout."""
    import torch
    M, K = gate.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, 2 * K, dirs, n_col_blocks, gate.device, kblock)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    dd = torch.empty((M, 2 * K), dtype=torch.bfloat16, device=gate.device) if dense else None
    ds = torch.empty(M, dtype=torch.float32, device=gate.device) if want_dscale else None
    nws = mxq_swiglu_quantize_bwd_workspace(M, K, dirs)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=gate.device) if (want_dscale and nws) else None
    _hold(ws, stream)
    act = make_act(ACT_CLAMPED_SWIGLU if clamped else ACT_SWIGLU, limit, interleave)
    uo = interleave if interleave else K
    check(mxq_swiglu_quantize_bwd(act, grad, gate, up, scale, make_groups(row_off, block_off),
                                  dd[:, :K] if dense else None, dd[:, uo:uo + K] if dense else None, ds,
                                  dirs, ro, co, ws, stream))
    return rc, cc, rs, cs, dd, ds


def srelu_quantize_bwd(grad, x, scale=None, rowwise=True, colwise=False, row_off=None, block_off=None,
                       n_col_blocks=None, dense=True, want_dscale=True, kblock=False, stream=None):
    """The row-scaled SReLU backward: (codes_row, codes_col, scales_row,
    scales_col, dx, dscale), the codes covering the (M, K) dx."""
    import torch
    M, K = x.shape
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = (M + 31) // 32 if row_off is None else colwise_scale_rows_bound(M, row_off.numel() - 1)
    rc, cc, rs, cs = _alloc_mx(M, K, dirs, n_col_blocks, x.device, kblock)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    dx = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if dense else None
    ds = torch.empty(M, dtype=torch.float32, device=x.device) if want_dscale else None
    nws = mxq_swiglu_quantize_bwd_workspace(M, K, dirs)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device) if (want_dscale and nws) else None
    _hold(ws, stream)
    check(mxq_swiglu_quantize_bwd(make_act(ACT_SRELU), grad, x, None, scale, make_groups(row_off, block_off), dx,
                                  None, ds, dirs, ro, co, ws, stream))
    return rc, cc, rs, cs, dx, ds


class KBlocked:
    """An operand K-blocked by 64 bytes (the layout of mxq_operand.kblock_plane
    and mxq_mx_out.kblock_plane): with e = 64 / element size elements per
    plane row, element (r, k) of a (rows, K) matrix sits at [k // e, r, k % e]
    of `data`, a (K / e, rows, e) tensor (uint8 MXFP8 codes or bf16) whose
    plane stride is data.stride(0) elements; a (G, N, K) stack of per-group
    matrices is blocked over its G * N rows.  `shape` is the logical
    (row-major) shape."""

    def __init__(self, data, shape):
        self.data = data
        self.shape = tuple(shape)
        if (self.shape[-1] * data.element_size()) % 64 != 0:
            raise ValueError("K-blocked operands need rows of a multiple of 64 bytes")

    @property
    def device(self):
        return self.data.device

    @property
    def epp(self):
        """Elements per 64-byte plane row."""
        return 64 // self.data.element_size()

    @property
    def plane(self):
        """Bytes between planes (at least 64, so that an empty matrix still
        reads as K-blocked)."""
        return max(self.data.stride(0) * self.data.element_size(), 64)

    @classmethod
    def from_rowmajor(cls, t):
        """Blocked copy of a row-major (R, K) or (G, N, K) tensor: a layout
        change done by torch, for tests, benchmarks and operands that were not
        written blocked by the kernels."""
        K = t.shape[-1]
        e = 64 // t.element_size()
        rows = t.numel() // K
        d = t.reshape(rows, K // e, e).transpose(0, 1).contiguous()
        return cls(d, t.shape)

    def to_rowmajor(self):
        return self.data.transpose(0, 1).reshape(self.shape).contiguous()

    @classmethod
    def empty(cls, shape, device, dtype=None):
        torch = _torch()
        dtype = torch.uint8 if dtype is None else dtype
        e = 64 // torch.empty((), dtype=dtype).element_size()
        K = shape[-1]
        rows = 1
        for d in shape[:-1]:
            rows *= d
        return cls(torch.empty((K // e, rows, e), dtype=dtype, device=device), shape)


def rowmajor(codes):
    """Row-major view of codes that may be K-blocked (a layout change by
    torch, for inspection)."""
    return codes.to_rowmajor() if isinstance(codes, KBlocked) else codes


def _operand(data, scales=None, group_dim=False):
    """mxq_operand from a data tensor (2-D, or 3-D stacked per group), or
    KBlocked codes, and its E8M0 scale tensor (same rank as the logical
    shape)."""
    if isinstance(data, KBlocked):
        f8 = data.data.dtype == _torch().uint8
        gs = data.shape[1] * data.epp if group_dim else 0
        op = mxq_operand(DTYPE_MXFP8 if f8 else DTYPE_BF16, data.data.data_ptr(), data.epp, gs, None, 0, 0,
                         data.plane)
    else:
        f8 = data.dtype == _torch().uint8
        if group_dim:
            ld = data.stride(1)
            gs = data.stride(0)
        else:
            ld = data.stride(0)
            gs = 0
        op = mxq_operand(DTYPE_MXFP8 if f8 else DTYPE_BF16, data.data_ptr(), ld, gs, None, 0, 0, 0)
    if scales is not None:
        op.scales = scales.data_ptr()
        op.ld_scales = scales.stride(1) if group_dim else scales.stride(0)
        op.scale_gstride = scales.stride(0) if group_dim else 0
    return op


def _torch():
    import torch
    return torch


def grouped_gemm(mode, row_off, A, B, out, A_scales=None, B_scales=None, block_off=None,
                 accumulate=False, max_workgroups=0, stream=None):
    """Run the grouped GEMM.  Shapes (bf16 tensors or uint8 E4M3 codes):
      NT: A (R, K), B (G, N, K), out (R, N); MXFP8 scales (R, K/32), (G, N, K/32)
      NN: A (R, K), B (G, K, N), out (R, N); MXFP8 scales (R, K/32), (G, K/32, N)
      TN: A (R, M), B (R, N), out (G, M, N); MXFP8 scales (n_blocks, M), (n_blocks, N)
    """
    G = row_off.numel() - 1
    if mode == GEMM_TN:
        R, M = A.shape
        N = B.shape[1]
        K = 0
        args = mxq_gemm_args(mode, G, row_off.data_ptr(), None if block_off is None else block_off.data_ptr(),
                             M, N, K, R, _operand(A, A_scales), _operand(B, B_scales),
                             DTYPE_F32 if out.dtype == _torch().float32 else DTYPE_BF16, out.data_ptr(),
                             out.stride(1), out.stride(0), int(accumulate), int(max_workgroups))
    else:
        R, K = A.shape
        N = B.shape[1] if mode == GEMM_NT else B.shape[2]
        args = mxq_gemm_args(mode, G, row_off.data_ptr(), None if block_off is None else block_off.data_ptr(),
                             R, N, K, R, _operand(A, A_scales), _operand(B, B_scales, group_dim=True),
                             DTYPE_F32 if out.dtype == _torch().float32 else DTYPE_BF16, out.data_ptr(),
                             out.stride(0), 0, int(accumulate), int(max_workgroups))
    ws = None
    need = mxq_grouped_gemm_workspace(args)
    if need:
        ws = _torch().empty(need, dtype=_torch().uint8, device=out.device)
        _hold(ws, stream)
    check(mxq_grouped_gemm(args, ws, stream))
    return out


def grouped_gemm_swiglu(row_off, x, w13, out, scale=None, rowwise=True, colwise=False, block_off=None,
                        n_col_blocks=None, clamped=False, limit=7.0, max_workgroups=0, stream=None):
    """FC1 with the row-scaled SwiGLU + MXFP8 in its epilogue: x (R, H) bf16,
    w13 (G, 2I, H) bf16 whose rows interleave gate and up in blocks of 128,
    out (R, 2I) bf16 (the interleaved product).  Returns the MXFP8 activation
    (codes_row, codes_col, scales_row, scales_col) of (R, I); a disabled
    direction comes back zero-sized."""
    G = row_off.numel() - 1
    R, H = x.shape
    N = w13.shape[1]
    I = N // 2
    dirs = (ROWWISE if rowwise else 0) | (COLWISE if colwise else 0)
    if n_col_blocks is None:
        n_col_blocks = colwise_scale_rows_bound(R, G)
    rc, cc, rs, cs = _alloc_mx(R, I, dirs, n_col_blocks, out.device)
    ro, co = _outs(rc, cc, rs, cs, dirs)
    args = mxq_gemm_args(GEMM_NT, G, row_off.data_ptr(), None if block_off is None else block_off.data_ptr(),
                         R, N, H, R, _operand(x), _operand(w13, None, group_dim=True), DTYPE_BF16, out.data_ptr(),
                         out.stride(0), 0, 0, int(max_workgroups))
    act = make_act(ACT_CLAMPED_SWIGLU if clamped else ACT_SWIGLU, limit, 128)
    check(mxq_grouped_gemm_swiglu(args, act, scale, dirs, ro, co, stream))
    return rc, cc, rs, cs


def interleave_rows(w, block=128):
    """(G, 2I, X) with rows [gate | up] -> rows interleaved in blocks of `block`
    (gate 0..block-1, up 0..block-1, gate block.., ...): the weight layout the
    fused FC1 epilogue reads.  A one-time layout change of a stored weight."""
    G, I2, X = w.shape
    I = I2 // 2
    nb = I // block
    return w.view(G, 2, nb, block, X).transpose(1, 2).reshape(G, I2, X).contiguous()
