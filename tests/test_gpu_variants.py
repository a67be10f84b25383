"""GPU parity of the activation variants against the CPU oracle, through the C
ABI: the row-scaled SReLU (forward and backward, unary) and gate / up
interleaved in blocks of B columns (forward and backward, the gradient in the
same interleaved layout).

Page "Activation + GroupedLinear Fusion for MOE and other MOE
optimizations": Greptile Summary (the scaled activations SReLU, SwiGLU and
ClampedSwiGLU) and Important Files Changed (the GLU interleave handled inside
the scaled SwiGLU kernels).  Page "[mxfp8 training] Add a fused gated-
activation (SwiGLU) + MXFP8 quantization kernel", Follow-ups (more
activations through the compile-time activation policy).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import compare_bf16, compare_mx, rowblock_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


def bits(t):
    return W.bf16_bits(t)


def u8(t):
    return t.cpu().numpy()


def assert_exact(rep):
    bad = {k: v for k, v in rep.items() if not k.endswith("maxerr") and v}
    assert not bad, f"outputs differ from the oracle: {bad}"


def offsets(m, splits):
    if splits is None:
        return None, None, None
    ro, bo, _ = m.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    return ro, bo, O.splits_to_offsets(splits)[0]


# ------------------------------------------------------------------ SReLU

SRELU_SHAPES = [(96, 64), (100, 256), (33, 32), (64, 2048), (40, 7168), (256, 768)]


@pytest.mark.parametrize("shape", SRELU_SHAPES)
@pytest.mark.parametrize("d", [1, 2, 3])
def test_srelu_forward(mxq, shape, d):
    M, K = shape
    x = W.packed_gate_up(M, K, seed=M + K, std=2.0)[:, :K].contiguous()
    sc = W.row_scale(M, seed=M + K)
    rc, cc, rs, cs, h, close = O.srelu_quantize_fwd(bits(x), sc.numpy(), d, want_close=True)
    out = mxq.srelu_quantize_fwd(x.cuda(), sc.cuda(), rowwise=bool(d & 1), colwise=bool(d & 2))
    torch.cuda.synchronize()
    rep = {}
    if d & 1:
        compare_mx("srelu.row", u8(out[0]), u8(out[2]), rc, rs, close != 0, True, report=rep)
    if d & 2:
        compare_mx("srelu.col", u8(out[1]), u8(out[3]), cc, cs, close != 0, False, rowblock_of(M), report=rep)
    assert_exact(rep)


def test_srelu_forward_every_bf16_input(mxq):
    """All 65,536 bf16 patterns as x (2048 rows of 32), s = 1 and a second
    pass with a row scale: NaN / Inf blocks, subnormal squares, ties of the
    square, both directions, bit-exact."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).reshape(-1, 32)
    xt = W.from_bits(x, "cuda")
    for sc in (None, W.row_scale(x.shape[0], seed=9)):
        ref = O.srelu_quantize_fwd(x, None if sc is None else sc.numpy(), 3)
        out = mxq.srelu_quantize_fwd(xt, None if sc is None else sc.cuda(), rowwise=True, colwise=True)
        torch.cuda.synchronize()
        for got, r, name in zip(out, ref[:4], ("row codes", "col codes", "row scales", "col scales")):
            assert np.array_equal(u8(got), r), name


@pytest.mark.parametrize("shape", SRELU_SHAPES)
@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_srelu_backward(mxq, shape, d):
    M, K = shape
    x = W.packed_gate_up(M, K, seed=3 * M + K, std=2.0)[:, :K].contiguous()
    sc = W.row_scale(M, seed=3 * M + K)
    dy = W.grad_out(M, K, seed=3 * M + K)
    rc, cc, rs, cs, dx, ds, close, tol = O.srelu_quantize_bwd(bits(dy), bits(x), sc.numpy(), d, want_close=True)
    out = mxq.srelu_quantize_bwd(dy.cuda(), x.cuda(), sc.cuda(), rowwise=bool(d & 1), colwise=bool(d & 2))
    torch.cuda.synchronize()
    rep = {}
    closeb = close != 0
    if d & 1:
        compare_mx("srelu.bwd.row", u8(out[0]), u8(out[2]), rc, rs, closeb, True, report=rep)
    if d & 2:
        compare_mx("srelu.bwd.col", u8(out[1]), u8(out[3]), cc, cs, closeb, False, rowblock_of(M), report=rep)
    compare_bf16("dx", bits(out[4]), dx, closeb, rep)
    err = np.abs(out[5].cpu().numpy().astype(np.float64) - ds.astype(np.float64))
    assert np.all(err <= tol + 1e-30), f"dscale off by {err.max()}"
    assert_exact(rep)


def test_srelu_grouped_and_special_values(mxq):
    """Per-expert colwise blocks, and inputs with zeros, -0, negative and
    subnormal values, NaN and Inf, forward and backward."""
    splits = [33, 0, 70, 1, 24]
    M, K = sum(splits), 128
    ro, bo, ro_np = offsets(mxq, splits)
    x = W.packed_gate_up(M, K, seed=61, std=3.0)[:, :K].contiguous()
    xb = bits(x)
    rng = np.random.default_rng(61)
    special = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x7F80, 0xFF80, 0x7FC0, 0x1F00], np.uint16)
    pos = rng.choice(M * K, 40, replace=False)
    xb.reshape(-1)[pos] = special[np.arange(40) % len(special)]
    xt = W.from_bits(xb, "cuda")
    sc = W.row_scale(M, seed=61)
    dy = W.grad_out(M, K, seed=61)
    ncb = sum((s + 31) // 32 for s in splits)
    f = O.srelu_quantize_fwd(xb, sc.numpy(), 3, ro_np, want_close=True)
    out = mxq.srelu_quantize_fwd(xt, sc.cuda(), True, True, ro, bo, n_col_blocks=ncb)
    b = O.srelu_quantize_bwd(bits(dy), xb, sc.numpy(), 3, ro_np, want_close=True)
    outb = mxq.srelu_quantize_bwd(dy.cuda(), xt, sc.cuda(), True, True, ro, bo, n_col_blocks=ncb)
    torch.cuda.synchronize()
    rep = {}
    compare_mx("f.row", u8(out[0]), u8(out[2]), f[0], f[2], f[5] != 0, True, report=rep)
    compare_mx("f.col", u8(out[1]), u8(out[3]), f[1], f[3], f[5] != 0, False, rowblock_of(M, ro_np), report=rep)
    compare_mx("b.row", u8(outb[0]), u8(outb[2]), b[0], b[2], b[6] != 0, True, report=rep)
    compare_mx("b.col", u8(outb[1]), u8(outb[3]), b[1], b[3], b[6] != 0, False, rowblock_of(M, ro_np), report=rep)
    compare_bf16("dx", bits(outb[4]), b[4], b[6] != 0, rep)
    got_ds, ref_ds = outb[5].cpu().numpy().astype(np.float64), b[5].astype(np.float64)
    fin = np.isfinite(ref_ds)
    assert np.array_equal(np.isnan(got_ds), np.isnan(ref_ds))
    inf = np.isinf(ref_ds)
    assert np.array_equal(got_ds[inf], ref_ds[inf])
    assert np.all(np.abs(got_ds[fin] - ref_ds[fin]) <= b[7][fin] + 1e-30)
    assert_exact(rep)


def test_swiglu_backward_infinite_gate_dscale(mxq):
    """An infinite gate makes a = bf16(silu(g)) infinite (or NaN for -Inf):
    dscale's fast sum and its exact-path correction must give the oracle's
    +-Inf / NaN row sums, not a NaN from Inf - Inf (regression)."""
    M, K = 64, 128
    p = W.packed_gate_up(M, K, seed=81)
    pb = bits(p)
    pb[3, 5] = 0x7F80          # +Inf gate
    pb[7, 9] = 0xFF80          # -Inf gate
    pb[11, 2] = 0x7F80
    pb[11, K + 2] = 0x0000     # +Inf gate times a zero up
    pt = W.from_bits(pb, "cuda")
    sc = W.row_scale(M, seed=81)
    dy = W.grad_out(M, K, seed=81)
    r = O.swiglu_quantize_bwd(bits(dy), pb[:, :K], pb[:, K:], sc.numpy(), 3, want_close=True)
    out = mxq.swiglu_quantize_bwd(dy.cuda(), pt[:, :K], pt[:, K:], sc.cuda(), True, True)
    torch.cuda.synchronize()
    rep = {}
    closeb = r[7] != 0
    compare_mx("row", u8(out[0]), u8(out[2]), r[0], r[2], closeb, True, report=rep)
    compare_mx("col", u8(out[1]), u8(out[3]), r[1], r[3], closeb, False, rowblock_of(M), report=rep)
    dd = bits(out[4])
    compare_bf16("dgate", dd[:, :K], r[4], closeb[:, :K], rep)
    compare_bf16("dup", dd[:, K:], r[5], closeb[:, K:], rep)
    got, ref = out[5].cpu().numpy().astype(np.float64), r[6].astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    inf = np.isinf(ref)
    assert inf.sum() + np.isnan(ref).sum() >= 2
    assert np.array_equal(got[inf], ref[inf])
    fin = np.isfinite(ref)
    assert np.all(np.abs(got[fin] - ref[fin]) <= r[8][fin] + 1e-30)
    assert_exact(rep)


# ------------------------------------------------------------------ GLU interleave

@pytest.mark.parametrize("B,K", [(32, 128), (128, 768), (256, 768), (64, 2048)])
@pytest.mark.parametrize("clamped", [False, True])
def test_interleaved_forward(mxq, B, K, clamped):
    splits = [40, 0, 97, 31]
    M = sum(splits)
    ro, bo, ro_np = offsets(mxq, splits)
    p = W.packed_gate_up(M, K, seed=B + K, std=4.0 if clamped else 1.0)
    sc = W.row_scale(M, seed=B + K)
    g, u = O.glu_split(bits(p), B)
    kind = O.CLAMPED_SWIGLU if clamped else O.SWIGLU
    rc, cc, rs, cs, h, close = O.swiglu_quantize_fwd(g, u, sc.numpy(), 3, ro_np, kind, 7.0, want_close=True)
    pd = p.cuda()
    ncb = cs.shape[0]
    out = mxq.swiglu_quantize_fwd(pd[:, :K], pd[:, B:B + K], sc.cuda(), True, True, ro, bo, n_col_blocks=ncb,
                                  clamped=clamped, interleave=B)
    torch.cuda.synchronize()
    rep = {}
    compare_mx("il.row", u8(out[0]), u8(out[2]), rc, rs, close != 0, True, report=rep)
    compare_mx("il.col", u8(out[1]), u8(out[3]), cc, cs, close != 0, False, rowblock_of(M, ro_np), report=rep)
    assert_exact(rep)


@pytest.mark.parametrize("B,K", [(32, 128), (128, 768), (64, 2048)])
@pytest.mark.parametrize("d", [0, 1, 3])
def test_interleaved_backward(mxq, B, K, d):
    splits = [40, 0, 97, 31]
    M = sum(splits)
    ro, bo, ro_np = offsets(mxq, splits)
    p = W.packed_gate_up(M, K, seed=2 * B + K)
    sc = W.row_scale(M, seed=2 * B + K)
    dy = W.grad_out(M, K, seed=2 * B + K)
    r = O.swiglu_quantize_bwd_interleaved(bits(dy), bits(p), B, sc.numpy(), d, ro_np, want_close=True)
    rc, cc, rs, cs, dref, ds, close, tol = r
    pd = p.cuda()
    ncb = O.colwise_scale_rows(M, ro_np)
    out = mxq.swiglu_quantize_bwd(dy.cuda(), pd[:, :K], pd[:, B:B + K], sc.cuda(), bool(d & 1), bool(d & 2), ro, bo,
                                  n_col_blocks=ncb, interleave=B)
    torch.cuda.synchronize()
    rep = {}
    closeb = close != 0
    if d & 1:
        compare_mx("il.bwd.row", u8(out[0]), u8(out[2]), rc, rs, closeb, True, report=rep)
    if d & 2:
        compare_mx("il.bwd.col", u8(out[1]), u8(out[3]), cc, cs, closeb, False, rowblock_of(M, ro_np), report=rep)
    compare_bf16("d_packed", bits(out[4]), dref, closeb, rep)
    err = np.abs(out[5].cpu().numpy().astype(np.float64) - ds.astype(np.float64))
    assert np.all(err <= tol + 1e-30), f"dscale off by {err.max()}"
    assert_exact(rep)


def test_interleave_block_k_equals_plain(mxq):
    """B = K is the plain packed [gate | up]: the same outputs as without
    interleaving, forward and backward."""
    M, K = 96, 256
    p = W.packed_gate_up(M, K, seed=71).cuda()
    sc = W.row_scale(M, seed=71).cuda()
    dy = W.grad_out(M, K, seed=71).cuda()
    a = mxq.swiglu_quantize_fwd(p[:, :K], p[:, K:], sc, True, True)
    b = mxq.swiglu_quantize_fwd(p[:, :K], p[:, K:], sc, True, True, interleave=K)
    c = mxq.swiglu_quantize_bwd(dy, p[:, :K], p[:, K:], sc, True, True)
    e = mxq.swiglu_quantize_bwd(dy, p[:, :K], p[:, K:], sc, True, True, interleave=K)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(c[:4], e[:4]):
        assert torch.equal(x, y)
    assert torch.equal(c[4].view(torch.int16), e[4].view(torch.int16)) and torch.equal(c[5], e[5])
