"""K-blocked MXFP8 codes (include/mxq.h: mxq_operand.kblock_plane and
mxq_mx_out.kblock_plane): the fused activation kernels and the quantizer
write their rowwise codes in planes of 64 contraction bytes, and the grouped
GEMM reads such operands.  The layout changes only where the bytes sit, so
every result must equal the row-major path's bit for bit; the GEMM cases are
also compared with the oracle, within the GEMM tolerance
(|gpu - oracle| <= 1e-2 + 2e-2 |oracle| on identical quantized operands).

Pages: "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel" (Summary: rowwise 1x32 MXFP8 of the activation);
"Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
(Sequence Diagram: the quantized activation, dY and dact feed the grouped
forward and dgrad GEMMs).
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


def say(*a):
    print(*a, flush=True)


def u8(t):
    return t.cpu().numpy()


def eq(a, b, what):
    assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                       b.view(torch.uint8) if b.dtype != torch.uint8 else b), what


def offsets(m, splits):
    ro, bo, _ = m.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    return ro, bo


def col_scale_rows(M, splits):
    """Colwise scale rows the kernels write (the allocation's bound adds
    padding rows that nothing writes)."""
    if splits is None:
        return (M + 31) // 32
    return O.colwise_scale_rows(M, O.splits_to_offsets(splits)[0])


def test_kblocked_roundtrip(mxq):
    """The binding's layout change: (k // 64, r, k % 64) holds code (r, k)."""
    x = torch.arange(5 * 192, dtype=torch.int64).remainder(251).to(torch.uint8).view(5, 192).cuda()
    kb = mxq.KBlocked.from_rowmajor(x)
    assert kb.data.shape == (3, 5, 64) and kb.plane == 5 * 64
    assert torch.equal(kb.data[2, 4], x[4, 128:192])
    assert torch.equal(kb.to_rowmajor(), x)


FWD_CASES = [((96, 768), None, False, 0), ((100, 1024), None, True, 0), ((33, 128), None, False, 0),
             ((None, 256), [33, 0, 31, 1, 64, 0, 7], False, 0), ((70, 256), None, False, 128)]


@pytest.mark.parametrize("shape,splits,clamped,il", FWD_CASES)
def test_forward_kblock_equals_rowmajor(mxq, shape, splits, clamped, il):
    M, K = shape
    if splits is not None:
        M = sum(splits)
    say("fwd kblock", M, K, splits is not None, clamped, il)
    gu = W.packed_gate_up(M, K, seed=M + K, std=3.0 if clamped else 1.0).cuda()
    sc = W.row_scale(M, seed=M + K).cuda()
    g, u = gu[:, :K], (gu[:, il:il + K] if il else gu[:, K:])
    kw = dict(clamped=clamped, interleave=il, rowwise=True, colwise=True)
    if splits is not None:
        ro, bo = offsets(mxq, splits)
        kw.update(row_off=ro, block_off=bo)
    ref = mxq.swiglu_quantize_fwd(g, u, sc, **kw)
    got = mxq.swiglu_quantize_fwd(g, u, sc, kblock=True, **kw)
    torch.cuda.synchronize()
    assert isinstance(got[0], mxq.KBlocked)
    eq(got[0].to_rowmajor(), ref[0], "rowwise codes")
    for i, what in ((1, "colwise codes"), (2, "rowwise scales")):
        eq(got[i], ref[i], what)
    ncb = col_scale_rows(M, splits)
    eq(got[3][:ncb], ref[3][:ncb], "colwise scales")
    if il == 0 and splits is None and not clamped:
        # and against the oracle directly
        rc, _, rs, _, _ = O.swiglu_quantize_fwd(W.bf16_bits(g), W.bf16_bits(u), sc.cpu().numpy(), 1, None,
                                                O.SWIGLU, 7.0)
        assert np.array_equal(u8(got[0].to_rowmajor()), rc) and np.array_equal(u8(got[2]), rs)


BWD_CASES = [((96, 768), None, 0), ((64, 2048), None, 0), ((None, 128), [33, 0, 31, 1, 64, 0, 7], 0),
             ((70, 256), None, 128)]


@pytest.mark.parametrize("shape,splits,il", BWD_CASES)
@pytest.mark.parametrize("dirs", [1, 3])
def test_backward_kblock_equals_rowmajor(mxq, shape, splits, il, dirs):
    M, K = shape
    if splits is not None:
        M = sum(splits)
    say("bwd kblock", M, K, splits is not None, il, dirs)
    gu = W.packed_gate_up(M, K, seed=3 * M + K).cuda()
    sc = W.row_scale(M, seed=3 * M + K).cuda()
    dy = W.grad_out(M, K, seed=3 * M + K).cuda()
    g, u = gu[:, :K], (gu[:, il:il + K] if il else gu[:, K:])
    kw = dict(rowwise=True, colwise=bool(dirs & 2), interleave=il)
    if splits is not None:
        ro, bo = offsets(mxq, splits)
        kw.update(row_off=ro, block_off=bo)
    ref = mxq.swiglu_quantize_bwd(dy, g, u, sc, **kw)
    got = mxq.swiglu_quantize_bwd(dy, g, u, sc, kblock=True, **kw)
    torch.cuda.synchronize()
    eq(got[0].to_rowmajor(), ref[0], "rowwise codes of [dgate | dup]")
    for i, what in ((1, "colwise codes"), (2, "rowwise scales"), (4, "dgate|dup")):
        eq(got[i], ref[i], what)
    if dirs & 2:
        ncb = col_scale_rows(M, splits)
        eq(got[3][:ncb], ref[3][:ncb], "colwise scales")
    assert torch.equal(got[5].view(torch.int32), ref[5].view(torch.int32)), "dscale"


@pytest.mark.parametrize("M,K,splits", [(256, 2048, None), (None, 768, [5, 0, 17, 130, 1, 64, 0, 40])])
def test_quantize_kblock_equals_rowmajor(mxq, M, K, splits):
    if splits is not None:
        M = sum(splits)
    x = W._normal((M, K), 1.0, 5, 41, "cuda")
    kw = dict(rowwise=True, colwise=True)
    if splits is not None:
        ro, bo = offsets(mxq, splits)
        kw.update(row_off=ro, block_off=bo)
    ref = mxq.quantize(x, **kw)
    got = mxq.quantize(x, kblock=True, **kw)
    torch.cuda.synchronize()
    eq(got[0].to_rowmajor(), ref[0], "rowwise codes")
    for i in (1, 2):
        eq(got[i], ref[i], f"output {i}")
    ncb = col_scale_rows(M, splits)
    eq(got[3][:ncb], ref[3][:ncb], "colwise scales")


SPLITS = [5, 0, 17, 130, 1, 64, 0, 40, 300]


def qrows(rng, shape, std=1.0):
    q = O.mx_quantize(W.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
                                  .to(torch.bfloat16)), 1)
    return q[0], q[2]


def qcols(rng, shape, std=1.0):
    q = O.mx_quantize(W.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
                                  .to(torch.bfloat16)), 2)
    return q[1], q[3]


def check_close(got, ref):
    err = np.abs(got - ref)
    tol = 1e-2 + 2e-2 * np.abs(ref)
    assert np.all(err <= tol), f"max err {err.max()}"


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


# K = 768: 12 stages, so the row-scale ring (24 scale bytes per row, a
# multiple of 4) spans two 8-stage groups per tile; K = 128: the per-stage path.
@pytest.mark.parametrize("K", [128, 768])
@pytest.mark.parametrize("max_wg", [0, 8])
def test_gemm_nt_kblock(mxq, K, max_wg):
    rng = np.random.default_rng(K + max_wg)
    ro, _ = offsets(mxq, SPLITS)
    ro_np = O.splits_to_offsets(SPLITS)[0]
    R, N, G = sum(SPLITS), 272, len(SPLITS)
    A, As = qrows(rng, (R, K))
    Bl = [qrows(rng, (N, K), 0.05) for _ in range(G)]
    B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = O.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "f32")
    Ad, Bd, Asd, Bsd = dev(A), dev(B), dev(As), dev(Bs)
    rm = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, Ad, Bd, rm, Asd, Bsd, max_workgroups=max_wg)
    for a_kb, b_kb in ((True, True), (True, False), (False, True)):
        out = torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NT, ro, mxq.KBlocked.from_rowmajor(Ad) if a_kb else Ad,
                         mxq.KBlocked.from_rowmajor(Bd) if b_kb else Bd, out, Asd, Bsd, max_workgroups=max_wg)
        torch.cuda.synchronize()
        eq(out, rm, f"NT K-blocked A={a_kb} B={b_kb} against row-major")
    check_close(out.cpu().numpy().astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("K", [192, 1536])
def test_gemm_nn_kblock(mxq, K):
    rng = np.random.default_rng(K)
    ro, _ = offsets(mxq, SPLITS)
    ro_np = O.splits_to_offsets(SPLITS)[0]
    R, N, G = sum(SPLITS), 176, len(SPLITS)
    A, As = qrows(rng, (R, K))
    Bl = [qcols(rng, (K, N), 0.05) for _ in range(G)]
    B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = O.Operand("mxfp8", B, K * N, 1, N, Bs, (K // 32) * N, 1, N)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "bf16")
    Ad, Bd, Asd, Bsd = dev(A), dev(B), dev(As), dev(Bs)
    rm = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(rm)
    mxq.grouped_gemm(mxq.GEMM_NN, ro, Ad, Bd, rm, Asd, Bsd)
    mxq.grouped_gemm(mxq.GEMM_NN, ro, mxq.KBlocked.from_rowmajor(Ad), Bd, out, Asd, Bsd)
    torch.cuda.synchronize()
    eq(out, rm, "NN K-blocked A against row-major")
    got = (W.bf16_bits(out).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    check_close(got, (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64))


def test_gemm_fc2_shape_kblock(mxq):
    """The expert layer's FC2 forward (65,536 rows over 128 experts, N 2048,
    K 768) and FC2 dgrad shapes: K-blocked operands give the row-major bits."""
    R, G, N, K = 65536, 128, 2048, 768
    ro, bo = offsets(mxq, [R // G] * G)
    a = mxq.quantize(W._normal((R, K), 1.0, 7, 42, "cuda"), rowwise=True)
    ak = mxq.quantize(W._normal((R, K), 1.0, 7, 42, "cuda"), rowwise=True, kblock=True)
    eq(ak[0].to_rowmajor(), a[0], "A codes")
    w = mxq.quantize(W._normal((G * N, K), 0.02, 8, 43, "cuda"), rowwise=True)
    b, bs = w[0].view(G, N, K), w[2].view(G, N, K // 32)
    y1 = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    mxq.grouped_gemm(mxq.GEMM_NT, ro, a[0], b, y1, a[2], bs)
    mxq.grouped_gemm(mxq.GEMM_NT, ro, ak[0], mxq.KBlocked.from_rowmajor(b), y2, ak[2], bs)
    torch.cuda.synchronize()
    eq(y2, y1, "FC2 forward")


@pytest.mark.parametrize("recipe,fused", [("mxfp8", False), ("bf16_wgrad", False), ("mxfp8", True)])
def test_layer_kblock_equals_rowmajor(mxq, recipe, fused):
    """The expert layer with K-blocked activation, dY and dact codes (the
    default) against the row-major layer: every output bit for bit."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    T, H, E, k, I = 256, 512, 16, 2, 256
    moe = W.moe_layer(13, skewed=True, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    R = int(moe["splits"].sum())
    splits, w13, w2 = moe["splits"].cuda(), moe["w13"].cuda(), moe["w2"].cuda()
    x, sc = moe["x_perm"].cuda(), moe["scale"].cuda()
    dy = W.moe_grad(R, H, seed=13).cuda()
    outs = []
    for kb in (True, False):
        layer = Layer(splits, w13, w2, fused_fc1=fused, recipe=recipe, kblock=kb)
        y = layer.forward(x, sc)
        dx, dw13, dw2, ds = layer.backward(dy)
        torch.cuda.synchronize()
        outs.append((y, dx, dw13, dw2, ds))
        if kb:
            assert isinstance(layer.grads["dy_r"], mxq.KBlocked)
    for a, b, what in zip(outs[0], outs[1], ("Y", "dX", "dW13", "dW2", "dscale")):
        eq(a, b, what)


@pytest.mark.parametrize("mode", ["NT", "NN"])
def test_gemm_bf16_kblock(mxq, mode):
    """bf16 operands K-blocked by 64 bytes (32 elements per plane row): NT
    with A, B or both blocked, NN with A blocked, against the row-major run
    bit for bit and against the oracle."""
    rng = np.random.default_rng(51 if mode == "NT" else 52)
    ro, _ = offsets(mxq, SPLITS)
    ro_np = O.splits_to_offsets(SPLITS)[0]
    R, N, K, G = sum(SPLITS), 208, 320, len(SPLITS)

    def bf(shape, std):
        return W.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))
    A = bf((R, K), 1.0)
    Ad = W.from_bits(A, "cuda")
    if mode == "NT":
        B = bf((G, N, K), 0.05)
        opB = O.Operand("bf16", B, N * K, K, 1)
    else:
        B = bf((G, K, N), 0.05)
        opB = O.Operand("bf16", B, K * N, 1, N)
    Bd = W.from_bits(B, "cuda")
    ref = O.grouped_gemm("m", ro_np, 0, N, K, O.Operand("bf16", A, 0, K, 1), opB, "f32")
    gm = mxq.GEMM_NT if mode == "NT" else mxq.GEMM_NN
    rm = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(gm, ro, Ad, Bd, rm)
    combos = ((True, True), (True, False), (False, True)) if mode == "NT" else ((True, False),)
    for a_kb, b_kb in combos:
        out = torch.full((R, N), 7.0, dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(gm, ro, mxq.KBlocked.from_rowmajor(Ad) if a_kb else Ad,
                         mxq.KBlocked.from_rowmajor(Bd) if b_kb else Bd, out)
        torch.cuda.synchronize()
        eq(out, rm, f"{mode} bf16 K-blocked A={a_kb} B={b_kb} against row-major")
    check_close(out.cpu().numpy().astype(np.float64), ref.astype(np.float64))


@pytest.mark.parametrize("M,K", [(96, 768), (64, 1024)])
def test_srelu_kblock_equals_rowmajor(mxq, M, K):
    """The row-scaled SReLU (unary) through the same stores: forward codes and
    the backward's dx codes K-blocked against row-major."""
    x = W._normal((M, K), 1.0, 9, 44, "cuda")
    sc = W.row_scale(M, seed=9).cuda()
    dy = W.grad_out(M, K, seed=9).cuda()
    ref = mxq.srelu_quantize_fwd(x, sc, rowwise=True, colwise=True)
    got = mxq.srelu_quantize_fwd(x, sc, rowwise=True, colwise=True, kblock=True)
    rb = mxq.srelu_quantize_bwd(dy, x, sc, rowwise=True, colwise=True)
    gb = mxq.srelu_quantize_bwd(dy, x, sc, rowwise=True, colwise=True, kblock=True)
    torch.cuda.synchronize()
    eq(got[0].to_rowmajor(), ref[0], "forward rowwise codes")
    eq(gb[0].to_rowmajor(), rb[0], "backward rowwise codes")
    for i in (1, 2, 3):
        eq(got[i], ref[i], f"forward output {i}")
        eq(gb[i], rb[i], f"backward output {i}")
    eq(gb[4], rb[4], "dx")


def test_gemm_fc1_shape_bf16_kblock(mxq):
    """The expert layer's FC1 in bf16 (65,536 rows over 128 experts, N 1536,
    K 2048) with the tokens and the weight K-blocked (32 elements per plane
    row): the row-major bits."""
    R, G, N, K = 65536, 128, 1536, 2048
    ro, _ = offsets(mxq, [R // G] * G)
    x = W._normal((R, K), 1.0, 10, 45, "cuda")
    w = W._normal((G * N, K), 0.02, 11, 46, "cuda").view(G, N, K)
    y1 = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y1)
    mxq.grouped_gemm(mxq.GEMM_NT, ro, x, w, y1)
    mxq.grouped_gemm(mxq.GEMM_NT, ro, mxq.KBlocked.from_rowmajor(x), mxq.KBlocked.from_rowmajor(w), y2)
    torch.cuda.synchronize()
    eq(y2, y1, "FC1 bf16 K-blocked against row-major")


@pytest.mark.parametrize("dirs", [1, 3])
def test_fused_fc1_kblock_operands(mxq, dirs):
    """FC1 with the SwiGLU + MXFP8 epilogue over K-blocked bf16 operands (the
    epilogue's own outputs stay row-major): every output equals the
    row-major launch's."""
    splits = [33, 0, 260, 1, 96, 0, 300, 64]
    G, H, I = len(splits), 256, 256
    R = sum(splits)
    ro, bo = offsets(mxq, splits)
    x = W._normal((R, H), 1.0, 12, 47, "cuda")
    w13 = mxq.interleave_rows(W._normal((G * 2 * I, H), 0.05, 13, 48, "cuda").view(G, 2 * I, H))
    sc = W.row_scale(R, seed=12).cuda()
    kw = dict(scale=sc, rowwise=True, colwise=bool(dirs & 2), block_off=bo)
    h1 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h1)
    ref = mxq.grouped_gemm_swiglu(ro, x, w13, h1, **kw)
    got = mxq.grouped_gemm_swiglu(ro, mxq.KBlocked.from_rowmajor(x), mxq.KBlocked.from_rowmajor(w13), h2, **kw)
    torch.cuda.synchronize()
    eq(h2, h1, "bf16 product")
    ncb = col_scale_rows(R, splits)
    for i, what in ((0, "rowwise codes"), (2, "rowwise scales")):
        eq(got[i], ref[i], what)
    if dirs & 2:
        eq(got[1], ref[1], "colwise codes")
        eq(got[3][:ncb], ref[3][:ncb], "colwise scales")
