"""GPU parity of the pieces of the BF16-wgrad recipe, through the C ABI.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel", Performance: under the recipe the fused kernel emits
rowwise-only MXFP8 casts, and the activation is recomputed in bf16 for the two
wgrad GEMMs, which then run in bf16.  Checked here:
  * mxq_swiglu_fwd_bf16: the dense bf16 activation (alone, dirs = 0, or with
    its MXFP8 forms from the same pass), bit-exact against the oracle's
    activation, for the plain, clamped and SReLU kinds, grouped, interleaved;
  * the bf16 grouped GEMM in the modes whose operands are strided along the
    contraction (NN, the dgrad shape; TN, the K-grouped wgrad) against the
    oracle's grouped GEMM: ragged and empty groups, several tiles and a
    ragged tile on both sides, the dynamic tile order of skewed groups, fp32
    accumulation, and workgroups chaining tiles.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import compare_bf16, compare_mx, rowblock_of, rowmajor

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
    bad = {k: v for k, v in rep.items() if v}
    assert not bad, f"mismatches: {bad}"


def offsets(m, splits):
    if splits is None:
        return None, None, None
    ro, bo, _ = m.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    return ro, bo, O.splits_to_offsets(splits)[0]


# ------------------------------------------------------------------ the dense activation

@pytest.mark.parametrize("kind", ["swiglu", "clamped", "srelu"])
@pytest.mark.parametrize("M,K,splits", [(70, 96, None), (257, 1056, None), (168, 768, [40, 0, 97, 31])])
@pytest.mark.parametrize("d", [0, 1, 3])
def test_swiglu_fwd_bf16(mxq, kind, M, K, splits, d):
    ro, bo, ro_np = offsets(mxq, splits)
    seed = M + K + d
    p = W.packed_gate_up(M, K, seed=seed, std=4.0 if kind == "clamped" else 1.0)
    sc = W.row_scale(M, seed=seed)
    g, u = bits(p[:, :K]), bits(p[:, K:])
    if kind == "srelu":
        h, close = O.srelu_fwd(g, sc.numpy(), want_close=True)
    else:
        h, close = O.swiglu_fwd(g, u, sc.numpy(), O.CLAMPED_SWIGLU if kind == "clamped" else O.SWIGLU, 7.0,
                                want_close=True)
    pd = p.cuda()
    x = pd[:, :K].contiguous() if kind == "srelu" else pd[:, :K]
    ncb = O.colwise_scale_rows(M, ro_np)
    got = mxq.swiglu_bf16(x, None if kind == "srelu" else pd[:, K:], sc.cuda(), bool(d & 1), bool(d & 2), ro, bo,
                          n_col_blocks=ncb, clamped=kind == "clamped", srelu=kind == "srelu")
    torch.cuda.synchronize()
    rep = {}
    closeb = close != 0
    compare_bf16("h", bits(got[0]), h, closeb, rep)
    if d:
        rc, cc, rs, cs = O.mx_quantize(h, d, ro_np)
        if d & 1:
            compare_mx("row", u8(got[1]), u8(got[3]), rc, rs, closeb, True, report=rep)
        if d & 2:
            compare_mx("col", u8(got[2]), u8(got[4]), cc, cs, closeb, False, rowblock_of(M, ro_np), report=rep)
    assert_exact(rep)


def test_swiglu_fwd_bf16_matches_quantizing_forward(mxq):
    """The MXFP8 outputs of the dense-output forward are those of
    mxq_swiglu_quantize_fwd, bit for bit, at a multi-slab shape."""
    M, K = 512, 2048
    p = W.packed_gate_up(M, K, seed=5).cuda()
    sc = W.row_scale(M, seed=5).cuda()
    a = mxq.swiglu_bf16(p[:, :K], p[:, K:], sc, True, True)
    b = mxq.swiglu_quantize_fwd(p[:, :K], p[:, K:], sc, True, True)
    torch.cuda.synchronize()
    for x, y in zip(a[1:], b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,K", [(128, 768), (64, 2048)])
def test_swiglu_fwd_bf16_interleaved(mxq, B, K):
    """Gate and up interleaved in blocks of B: h comes out in logical order."""
    M = 200
    p = W.packed_gate_up(M, K, seed=B + K)
    sc = W.row_scale(M, seed=B + K)
    g, u = O.glu_split(bits(p), B)
    h, close = O.swiglu_fwd(g, u, sc.numpy(), want_close=True)
    pd = p.cuda()
    got = mxq.swiglu_bf16(pd[:, :K], pd[:, B:B + K], sc.cuda(), interleave=B)
    torch.cuda.synchronize()
    rep = {}
    compare_bf16("h", bits(got[0]), h, close != 0, rep)
    assert_exact(rep)


def test_swiglu_fwd_bf16_every_gate(mxq):
    """Every finite bf16 gate value (the exact-path decisions included) through
    the dense output, with random up and row scale."""
    g = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    g = g[(g & 0x7F80) != 0x7F80].reshape(-1, 32)   # the 65,280 finite patterns
    M = g.shape[0]
    u = bits(W.packed_gate_up(M, 32, seed=17)[:, 32:])
    sc = W.row_scale(M, seed=17)
    h = O.swiglu_fwd(g, u, sc.numpy())
    got = mxq.swiglu_bf16(W.from_bits(g, "cuda"), W.from_bits(u, "cuda"), sc.cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits(got[0]), h)


def test_swiglu_fwd_bf16_empty_and_errors(mxq):
    e = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    h = mxq.swiglu_bf16(e, e)[0]
    assert h.shape == (0, 64)
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mxq.MxqError):   # no dense output: the quantizing forward's job
        mxq.check(mxq.mxq_swiglu_fwd_bf16(mxq.make_act(), x, x, None, None, 0, None, None, None))
    with pytest.raises(mxq.MxqError):   # h on top of an input
        mxq.check(mxq.mxq_swiglu_fwd_bf16(mxq.make_act(), x, x, None, None, 0, None, None, x))


# ------------------------------------------------------------------ bf16 GEMMs strided along the contraction

def rand_bf16(rng, shape, std=1.0):
    return W.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))


def out_np(t):
    if t.dtype == torch.bfloat16:
        return (W.bf16_bits(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def ref_np(o, out_dtype):
    if out_dtype == "bf16":
        return (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return o.astype(np.float64)


def check_close(got, ref):
    """fp32 accumulation in another order, one rounding to the output."""
    err = np.abs(got - ref)
    tol = 1e-2 + 2e-2 * np.abs(ref)
    assert np.all(err <= tol), f"max err {err.max()} at {np.unravel_index(np.argmax(err - tol), err.shape)}"


def dev(x):
    return W.from_bits(x, "cuda")


NN_SPLITS = [5, 0, 17, 300, 1, 64, 0, 40]


@pytest.mark.parametrize("K", [192, 352, 1536])
@pytest.mark.parametrize("out_dtype,max_wg", [("bf16", 0), ("f32", 8)])
def test_nn_bf16(mxq, K, out_dtype, max_wg):
    """dgrad shape: C[r, n] = sum_k A[r, k] B_g[k, n], B (G, K, N)."""
    rng = np.random.default_rng(K)
    ro, _, ro_np = offsets(mxq, NN_SPLITS)
    R, N, G = sum(NN_SPLITS), 272, len(NN_SPLITS)
    A = rand_bf16(rng, (R, K))
    B = rand_bf16(rng, (G, K, N), 0.05)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, O.Operand("bf16", A, 0, K, 1), O.Operand("bf16", B, K * N, 1, N),
                         out_dtype)
    out = torch.empty((R, N), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NN, ro, dev(A), dev(B), out, max_workgroups=max_wg)
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, out_dtype))


TN_SPLITS = [33, 0, 31, 200, 1, 0, 64, 290]


@pytest.mark.parametrize("M,N", [(160, 144), (288, 272)])
@pytest.mark.parametrize("accumulate,max_wg", [(False, 0), (True, 0), (False, 8)])
def test_tn_bf16(mxq, M, N, accumulate, max_wg):
    """wgrad shape: C_g[m, n] = sum over group g's rows r of A[r, m] B[r, n];
    groups of 1..290 rows (contraction tails inside a 32-row stage), empty
    groups write zeros (or, accumulating, leave C_g as it was)."""
    rng = np.random.default_rng(M + N)
    ro, _, ro_np = offsets(mxq, TN_SPLITS)
    R, G = sum(TN_SPLITS), len(TN_SPLITS)
    A = rand_bf16(rng, (R, M))
    B = rand_bf16(rng, (R, N), 0.05)
    opA = O.Operand("bf16", A, 0, 1, M)
    opB = O.Operand("bf16", B, 0, 1, N)
    od = "f32" if accumulate else "bf16"
    base = (rng.standard_normal((G, M, N)) * 0.5).astype(np.float32)
    ref = O.grouped_gemm("k", ro_np, M, N, 0, opA, opB, od, out=base.copy() if accumulate else None,
                         accumulate=accumulate)
    if accumulate:
        out = torch.from_numpy(base.copy()).cuda()
    else:
        out = torch.full((G, M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, dev(A), dev(B), out, accumulate=accumulate, max_workgroups=max_wg)
    torch.cuda.synchronize()
    got = out_np(out)
    check_close(got, ref_np(ref, od))
    if not accumulate:
        assert np.all(got[1] == 0) and np.all(got[5] == 0)


SKEW_SPLITS = [1300, 0, 3, 0, 40, 7, 0, 90, 1, 1, 2, 300, 0, 5, 64, 0, 33, 2, 0, 150]


@pytest.mark.parametrize("max_wg", [8, 0])
def test_tn_bf16_skewed_dynamic_order(mxq, max_wg):
    """One large group among small and empty ones: the tiles are taken
    largest group first from the workspace counter."""
    rng = np.random.default_rng(29)
    ro, _, ro_np = offsets(mxq, SKEW_SPLITS)
    R, M, N, G = sum(SKEW_SPLITS), 768, 512, len(SKEW_SPLITS)
    A = rand_bf16(rng, (R, M))
    B = rand_bf16(rng, (R, N), 0.05)
    ref = O.grouped_gemm("k", ro_np, M, N, 0, O.Operand("bf16", A, 0, 1, M), O.Operand("bf16", B, 0, 1, N), "bf16")
    out = torch.empty((G, M, N), dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, dev(A), dev(B), out, max_workgroups=max_wg)
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, "bf16"))


def test_tn_bf16_integer_exact(mxq):
    """Small integers: every product and partial sum is exact in fp32, so the
    result is the oracle's bit for bit whatever the summation order."""
    rng = np.random.default_rng(31)
    splits = [37, 0, 130, 255, 3]
    ro, _, ro_np = offsets(mxq, splits)
    R, M, N, G = sum(splits), 96, 80, len(splits)
    A = W.bf16_bits(torch.from_numpy(rng.integers(-8, 9, (R, M)).astype(np.float32)).to(torch.bfloat16))
    B = W.bf16_bits(torch.from_numpy(rng.integers(-8, 9, (R, N)).astype(np.float32)).to(torch.bfloat16))
    ref = O.grouped_gemm("k", ro_np, M, N, 0, O.Operand("bf16", A, 0, 1, M), O.Operand("bf16", B, 0, 1, N), "f32")
    out = torch.empty((G, M, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, dev(A), dev(B), out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref)


# ------------------------------------------------------------------ the expert layer under the recipe

@pytest.mark.parametrize("skewed,clamped,fused", [(False, False, False), (True, True, False), (True, False, True)])
def test_layer_bf16_wgrad_recipe(mxq, skewed, clamped, fused):
    """The expert layer under the BF16-wgrad recipe against the MXFP8 recipe
    on the same inputs: Y, dA, dscale, the dense [dgate | dup], its rowwise
    MXFP8 form and dX are the same bits (the same kernels on the same data);
    the recomputed bf16 activation equals the oracle's activation of the
    saved H13 bit for bit, and both bf16 wgrads are within the GEMM tolerance
    of the oracle's K-grouped GEMM of the GPU's operands."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    T, H, E, k, I = 64, 128, 16, 2, 128
    moe = W.moe_layer(7, skewed=skewed, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    splits = moe["splits"]
    R = int(splits.sum())
    ro_np = O.splits_to_offsets(splits.numpy())[0]
    x, sc, dy = moe["x_perm"].cuda(), moe["scale"].cuda(), W.moe_grad(R, H, seed=7).cuda()
    layers = {}
    for recipe in ("mxfp8", "bf16_wgrad"):
        L = Layer(splits.cuda(), moe["w13"].cuda(), moe["w2"].cuda(), clamped=clamped, fused_fc1=fused,
                  recipe=recipe)
        y = L.forward(x, sc)
        L.backward(dy)
        torch.cuda.synchronize()
        layers[recipe] = (L, y)
    (lm, ym), (lb, yb) = layers["mxfp8"], layers["bf16_wgrad"]
    assert torch.equal(ym.view(torch.int16), yb.view(torch.int16))
    gm, gb = lm.grads, lb.grads
    for key in ("da", "dd", "dx"):
        assert torch.equal(gm[key].view(torch.int16), gb[key].view(torch.int16)), key
    for key in ("dq_r", "dqs_r"):
        assert torch.equal(rowmajor(gm[key]), rowmajor(gb[key])), key
    assert torch.equal(gm["dscale"].view(torch.int32), gb["dscale"].view(torch.int32))
    assert gb["dy_c"].numel() == 0 and gb["dq_c"].numel() == 0 and lb.saved["a_c"].numel() == 0
    # the recomputed activation, in logical column order
    h13 = bits(lb.saved["h13"])
    if fused:
        g, u = O.glu_split(h13, 128)
    else:
        g, u = h13[:, :I], h13[:, I:]
    a_ref = O.swiglu_fwd(g, u, moe["scale"].numpy(), O.CLAMPED_SWIGLU if clamped else O.SWIGLU, 7.0)
    a_got = bits(gb["a_bf16"])
    assert np.array_equal(a_got, a_ref)
    # the two bf16 wgrads
    dyb, ddb, xb = bits(dy), bits(gb["dd"]), bits(moe["x_perm"])
    ref2 = O.grouped_gemm("k", ro_np, H, I, 0, O.Operand("bf16", dyb, 0, 1, H), O.Operand("bf16", a_got, 0, 1, I),
                          "bf16")
    check_close(out_np(lb.grads["dw2"]), ref_np(ref2, "bf16"))
    ref13 = O.grouped_gemm("k", ro_np, 2 * I, H, 0, O.Operand("bf16", ddb, 0, 1, 2 * I),
                           O.Operand("bf16", xb, 0, 1, H), "bf16")
    check_close(out_np(lb.grads["dw13"]), ref_np(ref13, "bf16"))


def many_splits(rng, G, busy, top):
    splits = [0] * G
    for g in rng.choice(G, busy, replace=False):
        splits[int(g)] = int(rng.integers(1, top))
    splits[G - 1] = 257
    return splits


def test_bf16_many_groups_scan_path(mxq):
    """More groups than the LDS group tables hold (1024): the launches look
    every tile's group up by scanning the offsets (NN) or read them from
    global memory (TN, static order: the dynamic order needs the tables);
    mostly empty groups, a few of several tiles."""
    rng = np.random.default_rng(37)
    G, N, K = 1500, 48, 96
    splits = many_splits(rng, G, 30, 300)
    ro, _, ro_np = offsets(mxq, splits)
    R = sum(splits)
    A = rand_bf16(rng, (R, K))
    B = rand_bf16(rng, (G, K, N), 0.05)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, O.Operand("bf16", A, 0, K, 1), O.Operand("bf16", B, K * N, 1, N), "bf16")
    for max_wg in (0, 8):
        out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NN, ro, dev(A), dev(B), out, max_workgroups=max_wg)
        torch.cuda.synchronize()
        check_close(out_np(out), ref_np(ref, "bf16"))
    M, N2 = 32, 48
    At = rand_bf16(rng, (R, M))
    Bt = rand_bf16(rng, (R, N2), 0.05)
    ref = O.grouped_gemm("k", ro_np, M, N2, 0, O.Operand("bf16", At, 0, 1, M), O.Operand("bf16", Bt, 0, 1, N2), "f32")
    out = torch.full((G, M, N2), 7.0, dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, dev(At), dev(Bt), out)
    torch.cuda.synchronize()
    got = out_np(out)
    check_close(got, ref_np(ref, "f32"))
    empty = [g for g in range(G) if splits[g] == 0]
    assert np.all(got[empty] == 0)
