"""GPU parity of the whole expert-layer hot path (swiglu_mxfp8_quant_amd.moe):
every stage of one forward + backward is checked against the CPU oracle run on
that stage's GPU inputs, so layouts, strides, group offsets and the handoffs
between kernels are all covered.

Pages: "Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
(Sequence Diagram: forward and backward of the grouped expert MLP with the
fused activation); NVIDIA/TransformerEngine pull 3224 (grouped GEMM over
expert row groups).  Small Qwen3-MoE-shaped layers: uniform top-k routing
with the plain SwiGLU, and skewed Zipf routing (empty experts) with the
clamped SwiGLU.
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


def bits(t):
    return W.bf16_bits(t)


def u8(t):
    return t.cpu().numpy()


def f64_bf16(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def close(got_bf16_bits, ref_bf16_bits, what):
    g, r = f64_bf16(got_bf16_bits), f64_bf16(ref_bf16_bits)
    err = np.abs(g - r)
    assert np.all(err <= 1e-2 + 2e-2 * np.abs(r)), f"{what}: max err {err.max()}"


def same(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    bad = got != ref
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} differ"


@pytest.mark.parametrize("skewed,clamped", [(False, False), (True, True)])
def test_layer_forward_backward(mxq, skewed, clamped):
    from swiglu_mxfp8_quant_amd.moe import Layer
    T, H, E, k, I = 64, 128, 16, 2, 64
    moe = W.moe_layer(3, skewed=skewed, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    splits = moe["splits"]
    R = int(splits.sum())
    if skewed:
        assert (splits == 0).sum() >= 2
    ro, bo = O.splits_to_offsets(splits.numpy())
    kind = O.CLAMPED_SWIGLU if clamped else O.SWIGLU

    layer = Layer(splits.cuda(), moe["w13"].cuda(), moe["w2"].cuda(), clamped=clamped)
    x, sc = moe["x_perm"].cuda(), moe["scale"].cuda()
    y = layer.forward(x, sc)
    dy = W.moe_grad(R, H, seed=3).cuda()
    layer.backward(dy)
    torch.cuda.synchronize()
    s, gr = layer.saved, layer.grads
    scale = moe["scale"].numpy()
    xb, w13b, w2b = bits(moe["x_perm"]), bits(moe["w13"]), bits(moe["w2"])

    # FC1 (bf16, M-grouped)
    h13 = bits(s["h13"])
    ref = O.grouped_gemm("m", ro, 0, 2 * I, H, O.Operand("bf16", xb, 0, H, 1),
                         O.Operand("bf16", w13b, 2 * I * H, H, 1), "bf16")
    close(h13, ref, "FC1")

    # fused activation forward on the GPU's H13: rowwise + per-expert colwise
    rc, cc, rs, cs, _h = O.swiglu_quantize_fwd(h13[:, :I], h13[:, I:], scale, 3, ro, kind, 7.0)
    nb = cs.shape[0]
    same(u8(s["a_r"]), rc, "act fwd row codes")
    same(u8(s["as_r"]), rs, "act fwd row scales")
    same(u8(s["a_c"]), cc, "act fwd col codes")
    same(u8(s["as_c"])[:nb], cs, "act fwd col scales")

    # W2 rowwise quantization and FC2 (MXFP8 NT)
    wq = O.mx_quantize(w2b.reshape(E * H, I), 1)
    same(u8(s["w2q"]).reshape(E * H, I), wq[0], "W2 row codes")
    same(u8(s["w2s"]).reshape(E * H, I // 32), wq[2], "W2 row scales")
    ref = O.grouped_gemm("m", ro, 0, H, I, O.Operand("mxfp8", rc, 0, I, 1, rs, 0, I // 32, 1),
                         O.Operand("mxfp8", wq[0].reshape(E, H, I), H * I, I, 1,
                                   wq[2].reshape(E, H, I // 32), H * (I // 32), I // 32, 1), "bf16")
    close(bits(y), ref, "FC2")

    # backward: dY quantized both ways (colwise per expert)
    dyb = bits(dy)
    q = O.mx_quantize(dyb, 3, ro)
    same(u8(gr["dy_r"]), q[0], "dY row codes")
    same(u8(gr["dys_r"]), q[2], "dY row scales")
    same(u8(gr["dy_c"]), q[1], "dY col codes")
    same(u8(gr["dys_c"])[:q[3].shape[0]], q[3], "dY col scales")

    # FC2 dgrad (NN): dA = dY . W2_g with W2 colwise per expert (32x1 blocks along H)
    w2c = O.mx_quantize(w2b.reshape(E * H, I), 2, np.arange(E + 1, dtype=np.int64) * H)
    same(u8(gr["w2c"]).reshape(E * H, I), w2c[1], "W2 col codes")
    same(u8(gr["w2cs"]).reshape(E * H // 32, I), w2c[3], "W2 col scales")
    ref = O.grouped_gemm("m", ro, 0, I, H, O.Operand("mxfp8", q[0], 0, H, 1, q[2], 0, H // 32, 1),
                         O.Operand("mxfp8", w2c[1].reshape(E, H, I), H * I, 1, I,
                                   w2c[3].reshape(E, H // 32, I), (H // 32) * I, 1, I), "bf16")
    close(bits(gr["da"]), ref, "FC2 dgrad")

    # FC2 wgrad (TN): dW2_g = dY_g^T A_g, empty experts -> 0
    ref = O.grouped_gemm("k", ro, H, I, 0, O.Operand("mxfp8", q[1], 0, 1, H, q[3], 0, 1, H),
                         O.Operand("mxfp8", cc, 0, 1, I, cs, 0, 1, I), "bf16")
    close(bits(gr["dw2"]), ref, "FC2 wgrad")

    # fused activation backward on the GPU's dA and H13
    da = bits(gr["da"])
    b = O.swiglu_quantize_bwd(da, h13[:, :I], h13[:, I:], scale, 3, ro, kind, 7.0, want_close=True)
    brc, bcc, brs, bcs, dg, du, ds, _close, tol = b
    same(u8(gr["dq_r"]), brc, "act bwd row codes")
    same(u8(gr["dqs_r"]), brs, "act bwd row scales")
    same(u8(gr["dq_c"]), bcc, "act bwd col codes")
    same(u8(gr["dqs_c"])[:bcs.shape[0]], bcs, "act bwd col scales")
    dd = bits(gr["dd"])
    same(dd[:, :I], dg, "dgate")
    same(dd[:, I:], du, "dup")
    err = np.abs(gr["dscale"].cpu().numpy().astype(np.float64) - ds)
    assert np.all(err <= tol + 1e-30), f"dscale off by {err.max()}"

    # FC1 dgrad (NN) with W13 colwise per expert (32x1 blocks along 2I)
    w13c = O.mx_quantize(w13b.reshape(E * 2 * I, H), 2, np.arange(E + 1, dtype=np.int64) * (2 * I))
    same(u8(gr["w13c"]).reshape(E * 2 * I, H), w13c[1], "W13 col codes")
    same(u8(gr["w13cs"]).reshape(E * 2 * I // 32, H), w13c[3], "W13 col scales")
    ref = O.grouped_gemm("m", ro, 0, H, 2 * I, O.Operand("mxfp8", brc, 0, 2 * I, 1, brs, 0, 2 * I // 32, 1),
                         O.Operand("mxfp8", w13c[1].reshape(E, 2 * I, H), 2 * I * H, 1, H,
                                   w13c[3].reshape(E, 2 * I // 32, H), (2 * I // 32) * H, 1, H), "bf16")
    close(bits(gr["dx"]), ref, "FC1 dgrad")

    # FC1 wgrad (TN): dW13_g = dact_g^T X_g with X colwise per expert
    xq = O.mx_quantize(xb, 2, ro)
    same(u8(gr["x_c"]), xq[1], "X col codes")
    same(u8(gr["xs_c"])[:xq[3].shape[0]], xq[3], "X col scales")
    ref = O.grouped_gemm("k", ro, 2 * I, H, 0, O.Operand("mxfp8", bcc, 0, 1, 2 * I, bcs, 0, 1, 2 * I),
                         O.Operand("mxfp8", xq[1], 0, 1, H, xq[3], 0, 1, H), "bf16")
    close(bits(gr["dw13"]), ref, "FC1 wgrad")
