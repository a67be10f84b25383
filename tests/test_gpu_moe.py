"""GPU parity of the whole expert-layer hot path (swiglu_mxfp8_quant_amd.moe):
every stage of one forward + backward is checked against the CPU oracle run on
that stage's GPU inputs, so layouts, strides, group offsets and the handoffs
between kernels are all covered.

Pages: "Activation + GroupedLinear Fusion for MOE and other MOE optimizations"
(Sequence Diagram: forward and backward of the grouped expert MLP with the
fused activation); NVIDIA/TransformerEngine pull 3224 (grouped GEMM over
expert row groups).  Small Qwen3-MoE-shaped layers: uniform top-k routing
with the plain SwiGLU, and skewed Zipf routing (empty experts) with the plain
and the clamped SwiGLU; and the full-size layer (65,536 routed rows, 128
experts) in the benchmark's launch configuration, checked on sampled experts,
rows and columns.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import rowmajor

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


@pytest.mark.parametrize("skewed,clamped", [(False, False), (True, False), (True, True)])
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
    same(u8(rowmajor(s["a_r"])), rc, "act fwd row codes")
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
    same(u8(rowmajor(gr["dy_r"])), q[0], "dY row codes")
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
    same(u8(rowmajor(gr["dq_r"])), brc, "act bwd row codes")
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


# ------------------------------------------------------------------ full size, sampled

def _pick_experts(splits):
    """The largest expert, the smallest non-empty one, and the one whose last
    256-row tile is closest to half full."""
    nz = [g for g in range(len(splits)) if splits[g] > 0]
    big = max(nz, key=lambda g: (splits[g], -g))
    small = min(nz, key=lambda g: (splits[g], g))
    rest = [g for g in nz if g not in (big, small)]
    mid = max(rest, key=lambda g: (min(splits[g] % 256, 256 - splits[g] % 256), -g))
    return [big, small, mid]


def _rows(r0, r1):
    """The first and last 40 rows of a group (every row of a small one)."""
    if r1 - r0 <= 80:
        return np.arange(r0, r1)
    return np.concatenate([np.arange(r0, r0 + 40), np.arange(r1 - 40, r1)])


def _host(t, rows=None):
    x = t if rows is None else t[torch.as_tensor(rows, device=t.device)]
    return bits(x) if x.dtype == torch.bfloat16 else u8(x)


@pytest.mark.parametrize("routing", ["uniform_plain", "zipf_plain", "zipf_clamped"])
def test_full_size_layer_sampled(mxq, routing):
    """The expert layer at its full size (8192 tokens, top-8: 65,536 routed rows,
    hidden 2048, 128 experts, intermediate 768), forward + backward through
    the same calls the benchmark times.  For the largest expert, the smallest
    non-empty one and one ending mid-tile: each of the six GEMMs on a
    64-column slice that crosses a 256-column tile boundary (M-grouped: the
    first and last 40 rows of the expert; K-grouped: a 64 x 64 block of the
    expert's weight gradient, summed over all its rows), and every
    quantization (activation forward and backward, dY, X, W2, W13) over the
    expert's whole row range, against the oracle on the GPU's own inputs to
    that stage."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    skewed, clamped = routing.startswith("zipf"), routing.endswith("clamped")
    print(routing, flush=True)
    moe = W.moe_layer(0, device="cuda", skewed=skewed)
    cfg = moe["cfg"]
    H, I, E = cfg["hidden"], cfg["inter"], cfg["experts"]
    splits = moe["splits"].cpu().numpy()
    R = int(splits.sum())
    assert R == 65536 and (not skewed or (splits == 0).sum() == 8)
    ro, bo = O.splits_to_offsets(splits)
    kind = O.CLAMPED_SWIGLU if clamped else O.SWIGLU
    layer = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped)
    y = layer.forward(moe["x_perm"], moe["scale"])
    dy = W.moe_grad(R, H, seed=0, device="cuda")
    layer.backward(dy)
    torch.cuda.synchronize()
    s, gr = layer.saved, layer.grads
    scale = moe["scale"].cpu().numpy()
    c16 = lambda c0: slice(c0, c0 + 64)
    for g in _pick_experts(splits):
        r0, r1 = int(ro[g]), int(ro[g + 1])
        b0, b1 = int(bo[g]), int(bo[g + 1])
        S = _rows(r0, r1)
        n = len(S)
        one = np.array([0, n], np.int64)
        print("  expert", g, "rows", r1 - r0, flush=True)
        # FC1 (bf16 NT): columns 224..287 of the (R, 2I) output
        cs = c16(224)
        xs = _host(s["x_perm"], S)
        w13g = bits(moe["w13"][g, cs, :])
        ref = O.grouped_gemm("m", one, 0, 64, H, O.Operand("bf16", xs, 0, H, 1), O.Operand("bf16", w13g, 0, H, 1),
                             "bf16")
        close(_host(s["h13"], S)[:, cs], ref, f"FC1 expert {g}")
        # FC2 (MXFP8 NT): columns 224..287 of (R, H)
        A, As = _host(rowmajor(s["a_r"]), S), _host(s["as_r"], S)
        B, Bs = u8(s["w2q"][g, cs, :]), u8(s["w2s"][g, cs, :])
        ref = O.grouped_gemm("m", one, 0, 64, I, O.Operand("mxfp8", A, 0, I, 1, As, 0, I // 32, 1),
                             O.Operand("mxfp8", B, 0, I, 1, Bs, 0, I // 32, 1), "bf16")
        close(_host(y, S)[:, cs], ref, f"FC2 expert {g}")
        # FC2 dgrad (MXFP8 NN): columns 224..287 of (R, I)
        A, As = _host(rowmajor(gr["dy_r"]), S), _host(gr["dys_r"], S)
        B = np.ascontiguousarray(u8(gr["w2c"][g])[:, cs])
        Bs = np.ascontiguousarray(u8(gr["w2cs"][g])[:, cs])
        ref = O.grouped_gemm("m", one, 0, 64, H, O.Operand("mxfp8", A, 0, H, 1, As, 0, H // 32, 1),
                             O.Operand("mxfp8", B, 0, 1, 64, Bs, 0, 1, 64), "bf16")
        close(_host(gr["da"], S)[:, cs], ref, f"FC2 dgrad expert {g}")
        # FC1 dgrad (MXFP8 NN): columns 224..287 of (R, H)
        A, As = _host(rowmajor(gr["dq_r"]), S), _host(gr["dqs_r"], S)
        B = np.ascontiguousarray(u8(gr["w13c"][g])[:, cs])
        Bs = np.ascontiguousarray(u8(gr["w13cs"][g])[:, cs])
        ref = O.grouped_gemm("m", one, 0, 64, 2 * I, O.Operand("mxfp8", A, 0, 2 * I, 1, As, 0, 2 * I // 32, 1),
                             O.Operand("mxfp8", B, 0, 1, 64, Bs, 0, 1, 64), "bf16")
        close(_host(gr["dx"], S)[:, cs], ref, f"FC1 dgrad expert {g}")
        # the wgrads (MXFP8 TN) over the expert's whole row range
        allr = np.arange(r0, r1)
        grp = np.array([0, r1 - r0], np.int64)
        for name, Ac, Acs, Bc, Bcs, out, ms, ns in (
                ("FC2 wgrad", gr["dy_c"], gr["dys_c"], s["a_c"], s["as_c"], gr["dw2"], c16(224), c16(224)),
                ("FC1 wgrad", gr["dq_c"], gr["dqs_c"], gr["x_c"], gr["xs_c"], gr["dw13"], c16(736), c16(224))):
            A = np.ascontiguousarray(_host(Ac, allr)[:, ms])
            As = np.ascontiguousarray(u8(Acs[b0:b1])[:, ms])
            B = np.ascontiguousarray(_host(Bc, allr)[:, ns])
            Bs = np.ascontiguousarray(u8(Bcs[b0:b1])[:, ns])
            ref = O.grouped_gemm("k", grp, 64, 64, 0, O.Operand("mxfp8", A, 0, 1, 64, As, 0, 1, 64),
                                 O.Operand("mxfp8", B, 0, 1, 64, Bs, 0, 1, 64), "bf16")
            close(bits(out[g, ms, ns]), ref[0], f"{name} expert {g}")
        # activation forward on the expert's rows of the GPU's H13 (one group:
        # colwise blocks restart at the expert's first row)
        h13 = _host(s["h13"], allr)
        rc, cc, rs, cs_, _h = O.swiglu_quantize_fwd(h13[:, :I], h13[:, I:], scale[r0:r1], 3, None, kind, 7.0)
        same(u8(rowmajor(s["a_r"])[r0:r1]), rc, "act fwd row codes")
        same(u8(s["as_r"][r0:r1]), rs, "act fwd row scales")
        same(u8(s["a_c"][r0:r1]), cc, "act fwd col codes")
        same(u8(s["as_c"][b0:b1]), cs_, "act fwd col scales")
        # activation backward on the expert's rows of the GPU's dA and H13
        da = _host(gr["da"], allr)
        b = O.swiglu_quantize_bwd(da, h13[:, :I], h13[:, I:], scale[r0:r1], 3, None, kind, 7.0, want_close=True)
        same(u8(rowmajor(gr["dq_r"])[r0:r1]), b[0], "act bwd row codes")
        same(u8(gr["dqs_r"][r0:r1]), b[2], "act bwd row scales")
        same(u8(gr["dq_c"][r0:r1]), b[1], "act bwd col codes")
        same(u8(gr["dqs_c"][b0:b1]), b[3], "act bwd col scales")
        dd = bits(gr["dd"][r0:r1])
        same(dd[:, :I], b[4], "dgate")
        same(dd[:, I:], b[5], "dup")
        err = np.abs(gr["dscale"][r0:r1].cpu().numpy().astype(np.float64) - b[6])
        assert np.all(err <= b[8] + 1e-30), f"dscale off by {err.max()}"
        # dY (both directions) and X (colwise) over the expert's rows
        q = O.mx_quantize(bits(dy[r0:r1]), 3)
        same(u8(rowmajor(gr["dy_r"])[r0:r1]), q[0], "dY row codes")
        same(u8(gr["dys_r"][r0:r1]), q[2], "dY row scales")
        same(u8(gr["dy_c"][r0:r1]), q[1], "dY col codes")
        same(u8(gr["dys_c"][b0:b1]), q[3], "dY col scales")
        q = O.mx_quantize(_host(s["x_perm"], allr), 2)
        same(u8(gr["x_c"][r0:r1]), q[1], "X col codes")
        same(u8(gr["xs_c"][b0:b1]), q[3], "X col scales")
        # this expert's weights: W2 rowwise along I and colwise along H, W13 colwise along 2I
        q = O.mx_quantize(bits(moe["w2"][g]), 3)
        same(u8(s["w2q"][g]), q[0], "W2 row codes")
        same(u8(s["w2s"][g]), q[2], "W2 row scales")
        same(u8(s["w2c"][g]), q[1], "W2 col codes")
        same(u8(s["w2cs"][g]), q[3], "W2 col scales")
        q = O.mx_quantize(bits(moe["w13"][g]), 2)
        same(u8(gr["w13c"][g]), q[1], "W13 col codes")
        same(u8(gr["w13cs"][g]), q[3], "W13 col scales")
    del layer, moe, dy, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("routing", ["uniform_plain", "zipf_clamped"])
def test_full_size_layer_modes_sampled(mxq, routing):
    """The full-size expert layer (65,536 routed rows, the benchmark's launch
    configuration) with FC1's fused epilogue and under the BF16-wgrad recipe,
    against the plain layer on the same inputs (which the test above checks
    against the oracle):
      * fused FC1: H13, [dgate | dup], its MXFP8 forms and dW13 equal the plain
        layer's bit for bit up to the gate / up column interleave; the MXFP8
        activation, Y, dA, dW2 and dscale equal them outright; dX (its
        contraction runs over 2I in another order) to fp32-sum rounding;
      * the recipe: Y, dA, [dgate | dup], its rowwise MXFP8, dscale and dX
        equal the plain layer's bit for bit; the recomputed bf16 activation
        equals the oracle's on the sampled experts' rows, and each bf16 wgrad
        on a 64 x 64 block over each sampled expert's whole row range is
        within the GEMM tolerance of the oracle's K-grouped GEMM;
      * the recipe with the fused FC1: the recipe's results bit for bit, up
        to the gate / up interleave."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    skewed, clamped = routing.startswith("zipf"), routing.endswith("clamped")
    print(routing, flush=True)
    moe = W.moe_layer(0, device="cuda", skewed=skewed)
    cfg = moe["cfg"]
    H, I = cfg["hidden"], cfg["inter"]
    splits = moe["splits"].cpu().numpy()
    R = int(splits.sum())
    ro, bo = O.splits_to_offsets(splits)
    ncb = int(bo[-1])
    dy = W.moe_grad(R, H, seed=0, device="cuda")
    out = {}
    for mode in ("plain", "fused", "recipe", "fused_recipe"):
        L = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped, fused_fc1=mode.startswith("fused"),
                  recipe="bf16_wgrad" if mode.endswith("recipe") else "mxfp8")
        y = L.forward(moe["x_perm"], moe["scale"])
        L.backward(dy)
        torch.cuda.synchronize()
        out[mode] = (L, y)
        print("  ran", mode, flush=True)
    (lp, yp), (lf, yf), (lr, yr), (lfr, yfr) = out["plain"], out["fused"], out["recipe"], out["fused_recipe"]
    sp, gp = lp.saved, lp.grads

    def eq(a, b, what):
        a, b = rowmajor(a), rowmajor(b)
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b), what

    # fused FC1: logical column j of 2I at interleaved column perm[j]
    j = np.arange(2 * I)
    g = j % I
    perm = torch.as_tensor(np.where(j < I, (g // 128) * 256 + g % 128, (g // 128) * 256 + 128 + g % 128),
                           device="cuda")
    sf, gf = lf.saved, lf.grads
    eq(sp["h13"], sf["h13"][:, perm], "fused: H13")
    for k in ("a_r", "a_c", "as_r"):
        eq(sp[k], sf[k], f"fused: {k}")
    eq(sp["as_c"][:ncb], sf["as_c"][:ncb], "fused: as_c")
    eq(yp, yf, "fused: Y")
    for k in ("da", "dw2", "dscale"):
        eq(gp[k], gf[k], f"fused: {k}")
    eq(gp["dd"], gf["dd"][:, perm], "fused: [dgate | dup]")
    eq(gp["dq_r"], rowmajor(gf["dq_r"])[:, perm], "fused: dact rowwise codes")
    eq(gp["dq_c"], gf["dq_c"][:, perm], "fused: dact colwise codes")
    eq(gp["dqs_c"][:ncb], gf["dqs_c"][:ncb][:, perm], "fused: dact colwise scales")
    eq(gp["dw13"], gf["dw13"][:, perm, :], "fused: dW13")
    a, b = gp["dx"].double(), gf["dx"].double()
    assert torch.all((a - b).abs() <= 1e-2 * a.abs().max() + 1e-2 * a.abs()).item(), "fused: dX"
    # the recipe
    gr_ = lr.grads
    eq(yp, yr, "recipe: Y")
    for k in ("da", "dd", "dq_r", "dqs_r", "dscale", "dx"):
        eq(gp[k], gr_[k], f"recipe: {k}")
    kind = O.CLAMPED_SWIGLU if clamped else O.SWIGLU
    scale = moe["scale"].cpu().numpy()
    dyb_dev = dy
    for gi in _pick_experts(splits):
        r0, r1 = int(ro[gi]), int(ro[gi + 1])
        allr = np.arange(r0, r1)
        h13 = _host(lr.saved["h13"], allr)
        a_ref = O.swiglu_fwd(h13[:, :I], h13[:, I:], scale[r0:r1], kind, 7.0)
        a_got = _host(gr_["a_bf16"], allr)
        same(a_got, a_ref, f"recipe: bf16 activation, expert {gi}")
        grp = np.array([0, r1 - r0], np.int64)
        for name, Ah, Bh, outt, ms, ns in (
                ("FC2 wgrad", _host(dyb_dev, allr), a_got, gr_["dw2"], slice(224, 288), slice(224, 288)),
                ("FC1 wgrad", _host(gr_["dd"], allr), _host(moe["x_perm"], allr), gr_["dw13"], slice(736, 800),
                 slice(224, 288))):
            A = np.ascontiguousarray(Ah[:, ms])
            B = np.ascontiguousarray(Bh[:, ns])
            ref = O.grouped_gemm("k", grp, 64, 64, 0, O.Operand("bf16", A, 0, 1, 64), O.Operand("bf16", B, 0, 1, 64),
                                 "bf16")
            close(bits(outt[gi, ms, ns]), ref[0], f"recipe: {name} expert {gi}")
    # the recipe with the fused FC1 (rowwise cast in the epilogue): the
    # recipe's results up to the interleave of the gate / up columns
    gfr = lfr.grads
    eq(yr, yfr, "fused recipe: Y")
    eq(lr.saved["a_r"], lfr.saved["a_r"], "fused recipe: a_r")
    eq(lr.saved["h13"], lfr.saved["h13"][:, perm], "fused recipe: H13")
    for k in ("da", "dscale", "dw2", "a_bf16"):
        eq(gr_[k], gfr[k], f"fused recipe: {k}")
    eq(gr_["dd"], gfr["dd"][:, perm], "fused recipe: [dgate | dup]")
    eq(gr_["dq_r"], rowmajor(gfr["dq_r"])[:, perm], "fused recipe: dact rowwise codes")
    eq(gr_["dw13"], gfr["dw13"][:, perm, :], "fused recipe: dW13")
