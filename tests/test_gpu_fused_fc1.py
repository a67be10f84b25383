"""GPU parity of the FC1 grouped GEMM with the row-scaled SwiGLU + MXFP8 in
its epilogue (mxq_grouped_gemm_swiglu), through the C ABI.

Page "Activation + GroupedLinear Fusion for MOE and other MOE
optimizations", discussion: the activation and its grouped quantization
fused with the grouped linear (the FC1 - activation - FC2 module).  The
checks: the bf16 product equals the plain grouped GEMM's bit for bit (same
kernel arithmetic), it is within the GEMM tolerance of the oracle's grouped
GEMM, and the MXFP8 activation equals, bit for bit, the oracle's row-scaled
SwiGLU + quantizer applied to that product (and the unfused library call on
it), rowwise and per-expert colwise.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import compare_mx, rowblock_of, rowmajor

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


def run_case(m, splits, H, I, clamped, seed, w_std=0.05, max_wg=0, with_scale=True, dirs=3):
    G = len(splits)
    R = sum(splits)
    ro, bo, _ = m.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    ro_np = O.splits_to_offsets(splits)[0]
    x = W._normal((R, H), 1.0, seed, 50, "cuda")
    w13 = W._normal((G, 2 * I, H), w_std, seed, 51, "cuda")
    w13i = m.interleave_rows(w13, 128)
    sc = W.row_scale(R, seed=seed, device="cuda") if with_scale else None
    out = torch.empty((R, 2 * I), dtype=torch.bfloat16, device="cuda")
    ncb = O.colwise_scale_rows(R, ro_np)
    f = m.grouped_gemm_swiglu(ro, x, w13i, out, sc, bool(dirs & 1), bool(dirs & 2), block_off=bo, n_col_blocks=ncb,
                              clamped=clamped, max_workgroups=max_wg)
    plain = torch.empty_like(out)
    m.grouped_gemm(m.GEMM_NT, ro, x, w13i, plain, max_workgroups=max_wg)
    unf = m.swiglu_quantize_fwd(out[:, :I], out[:, 128:128 + I], sc, bool(dirs & 1), bool(dirs & 2), ro, bo,
                                n_col_blocks=ncb, clamped=clamped, interleave=128)
    torch.cuda.synchronize()
    # the bf16 product: the plain GEMM's bits
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))
    # the activation: the oracle on the GPU's product, and the unfused call
    hb = bits(out)
    g, u = O.glu_split(hb, 128)
    kind = O.CLAMPED_SWIGLU if clamped else O.SWIGLU
    rc, cc, rs, cs, _h, close = O.swiglu_quantize_fwd(g, u, None if sc is None else sc.cpu().numpy(), dirs, ro_np,
                                                      kind, 7.0, want_close=True)
    rep = {}
    if dirs & 1:
        compare_mx("fused.row", u8(f[0]), u8(f[2]), rc, rs, close != 0, True, report=rep)
        assert torch.equal(f[0], unf[0]) and torch.equal(f[2], unf[2])
    if dirs & 2:
        compare_mx("fused.col", u8(f[1]), u8(f[3]), cc, cs, close != 0, False, rowblock_of(R, ro_np), report=rep)
        assert torch.equal(f[1], unf[1]) and torch.equal(f[3], unf[3])
    bad = {k: v for k, v in rep.items() if v}
    assert not bad, bad
    return out, x, w13, ro_np


@pytest.mark.parametrize("clamped", [False, True])
@pytest.mark.parametrize("max_wg", [0, 8])
def test_fused_fc1_grouped(mxq, clamped, max_wg):
    """Several experts (one empty, one of a single row, tails of every size),
    two 256-column tiles of the activation, chained tiles with max_wg = 8."""
    splits = [70, 0, 300, 1, 129, 33, 256]
    run_case(mxq, splits, 256, 384, clamped, seed=3 + max_wg, w_std=0.2 if clamped else 0.05, max_wg=max_wg)


@pytest.mark.parametrize("dirs", [1, 2])
def test_fused_fc1_one_direction_no_scale(mxq, dirs):
    run_case(mxq, [100, 31, 0, 65], 128, 256, False, seed=7, with_scale=False, dirs=dirs)


def test_fused_fc1_against_oracle_gemm(mxq):
    """The bf16 product against the oracle's grouped GEMM (fp32 accumulation,
    rel 2e-2 / abs 1e-2), de-interleaved: gate and up columns land where the
    interleaved weight puts them."""
    splits = [40, 0, 97]
    H, I = 192, 256
    out, x, w13, ro_np = run_case(mxq, splits, H, I, False, seed=9)
    G = len(splits)
    xb, wb = bits(x), bits(w13)
    ref = O.grouped_gemm("m", ro_np, 0, 2 * I, H, O.Operand("bf16", xb, 0, H, 1),
                         O.Operand("bf16", wb, 2 * I * H, H, 1), "bf16")
    ref = O.glu_join(ref[:, :I], ref[:, I:], 128)   # the interleaved column order
    got = (bits(out).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    refv = (ref.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(got - refv) <= 1e-2 + 2e-2 * np.abs(refv))
    assert G == 3


def test_fused_fc1_expert_layer_shape(mxq):
    """The expert layer's FC1 at full size (65,536 routed rows, 128 experts,
    hidden 2048, intermediate 768), both directions, against the unfused
    library call bit for bit and, on the largest expert's rows, the oracle."""
    moe = W.moe_layer(0, device="cuda", skewed=True)
    splits = moe["splits"]
    R, H, I, G = int(splits.sum()), 2048, 768, 128
    ro, bo, _ = mxq.splits_to_offsets(splits)
    ro_np, bo_np = O.splits_to_offsets(splits.cpu().numpy())
    w13i = mxq.interleave_rows(moe["w13"], 128)
    out = torch.empty((R, 2 * I), dtype=torch.bfloat16, device="cuda")
    ncb = int(bo_np[-1])
    f = mxq.grouped_gemm_swiglu(ro, moe["x_perm"], w13i, out, moe["scale"], True, True, block_off=bo,
                                n_col_blocks=ncb, clamped=True)
    unf = mxq.swiglu_quantize_fwd(out[:, :I], out[:, 128:128 + I], moe["scale"], True, True, ro, bo,
                                  n_col_blocks=ncb, clamped=True, interleave=128)
    torch.cuda.synchronize()
    for a, b in zip(f, unf):
        assert torch.equal(a, b)
    g = int(np.argmax(np.diff(ro_np)))
    r0, r1, b0, b1 = int(ro_np[g]), int(ro_np[g + 1]), int(bo_np[g]), int(bo_np[g + 1])
    hb = bits(out[r0:r1])
    gg, uu = O.glu_split(hb, 128)
    rc, cc, rs, cs, _h = O.swiglu_quantize_fwd(gg, uu, moe["scale"][r0:r1].cpu().numpy(), 3, None,
                                               O.CLAMPED_SWIGLU, 7.0)
    assert np.array_equal(u8(f[0][r0:r1]), rc) and np.array_equal(u8(f[2][r0:r1]), rs)
    assert np.array_equal(u8(f[1][r0:r1]), cc) and np.array_equal(u8(f[3][b0:b1]), cs)


@pytest.mark.parametrize("skewed,clamped", [(False, False), (True, True)])
def test_layer_fused_fc1_matches_unfused(mxq, skewed, clamped):
    """The expert layer with FC1's fused epilogue against the unfused layer on
    the same weights: the forward (H13 up to the column interleave, the MXFP8
    activation, Y) and the backward's dA, dW2, dscale bit for bit; [dgate |
    dup], the MXFP8 dact and dW13 bit for bit after undoing the interleave;
    dX (whose contraction runs over 2I in another order) to fp32-sum
    rounding."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    T, H, E, k, I = 64, 128, 16, 2, 256
    moe = W.moe_layer(5, skewed=skewed, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    splits = moe["splits"]
    R = int(splits.sum())
    x, sc, dy = moe["x_perm"].cuda(), moe["scale"].cuda(), W.moe_grad(R, H, seed=5).cuda()
    outs = []
    for fused in (False, True):
        layer = Layer(splits.cuda(), moe["w13"].cuda(), moe["w2"].cuda(), clamped=clamped, fused_fc1=fused)
        y = layer.forward(x, sc)
        dx, dw13, dw2, dscale = layer.backward(dy)
        torch.cuda.synchronize()
        outs.append((layer, y, dx, dw13, dw2, dscale))
    (lp, yp, dxp, dw13p, dw2p, dsp), (lf, yf, dxf, dw13f, dw2f, dsf) = outs
    # logical column j of the interleaved 2I columns: gate j < I, up j >= I
    j = np.arange(2 * I)
    g = j % I
    perm = np.where(j < I, (g // 128) * 256 + g % 128, (g // 128) * 256 + 128 + g % 128)
    sp, sf = lp.saved, lf.saved
    assert np.array_equal(bits(sp["h13"]), bits(sf["h13"])[:, perm])
    # colwise scale rows past the per-expert blocks are padding of the bound
    ncb = O.colwise_scale_rows(R, O.splits_to_offsets(splits.numpy())[0])
    for key in ("a_r", "a_c", "as_r"):
        assert torch.equal(rowmajor(sp[key]), rowmajor(sf[key])), key
    assert torch.equal(sp["as_c"][:ncb], sf["as_c"][:ncb])
    assert torch.equal(yp.view(torch.int16), yf.view(torch.int16))
    gp, gf = lp.grads, lf.grads
    assert torch.equal(gp["da"].view(torch.int16), gf["da"].view(torch.int16))
    assert torch.equal(dw2p.view(torch.int16), dw2f.view(torch.int16))
    assert torch.equal(dsp.view(torch.int32), dsf.view(torch.int32))
    assert np.array_equal(bits(gp["dd"]), bits(gf["dd"])[:, perm])
    assert np.array_equal(u8(rowmajor(gp["dq_r"])), u8(rowmajor(gf["dq_r"]))[:, perm])
    assert np.array_equal(u8(gp["dq_c"]), u8(gf["dq_c"])[:, perm])
    bperm = perm[::32] // 32      # 32-column blocks move whole
    assert np.array_equal(u8(gp["dqs_r"]), u8(gf["dqs_r"])[:, bperm])
    assert np.array_equal(u8(gp["dqs_c"])[:ncb], u8(gf["dqs_c"])[:ncb][:, perm])
    assert np.array_equal(bits(dw13p), bits(dw13f)[:, perm, :])
    a, b = dxp.double().cpu().numpy(), dxf.double().cpu().numpy()
    assert np.all(np.abs(a - b) <= 1e-2 * np.abs(a).max() + 1e-2 * np.abs(a)), np.abs(a - b).max()


def test_fused_fc1_many_groups_scan_path(mxq):
    """More groups than the LDS group tables hold (1024): the fused epilogue
    in the launches that scan the offsets for every tile's group (and find
    each tile's colwise scale row through block_off)."""
    rng = np.random.default_rng(41)
    G = 1100
    splits = [0] * G
    for g in rng.choice(G, 12, replace=False):
        splits[int(g)] = int(rng.integers(1, 300))
    splits[G - 1] = 290
    run_case(mxq, splits, H=96, I=128, clamped=False, seed=41)
