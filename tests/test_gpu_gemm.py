"""GPU parity of the grouped GEMM (bf16 and MXFP8; M-grouped with B
contiguous or strided along the contraction, and K-grouped) against the CPU
oracle, through the C ABI.

Pages: NVIDIA/TransformerEngine pull 3224 and "[PyTorch] GroupedTensor
integration" (one grouped GEMM over per-expert row groups), "Activation +
GroupedLinear Fusion for MOE and other MOE optimizations" (Sequence Diagram:
forward, dgrad, wgrad).  Tolerance: |gpu - oracle| <= 1e-2 + 2e-2 |oracle|
on identical quantized operands (fp32 accumulation in a different order);
the integer-exact case is compared bit for bit.
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


def rand_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38
    c[(c & 0x78) == 0x78] &= 0xF7      # keep magnitudes moderate (exponent field <= 14)
    return c


def rand_scales(rng, shape, lo=118, hi=130):
    return rng.integers(lo, hi, shape).astype(np.uint8)


def rand_bf16(rng, shape, std=1.0):
    return W.bf16_bits(torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16))


def to_dev(x):
    if x.dtype == np.uint16:
        return W.from_bits(x, "cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def out_np(t):
    if t.dtype == torch.bfloat16:
        return (W.bf16_bits(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def ref_np(o, out_dtype):
    if out_dtype == "bf16":
        return (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return o.astype(np.float64)


def check_close(got, ref):
    err = np.abs(got - ref)
    tol = 1e-2 + 2e-2 * np.abs(ref)
    assert np.all(err <= tol), f"max err {err.max()} at {np.unravel_index(np.argmax(err - tol), err.shape)}"


def offsets(mxq, splits):
    ro, bo, _ = mxq.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    return ro, bo, *O.splits_to_offsets(splits)


SPLITS = [5, 0, 17, 130, 1, 64, 0, 40]


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_nt_bf16(mxq, out_dtype):
    rng = np.random.default_rng(1)
    ro, bo, ro_np, _ = offsets(mxq, SPLITS)
    R, N, K, G = sum(SPLITS), 272, 192, len(SPLITS)
    A = rand_bf16(rng, (R, K))
    B = rand_bf16(rng, (G, N, K), 0.05)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, O.Operand("bf16", A, 0, K, 1), O.Operand("bf16", B, N * K, K, 1), out_dtype)
    out = torch.empty((R, N), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out)
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, out_dtype))


def qrows(rng, shape, std=1.0):
    """Rowwise MXFP8 (codes, scales) of an N(0, std) bf16 matrix, by the oracle."""
    q = O.mx_quantize(rand_bf16(rng, shape, std), 1)
    return q[0], q[2]


def qcols(rng, shape, row_off=None, std=1.0):
    """Colwise MXFP8 (codes, scales) of an N(0, std) bf16 matrix, by the oracle."""
    q = O.mx_quantize(rand_bf16(rng, shape, std), 2, row_off)
    return q[1], q[3]


@pytest.mark.parametrize("K", [128, 352])
def test_nt_mxfp8(mxq, K):
    rng = np.random.default_rng(2)
    ro, bo, ro_np, _ = offsets(mxq, SPLITS)
    R, N, G = sum(SPLITS), 144, len(SPLITS)
    A, As = qrows(rng, (R, K))
    Bl = [qrows(rng, (N, K), 0.05) for _ in range(G)]
    B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = O.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "f32")
    out = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs))
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, "f32"))


def test_nn_mxfp8(mxq):
    rng = np.random.default_rng(3)
    ro, bo, ro_np, _ = offsets(mxq, SPLITS)
    R, N, K, G = sum(SPLITS), 176, 288, len(SPLITS)
    A, As = qrows(rng, (R, K))
    Bl = [qcols(rng, (K, N), None, 0.05) for _ in range(G)]
    B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = O.Operand("mxfp8", B, K * N, 1, N, Bs, (K // 32) * N, 1, N)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "bf16")
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs))
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, "bf16"))


@pytest.mark.parametrize("accumulate", [False, True])
def test_tn_mxfp8(mxq, accumulate):
    rng = np.random.default_rng(4)
    splits = [33, 0, 31, 200, 1, 0, 64]
    ro, bo, ro_np, bo_np = offsets(mxq, splits)
    R, M, N, G = sum(splits), 160, 144, len(splits)
    A, As = qcols(rng, (R, M), ro_np)
    B, Bs = qcols(rng, (R, N), ro_np, 0.01)
    opA = O.Operand("mxfp8", A, 0, 1, M, As, 0, 1, M)
    opB = O.Operand("mxfp8", B, 0, 1, N, Bs, 0, 1, N)
    base = (rng.standard_normal((G, M, N)) * 0.5).astype(np.float32)
    ref = O.grouped_gemm("k", ro_np, M, N, 0, opA, opB, "f32", out=base.copy() if accumulate else None,
                         accumulate=accumulate)
    out = torch.from_numpy(base.copy()).cuda() if accumulate else torch.full((G, M, N), 7.0, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs), block_off=bo,
                     accumulate=accumulate)
    torch.cuda.synchronize()
    got = out_np(out)
    check_close(got, ref_np(ref, "f32"))
    if not accumulate:
        assert np.all(got[1] == 0) and np.all(got[5] == 0)      # empty groups write zeros


# One large group among small and empty ones: the K-grouped launch takes its
# tiles largest group first from the workspace counter (7 dealt per workgroup,
# the rest taken as workgroups finish), then the empty groups' tiles.
SKEW_SPLITS = [1300, 0, 3, 0, 40, 7, 0, 90, 1, 1, 2, 300, 0, 5, 64, 0, 33, 2, 0, 150]


_SKEW_CACHE = {}


def skew_case(accumulate):
    """Inputs and the oracle's result of the skewed K-grouped case (computed
    once per output kind: the oracle is the slow part)."""
    if accumulate not in _SKEW_CACHE:
        rng = np.random.default_rng(23)
        splits = SKEW_SPLITS
        ro_np = O.splits_to_offsets(splits)[0]
        R, M, N, G = sum(splits), 768, 512, len(splits)
        A, As = qcols(rng, (R, M), ro_np)
        B, Bs = qcols(rng, (R, N), ro_np, 0.01)
        opA = O.Operand("mxfp8", A, 0, 1, M, As, 0, 1, M)
        opB = O.Operand("mxfp8", B, 0, 1, N, Bs, 0, 1, N)
        base = (rng.standard_normal((G, M, N)) * 0.5).astype(np.float32)
        ref = O.grouped_gemm("k", ro_np, M, N, 0, opA, opB, "f32" if accumulate else "bf16",
                             out=base.copy() if accumulate else None, accumulate=accumulate)
        _SKEW_CACHE[accumulate] = (A, As, B, Bs, base, ref)
    return _SKEW_CACHE[accumulate]


@pytest.mark.parametrize("max_wg", [8, 0])
@pytest.mark.parametrize("accumulate", [False, True])
def test_tn_skewed_dynamic_order(mxq, accumulate, max_wg):
    splits = SKEW_SPLITS
    ro, bo, ro_np, bo_np = offsets(mxq, splits)
    M, N, G = 768, 512, len(splits)
    A, As, B, Bs, base, ref = skew_case(accumulate)
    if accumulate:
        out = torch.from_numpy(base.copy()).cuda()
    else:
        out = torch.full((G, M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    for rep in range(2):   # the second call reuses a fresh workspace: no state carries over
        if accumulate and rep:
            out.copy_(torch.from_numpy(base))
        mxq.grouped_gemm(mxq.GEMM_TN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs), block_off=bo,
                         accumulate=accumulate, max_workgroups=max_wg)
        torch.cuda.synchronize()
        got = out_np(out)
        check_close(got, ref_np(ref, "f32" if accumulate else "bf16"))
        empty = [g for g, n in enumerate(splits) if n == 0]
        if accumulate:
            assert np.array_equal(got[empty], base[empty])   # empty groups leave C as it was
        else:
            assert np.all(got[empty] == 0)                   # empty groups write zeros


def deq(c, s):
    import refmath as R
    return R.E4M3[c] * np.exp2(s.astype(np.float64) - 127)


@pytest.mark.parametrize("mode", ["NT", "NN", "TN"])
def test_random_codes_error_bound(mxq, mode):
    """Adversarial operands (random codes over the whole E4M3 range, random
    block scales): the result stays within 1e-3 * sum|a*b| of the exact dot
    product.  The block-scaled matrix core sums each 128-element step with a
    limited-width internal adder (measured ~3e-4 of sum|a*b| at worst here),
    so the generic rel/abs tolerance is reserved for quantized data above."""
    rng = np.random.default_rng(7)
    splits = [5, 0, 17, 130, 1, 64, 0, 40]
    ro, bo, ro_np, bo_np = offsets(mxq, splits)
    R, N, K, G, M = sum(splits), 144, 256, len(splits), 160
    if mode == "NT":
        A, As = rand_codes(rng, (R, K)), rand_scales(rng, (R, K // 32))
        B, Bs = rand_codes(rng, (G, N, K)), rand_scales(rng, (G, N, K // 32))
        Av, Bv = deq(A, np.repeat(As, 32, 1)), deq(B, np.repeat(Bs, 32, 2))
        exact, absum = np.zeros((R, N)), np.zeros((R, N))
        for g in range(G):
            s = slice(ro_np[g], ro_np[g + 1])
            exact[s], absum[s] = Av[s] @ Bv[g].T, np.abs(Av[s]) @ np.abs(Bv[g]).T
        out = torch.empty((R, N), dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs))
    elif mode == "NN":
        A, As = rand_codes(rng, (R, K)), rand_scales(rng, (R, K // 32))
        B, Bs = rand_codes(rng, (G, K, N)), rand_scales(rng, (G, K // 32, N))
        Av, Bv = deq(A, np.repeat(As, 32, 1)), deq(B, np.repeat(Bs, 32, 1))
        exact, absum = np.zeros((R, N)), np.zeros((R, N))
        for g in range(G):
            s = slice(ro_np[g], ro_np[g + 1])
            exact[s], absum[s] = Av[s] @ Bv[g], np.abs(Av[s]) @ np.abs(Bv[g])
        out = torch.empty((R, N), dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs))
    else:
        nb = int(bo_np[-1])
        A, As = rand_codes(rng, (R, M)), rand_scales(rng, (nb, M))
        B, Bs = rand_codes(rng, (R, N)), rand_scales(rng, (nb, N))
        rowblk = np.zeros(R, np.int64)
        for g in range(G):
            rowblk[ro_np[g]:ro_np[g + 1]] = bo_np[g] + np.arange(splits[g]) // 32
        Av, Bv = deq(A, As[rowblk]), deq(B, Bs[rowblk])
        exact, absum = np.zeros((G, M, N)), np.zeros((G, M, N))
        for g in range(G):
            s = slice(ro_np[g], ro_np[g + 1])
            exact[g], absum[g] = Av[s].T @ Bv[s], np.abs(Av[s]).T @ np.abs(Bv[s])
        out = torch.zeros((G, M, N), dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_TN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs), block_off=bo)
    torch.cuda.synchronize()
    err = np.abs(out_np(out) - exact)
    assert np.all(err <= 1e-3 * absum + 1e-30), (err / np.maximum(absum, 1e-30)).max()


def test_integer_exact_bit_exact(mxq):
    """Codes in {-2..2}, scale bytes 126..128, K = 64: every partial sum is a
    small dyadic number, exact in fp32 and bf16, so GPU == oracle bit for bit."""
    rng = np.random.default_rng(5)
    vals = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8)
    splits = [3, 13, 0, 50]
    ro, bo, ro_np, _ = offsets(mxq, splits)
    R, N, K, G = sum(splits), 32, 64, len(splits)
    A, B = vals[rng.integers(0, 5, (R, K))], vals[rng.integers(0, 5, (G, N, K))]
    As, Bs = rand_scales(rng, (R, 2), 126, 129), rand_scales(rng, (G, N, 2), 126, 129)
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, 2, 1)
    opB = O.Operand("mxfp8", B, N * K, K, 1, Bs, N * 2, 2, 1)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "bf16")
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs))
    torch.cuda.synchronize()
    assert np.array_equal(W.bf16_bits(out), ref)


def test_single_group_equals_dense(mxq):
    rng = np.random.default_rng(6)
    R, N, K = 200, 128, 256
    A = rand_bf16(rng, (R, K))
    B = rand_bf16(rng, (1, N, K), 0.05)
    ro, _, _, _ = offsets(mxq, [R])
    out = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out)
    torch.cuda.synchronize()
    Av = (A.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    Bv = (B[0].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    check_close(out_np(out), Av @ Bv.T)


# ------------------------------------------------------------------ several tiles

BIG_SPLITS = [300, 0, 40, 1, 257]


def run_mxfp8(mxq, rng, mode, splits, N, KM, max_workgroups=0):
    """One MXFP8 grouped GEMM on quantized normal data against the oracle.
    KM is the contraction K (NT, NN) or the output row count M (TN)."""
    ro, bo, ro_np, bo_np = offsets(mxq, splits)
    R, G = sum(splits), len(splits)
    if mode == "NT":
        K = KM
        A, As = qrows(rng, (R, K))
        Bl = [qrows(rng, (N, K), 0.05) for _ in range(G)]
        B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
        opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
        opB = O.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
        ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "bf16")
        out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs),
                         max_workgroups=max_workgroups)
        rdt = "bf16"
    elif mode == "NN":
        K = KM
        A, As = qrows(rng, (R, K))
        Bl = [qcols(rng, (K, N), None, 0.05) for _ in range(G)]
        B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
        opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
        opB = O.Operand("mxfp8", B, K * N, 1, N, Bs, (K // 32) * N, 1, N)
        ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "f32")
        out = torch.empty((R, N), dtype=torch.float32, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs),
                         max_workgroups=max_workgroups)
        rdt = "f32"
    else:
        M = KM
        A, As = qcols(rng, (R, M), ro_np)
        B, Bs = qcols(rng, (R, N), ro_np, 0.01)
        opA = O.Operand("mxfp8", A, 0, 1, M, As, 0, 1, M)
        opB = O.Operand("mxfp8", B, 0, 1, N, Bs, 0, 1, N)
        ref = O.grouped_gemm("k", ro_np, M, N, 0, opA, opB, "bf16")
        out = torch.full((G, M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_TN, ro, to_dev(A), to_dev(B), out, to_dev(As), to_dev(Bs), block_off=bo,
                         max_workgroups=max_workgroups)
        rdt = "bf16"
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, rdt))


@pytest.mark.parametrize("mode,N,KM", [("NT", 272, 384), ("NN", 272, 416), ("TN", 288, 272)])
def test_multi_tile_mxfp8(mxq, mode, N, KM):
    """Several 256 x 256 output tiles in both dimensions, row and column tails,
    and contraction lengths of several 128-byte steps (the double-buffered
    pipeline), on quantized normal data."""
    run_mxfp8(mxq, np.random.default_rng(11), mode, BIG_SPLITS, N, KM)


# Many tiles per workgroup: the persistent loop, the next tile's first stage
# loaded during the current tile's last step, tiles with no contraction steps
# (empty K-groups) between tiles with steps, and the per-XCD tile ranges.
# Small groups keep the oracle's cost down while giving ~100 tiles.
PERSIST_SPLITS = [5, 0, 3, 140, 0, 0, 1, 7, 260, 2, 0, 31, 33, 0, 129, 1, 64, 0, 0, 9,
                  17, 4, 0, 2, 255, 0, 6, 8, 0, 1, 0, 44, 3, 0, 0, 12, 1, 0, 2, 70]


@pytest.mark.parametrize("max_wg", [8, 24])
@pytest.mark.parametrize("mode,N,KM", [("NT", 272, 256), ("NN", 272, 288), ("TN", 272, 272)])
def test_persistent_many_tiles_mxfp8(mxq, mode, N, KM, max_wg):
    run_mxfp8(mxq, np.random.default_rng(21), mode, PERSIST_SPLITS, N, KM, max_workgroups=max_wg)


def test_many_groups_scan_path(mxq):
    """More groups than the LDS group tables hold (1024): every tile lookup scans
    the offsets on the device; mostly empty groups, a few of several tiles."""
    rng = np.random.default_rng(22)
    G, N, K = 4500, 32, 64
    splits = [0] * G
    for g in rng.choice(G, 40, replace=False):
        splits[int(g)] = int(rng.integers(1, 300))
    splits[G - 1] = 257
    ro, bo, ro_np, _ = offsets(mxq, splits)
    R = sum(splits)
    A, As = qrows(rng, (R, K))
    B, Bs = qrows(rng, (G * N, K), 0.05)          # rowwise blocks: one call for all groups
    opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = O.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
    ref = ref_np(O.grouped_gemm("m", ro_np, 0, N, K, opA, opB, "bf16"), "bf16")
    for max_wg in (0, 8):
        out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
        mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B.reshape(G, N, K)), out, to_dev(As),
                         to_dev(Bs.reshape(G, N, K // 32)), max_workgroups=max_wg)
        torch.cuda.synchronize()
        check_close(out_np(out), ref)


@pytest.mark.parametrize("splits,max_wg", [(BIG_SPLITS, 0), (PERSIST_SPLITS, 8)])
def test_multi_tile_bf16(mxq, splits, max_wg):
    rng = np.random.default_rng(12)
    ro, bo, ro_np, _ = offsets(mxq, splits)
    R, N, K, G = sum(splits), 272, 192, len(splits)
    A = rand_bf16(rng, (R, K))
    B = rand_bf16(rng, (G, N, K), 0.05)
    ref = O.grouped_gemm("m", ro_np, 0, N, K, O.Operand("bf16", A, 0, K, 1), O.Operand("bf16", B, N * K, K, 1), "bf16")
    out = torch.empty((R, N), dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, to_dev(A), to_dev(B), out, max_workgroups=max_wg)
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, "bf16"))


# ------------------------------------------------------------------ the row-scale ring

# The K-contiguous row scales of MXFP8 NT / NN launches come through a two-slot
# LDS ring, 16 scale bytes per row per 8 stages of 64 contraction bytes, when
# every row-scale pitch is a multiple of 4 bytes and the contraction has
# ks = K/64 >= 3 stages with ks % 8 either 0 or >= 3.  The expert layer's
# launches all take it, with several ring groups per tile:
#   NT K = 768 (FC2 forward):  A and B pitches 24 B (24 % 4 == 0); ks = 12 =
#       one whole 8-stage group and a 4-stage tail group;
#   NT K = 1024:               pitches 32 B; ks = 16 = two whole groups;
#   NN K = 1536 (FC1 dgrad):   A's pitch 48 B (B's column scales stay per
#       stage); ks = 24 = three groups;
#   NN K = 2048 (FC2 dgrad):   A's pitch 64 B; ks = 32 = four groups.
# Empty groups sit between the others, and max_workgroups = 8 chains many
# tiles through each workgroup (the ring's slot parity carries across tiles).
RING_SPLITS = [70, 0, 300, 1, 0, 129, 33, 0]
_RING_CACHE = {}


def ring_case(mode, K, N=272):
    """Inputs and the oracle's result of a ring-path case (computed once)."""
    key = (mode, K)
    if key not in _RING_CACHE:
        rng = np.random.default_rng(41 + K)
        splits = RING_SPLITS
        ro_np = O.splits_to_offsets(splits)[0]
        R, G = sum(splits), len(splits)
        A, As = qrows(rng, (R, K))
        if mode == "NT":
            Bl = [qrows(rng, (N, K), 0.05) for _ in range(G)]
            opB_args = lambda B, Bs: O.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
        else:
            Bl = [qcols(rng, (K, N), None, 0.05) for _ in range(G)]
            opB_args = lambda B, Bs: O.Operand("mxfp8", B, K * N, 1, N, Bs, (K // 32) * N, 1, N)
        B, Bs = np.stack([b[0] for b in Bl]), np.stack([b[1] for b in Bl])
        assert As.shape[1] % 4 == 0 and (mode == "NN" or Bs.shape[2] % 4 == 0)
        ks = K // 64
        assert ks >= 3 and (ks % 8 == 0 or ks % 8 >= 3)
        opA = O.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
        ref = O.grouped_gemm("m", ro_np, 0, N, K, opA, opB_args(B, Bs), "bf16")
        _RING_CACHE[key] = (A, As, B, Bs, ref)
    return _RING_CACHE[key]


@pytest.mark.parametrize("max_wg", [0, 8])
@pytest.mark.parametrize("mode,K", [("NT", 768), ("NT", 1024), ("NN", 1536), ("NN", 2048)])
def test_scale_ring_mxfp8(mxq, mode, K, max_wg):
    A, As, B, Bs, ref = ring_case(mode, K)
    ro, bo, ro_np, _ = offsets(mxq, RING_SPLITS)
    R, N = A.shape[0], 272
    out = torch.full((R, N), 5.0, dtype=torch.bfloat16, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT if mode == "NT" else mxq.GEMM_NN, ro, to_dev(A), to_dev(B), out, to_dev(As),
                     to_dev(Bs), max_workgroups=max_wg)
    torch.cuda.synchronize()
    check_close(out_np(out), ref_np(ref, "bf16"))
