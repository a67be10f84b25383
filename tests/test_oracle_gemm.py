"""Pins of the oracle's grouped GEMM.

Page NVIDIA/TransformerEngine pull 3224 (Greptile Summary and Sequence
Diagram) and page "[PyTorch] GroupedTensor integration" (Changes): one grouped
GEMM over per-expert groups, with bf16 or MXFP8 operands.  Page "Activation +
GroupedLinear Fusion for MOE and other MOE optimizations", Sequence Diagram:
forward, dgrad and wgrad of the grouped linear.

The reference below dequantizes with refmath's E4M3 table (built from the
format's field layout) and multiplies with numpy in float64, so a transposed
operand, a wrong group offset or a wrong scale index fails.
"""
import numpy as np
import pytest

import refmath as R


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def rand_fp8(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38   # no NaN codes
    return c


def deq(codes, scales_expanded):
    return R.E4M3[codes] * np.exp2(scales_expanded.astype(np.float64) - 127)


def check(got, ref, out_dtype):
    g = R.bf16_bits_to_f64(got) if out_dtype == "bf16" else got.astype(np.float64)
    tol = 1e-2 if out_dtype == "bf16" else 1e-5
    assert np.allclose(g, ref, rtol=tol, atol=1e-6 * (np.abs(ref).max() + 1)), np.abs(g - ref).max()


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_m_grouped_bf16_kcontig(oracle_mod, out_dtype):
    rng = np.random.default_rng(30)
    splits = [5, 0, 17, 33]
    ro, _ = oracle_mod.splits_to_offsets(splits)
    R_, N, K, G = int(ro[-1]), 24, 64, len(splits)
    A = rand_bf16(rng, (R_, K))
    B = rand_bf16(rng, (G, N, K))
    opA = oracle_mod.Operand("bf16", A, 0, K, 1)
    opB = oracle_mod.Operand("bf16", B, N * K, K, 1)
    C = oracle_mod.grouped_gemm("m", ro, 0, N, K, opA, opB, out_dtype)
    Av, Bv = R.bf16_bits_to_f64(A), R.bf16_bits_to_f64(B)
    ref = np.zeros((R_, N))
    for g in range(G):
        ref[ro[g]:ro[g + 1]] = Av[ro[g]:ro[g + 1]] @ Bv[g].T
    check(C, ref, out_dtype)


def test_m_grouped_mxfp8_kcontig_and_kstrided(oracle_mod):
    rng = np.random.default_rng(31)
    splits = [0, 40, 7, 1]
    ro, _ = oracle_mod.splits_to_offsets(splits)
    R_, N, K, G = int(ro[-1]), 16, 96, len(splits)
    A = rand_fp8(rng, (R_, K))
    As = rng.integers(120, 134, (R_, K // 32)).astype(np.uint8)
    Av = deq(A, np.repeat(As, 32, 1))
    # B K-contiguous (G, N, K), rowwise scales (G, N, K/32)
    B = rand_fp8(rng, (G, N, K))
    Bs = rng.integers(120, 134, (G, N, K // 32)).astype(np.uint8)
    Bv = deq(B, np.repeat(Bs, 32, 2))
    opA = oracle_mod.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = oracle_mod.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
    C = oracle_mod.grouped_gemm("m", ro, 0, N, K, opA, opB, "f32")
    ref = np.zeros((R_, N))
    for g in range(G):
        ref[ro[g]:ro[g + 1]] = Av[ro[g]:ro[g + 1]] @ Bv[g].T
    check(C, ref, "f32")
    # the same B stored K-strided (G, K, N) with colwise scales (G, K/32, N)
    Bt = np.ascontiguousarray(B.transpose(0, 2, 1))
    Bts = np.ascontiguousarray(Bs.transpose(0, 2, 1))
    opBt = oracle_mod.Operand("mxfp8", Bt, K * N, 1, N, Bts, (K // 32) * N, 1, N)
    C2 = oracle_mod.grouped_gemm("m", ro, 0, N, K, opA, opBt, "f32")
    assert np.array_equal(C, C2)


def test_k_grouped_mxfp8_wgrad(oracle_mod):
    """C_g = A_g^T B_g over the rows of group g, colwise-quantized operands with
    per-group 32-row scale blocks; an empty group gives zeros."""
    rng = np.random.default_rng(32)
    splits = [33, 0, 31, 64]
    ro, bo = oracle_mod.splits_to_offsets(splits)
    R_, Md, N, G = int(ro[-1]), 24, 40, len(splits)
    A = rand_fp8(rng, (R_, Md))
    B = rand_fp8(rng, (R_, N))
    nb = int(bo[-1])
    As = rng.integers(120, 134, (nb, Md)).astype(np.uint8)
    Bs = rng.integers(120, 134, (nb, N)).astype(np.uint8)
    # expand scales to rows: row r of group g uses block bo[g] + (r - ro[g]) // 32
    rowblk = np.zeros(R_, np.int64)
    for g in range(G):
        rowblk[ro[g]:ro[g + 1]] = bo[g] + np.arange(splits[g]) // 32
    Av = deq(A, As[rowblk])
    Bv = deq(B, Bs[rowblk])
    opA = oracle_mod.Operand("mxfp8", A, 0, 1, Md, As, 0, 1, Md)
    opB = oracle_mod.Operand("mxfp8", B, 0, 1, N, Bs, 0, 1, N)
    C = oracle_mod.grouped_gemm("k", ro, Md, N, 0, opA, opB, "f32")
    for g in range(G):
        ref = Av[ro[g]:ro[g + 1]].T @ Bv[ro[g]:ro[g + 1]]
        check(C[g], ref, "f32")
    assert np.all(C[1] == 0)
    # accumulate leaves an empty group untouched and adds elsewhere
    base = np.full((G, Md, N), 0.5, np.float32)
    C3 = oracle_mod.grouped_gemm("k", ro, Md, N, 0, opA, opB, "f32", out=base.copy(), accumulate=True)
    assert np.all(C3[1] == 0.5)
    check(C3[0], Av[:33].T @ Bv[:33] + 0.5, "f32")


@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_k_grouped_bf16_wgrad(oracle_mod, out_dtype):
    """The bf16 K-grouped GEMM (the wgrad of the recipe that keeps the weight
    gradients in bf16): C_g = A_g^T B_g over the rows of group g; an empty
    group gives zeros."""
    rng = np.random.default_rng(33)
    splits = [40, 0, 7, 65]
    ro, _ = oracle_mod.splits_to_offsets(splits)
    R_, Md, N, G = int(ro[-1]), 24, 40, len(splits)
    A = rand_bf16(rng, (R_, Md))
    B = rand_bf16(rng, (R_, N), 0.1)
    Av, Bv = R.bf16_bits_to_f64(A), R.bf16_bits_to_f64(B)
    C = oracle_mod.grouped_gemm("k", ro, Md, N, 0, oracle_mod.Operand("bf16", A, 0, 1, Md),
                                oracle_mod.Operand("bf16", B, 0, 1, N), out_dtype)
    for g in range(G):
        check(C[g], Av[ro[g]:ro[g + 1]].T @ Bv[ro[g]:ro[g + 1]], out_dtype)
    assert np.all(C[1] == 0)


def test_integer_exact_case_bit_exact(oracle_mod):
    """Codes in {-2..2} with E in {126,127,128} and K <= 64: every partial sum
    is a small dyadic number, exact in fp32 and in bf16, so the result is
    bit-exact whatever the summation order."""
    rng = np.random.default_rng(33)
    vals = {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0}
    K, N, splits = 64, 8, [3, 13]
    ro, _ = oracle_mod.splits_to_offsets(splits)
    R_ = int(ro[-1])
    ai = rng.integers(-2, 3, (R_, K))
    bi = rng.integers(-2, 3, (2, N, K))
    A = np.vectorize(vals.get)(ai).astype(np.uint8)
    B = np.vectorize(vals.get)(bi).astype(np.uint8)
    As = rng.integers(126, 129, (R_, K // 32)).astype(np.uint8)
    Bs = rng.integers(126, 129, (2, N, K // 32)).astype(np.uint8)
    opA = oracle_mod.Operand("mxfp8", A, 0, K, 1, As, 0, K // 32, 1)
    opB = oracle_mod.Operand("mxfp8", B, N * K, K, 1, Bs, N * (K // 32), K // 32, 1)
    C = oracle_mod.grouped_gemm("m", ro, 0, N, K, opA, opB, "bf16")
    Av = ai * np.exp2(np.repeat(As, 32, 1) - 127.0)
    Bv = bi * np.exp2(np.repeat(Bs, 32, 2) - 127.0)
    ref = np.zeros((R_, N))
    for g in range(2):
        ref[ro[g]:ro[g + 1]] = Av[ro[g]:ro[g + 1]] @ Bv[g].T
    assert np.array_equal(R.bf16_bits_to_f64(C), ref)


def test_single_group_equals_dense(oracle_mod):
    rng = np.random.default_rng(34)
    A = rand_bf16(rng, (20, 32))
    B = rand_bf16(rng, (1, 12, 32))
    C = oracle_mod.grouped_gemm("m", [0, 20], 0, 12, 32, oracle_mod.Operand("bf16", A, 0, 32, 1),
                                oracle_mod.Operand("bf16", B, 0, 32, 1), "f32")
    ref = R.bf16_bits_to_f64(A) @ R.bf16_bits_to_f64(B[0]).T
    check(C, ref, "f32")
