"""Pins of the oracle's row-scaled SReLU (forward and backward) and of the GLU
interleaved layout of a gated input.

Page "Activation + GroupedLinear Fusion for MOE and other MOE
optimizations", Greptile Summary: the per-row-scaled activations are SReLU,
SwiGLU and ClampedSwiGLU (SReLU is the unary one), and (Important Files
Changed) the GLU interleave reshaping moves into the scaled SwiGLU kernels.
The pages print no formula for SReLU; the reading pinned here is the squared
ReLU, rounded to bf16 before the row scale multiplies it, as the SwiGLU
activation is.  The references are exact rationals: squares, products and
sums in Fractions, rounding by refmath's exact nearest search, and the
derivative by a central difference (exact for a quadratic away from the kink).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def bits(vals):
    return np.array([R.nearest_bf16_exact(Fraction(float(v))) for v in vals], dtype=np.uint16)


def f64(b):
    return R.bf16_bits_to_f64(b)


def test_square_exhaustive_all_bf16(oracle_mod):
    """a = bf16(max(x, 0)^2) for all 65,536 bf16 patterns: the exact square
    rounded by exhaustive search for x > 0, +0 for x <= 0 (and -Inf), NaN for
    NaN, Inf where the square passes the largest bf16."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = allb.reshape(-1, 32)
    h = oracle_mod.srelu_fwd(x).reshape(-1)
    v = f64(allb)
    for i in range(len(allb)):
        if np.isnan(v[i]):
            assert (h[i] & 0x7FFF) > 0x7F80, hex(allb[i])
        elif v[i] > 0:
            if np.isinf(v[i]):
                assert h[i] == 0x7F80
            else:
                assert h[i] == R.nearest_bf16_exact(Fraction(float(v[i])) ** 2), hex(allb[i])
        else:
            assert h[i] == 0x0000, hex(allb[i])


@pytest.mark.parametrize("case", GOLD["srelu"])
def test_srelu_hand(oracle_mod, case):
    x = bits([case["x"]] * 32).reshape(1, 32)
    s = np.array([case["s"]], np.float32)
    h = oracle_mod.srelu_fwd(x, s)
    assert f64(h)[0, 0] == case["h"]
    dh = bits([case["dh"]] + [0.0] * 31).reshape(1, 32)
    dx, ds = oracle_mod.srelu_bwd(dh, x, s)
    assert f64(dx)[0, 0] == case["dx"]


def test_row_scale_single_rounding(oracle_mod):
    """h = one RNE rounding of the exact a * s (a the rounded square)."""
    rng = np.random.default_rng(51)
    M, K = 16, 64
    x = bits(rng.standard_normal(M * K) * 3).reshape(M, K)
    s = rng.uniform(0.3, 1.7, M).astype(np.float32)
    h = oracle_mod.srelu_fwd(x, s)
    a = oracle_mod.srelu_fwd(x)
    for r in range(M):
        for j in range(K):
            t = Fraction(float(f64(a[r, j]))) * Fraction(float(s[r]))
            assert h[r, j] == R.nearest_bf16_exact(t)


def test_backward_against_central_difference(oracle_mod):
    """dx = bf16(dh * s * d/dx[max(x,0)^2]) with the derivative taken as an exact
    central difference of the square (exact for a quadratic), zero below the
    kink; dscale = fp32 of the exact sum of dh * a; its tolerance is
    64 * 2^-24 * sum |dh * a|."""
    rng = np.random.default_rng(52)
    M, K = 8, 64
    x = bits(rng.standard_normal(M * K) * 2).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    s = rng.uniform(0.5, 1.5, M).astype(np.float32)
    dx, ds, close, tol = oracle_mod.srelu_bwd(dh, x, s, want_close=True)
    a = oracle_mod.srelu_fwd(x)
    X, D = f64(x), f64(dh)
    for r in range(M):
        acc = Fraction(0)
        absum = Fraction(0)
        for j in range(K):
            xv = Fraction(float(X[r, j]))
            if xv > 0:
                h = min(xv / 2, Fraction(1, 1 << 20))
                deriv = ((xv + h) ** 2 - (xv - h) ** 2) / (2 * h)
            else:
                deriv = Fraction(0)
            t = Fraction(float(D[r, j])) * Fraction(float(s[r])) * deriv
            if t == 0:
                assert dx[r, j] & 0x7FFF == 0
            else:
                assert dx[r, j] == R.nearest_bf16_exact(t)
            term = Fraction(float(D[r, j])) * Fraction(float(f64(a[r, j])))
            acc += term
            absum += abs(term)
        assert ds[r] == np.float32(float(acc))
        assert abs(Fraction(float(tol[r])) - 64 * absum / (1 << 24)) <= absum * Fraction(1, 1 << 60)


def test_quantized_layouts(oracle_mod):
    """The MXFP8 outputs are the standalone quantizer applied to h (forward) and
    to dx (backward), both (M, K)."""
    rng = np.random.default_rng(53)
    M, K = 40, 64
    x = bits(rng.standard_normal(M * K)).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    f = oracle_mod.srelu_quantize_fwd(x, None, 3)
    q = oracle_mod.mx_quantize(f[4], 3)
    for u, v in zip(q, f[:4]):
        assert np.array_equal(u, v)
    b = oracle_mod.srelu_quantize_bwd(dh, x, None, 3)
    assert b[0].shape == (M, K) and b[3].shape == (2, K)
    q = oracle_mod.mx_quantize(b[4], 3)
    for u, v in zip(q, b[:4]):
        assert np.array_equal(u, v)


# ---------------------------------------------------------------- GLU interleave

@pytest.mark.parametrize("B", [32, 64, 128])
def test_glu_split_join_roundtrip(oracle_mod, B):
    rng = np.random.default_rng(54)
    M, K = 5, 256
    p = rng.integers(0, 1 << 16, (M, 2 * K)).astype(np.uint16)
    g, u = oracle_mod.glu_split(p, B)
    assert np.array_equal(oracle_mod.glu_join(g, u, B), p)
    # column j of gate is packed column 2B*(j//B) + j%B; up is B further on
    j = np.arange(K)
    col = 2 * B * (j // B) + j % B
    assert np.array_equal(g, p[:, col]) and np.array_equal(u, p[:, col + B])


def test_glu_block_k_is_the_plain_packing(oracle_mod):
    rng = np.random.default_rng(55)
    p = rng.integers(0, 1 << 16, (3, 128)).astype(np.uint16)
    g, u = oracle_mod.glu_split(p, 64)
    assert np.array_equal(g, p[:, :64]) and np.array_equal(u, p[:, 64:])


@pytest.mark.parametrize("B", [32, 64])
def test_interleaved_backward_is_a_column_permutation(oracle_mod, B):
    """With blocks of 32 or more columns no 1x32 block mixes gate and up, so the
    interleaved backward's outputs are the plain layout's outputs with the
    same column permutation (rowwise scales permuted by 32-column block)."""
    rng = np.random.default_rng(56)
    M, K = 70, 128
    ro = np.array([0, 33, 33, 70])
    g = bits(rng.standard_normal(M * K)).reshape(M, K)
    u = bits(rng.standard_normal(M * K)).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    s = rng.uniform(0.5, 1.5, M).astype(np.float32)
    plain = oracle_mod.swiglu_quantize_bwd(dh, g, u, s, 3, ro)
    il = oracle_mod.swiglu_quantize_bwd_interleaved(dh, oracle_mod.glu_join(g, u, B), B, s, 3, ro)
    j = np.arange(2 * K)
    # packed column c of the interleaved layout holds plain column perm[c]
    blk, off = j // (2 * B), j % (2 * B)
    perm = np.where(off < B, blk * B + off, K + blk * B + off - B)
    assert np.array_equal(il[0], plain[0][:, perm])                 # row codes
    assert np.array_equal(il[1], plain[1][:, perm])                 # col codes
    assert np.array_equal(il[2], plain[2][:, perm[::32] // 32])     # row scales
    assert np.array_equal(il[3], plain[3][:, perm])                 # col scales
    assert np.array_equal(il[4], np.concatenate([plain[4], plain[5]], 1)[:, perm])
    assert np.array_equal(il[5], plain[6])
