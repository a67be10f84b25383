"""Pins of the oracle's block quantizer and splits->offsets scan.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel", Summary (1x32 rowwise / 32x1 colwise blocks, RCEIL E8M0
scales, both directions from one pass) and Numerics and tests (cross-mode
consistency checked bitwise; zero, subnormal-tiny, NaN/Inf regimes).
Page "Activation + GroupedLinear Fusion for MOE and other MOE optimizations",
Greptile Summary (offsets precomputed once from the split sizes).
"""
import json
import os

import numpy as np
import pytest

import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def rand_bf16(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation is fine for test data


def brute_rowwise(x):
    """Per block: E by brute-force search, codes by brute-force nearest."""
    M, K = x.shape
    v = R.bf16_bits_to_f64(x)
    codes = np.zeros((M, K), np.uint8)
    scales = np.zeros((M, K // 32), np.uint8)
    for r in range(M):
        for b in range(K // 32):
            blk = v[r, b * 32:(b + 1) * 32]
            amax = np.nan if np.isnan(blk).any() else np.abs(blk).max()
            E = R.e8m0_bruteforce(amax)
            scales[r, b] = E
            for i in range(32):
                codes[r, b * 32 + i] = 0x7F if E == 255 else R.nearest_e4m3_bruteforce(
                    blk[i] * 2.0 ** (127 - E))
    return codes, scales


def test_rowwise_bruteforce(oracle_mod):
    rng = np.random.default_rng(10)
    x = rand_bf16(rng, (6, 64))
    x[1, :32] = rand_bf16(rng, (32,), 1e-3)
    x[2, 32:] = 0                      # zero block
    x[3, 5] = 0x7FC0                   # NaN block
    x[4, 40] = 0xFF80                  # -Inf block
    x[5, :32] = rand_bf16(rng, (32,), 1e-39)  # subnormal-tiny block
    rc, cc, rs, cs = oracle_mod.mx_quantize(x, oracle_mod.ROW)
    bc, bs = brute_rowwise(x)
    assert np.array_equal(rs, bs)
    assert np.array_equal(rc, bc)
    assert cc.size == 0 and cs.size == 0
    assert rs[2, 1] == 0 and rs[3, 0] == 255 and rs[4, 1] == 255
    assert np.all(rc[3, :32] == 0x7F) and np.all(rc[4, 32:] == 0x7F)


def test_colwise_is_rowwise_of_transpose(oracle_mod):
    """One group, M % 32 == 0: colwise quantization of x equals the
    rowwise quantization of x^T, transposed back (a transposed-index mistake
    in either direction fails this)."""
    rng = np.random.default_rng(11)
    x = rand_bf16(rng, (96, 64))
    x[0:32, 3] = 0
    x[40, 7] = 0x7FC1
    _, cc, _, cs = oracle_mod.mx_quantize(x, oracle_mod.COL)
    rc, _, rs, _ = oracle_mod.mx_quantize(np.ascontiguousarray(x.T), oracle_mod.ROW)
    assert np.array_equal(cc, rc.T)
    assert np.array_equal(cs, rs.T)


def test_both_is_union(oracle_mod):
    rng = np.random.default_rng(12)
    x = rand_bf16(rng, (70, 96))
    ro = np.array([0, 5, 5, 45, 70])
    b = oracle_mod.mx_quantize(x, 3, ro)
    r = oracle_mod.mx_quantize(x, 1, ro)
    c = oracle_mod.mx_quantize(x, 2, ro)
    assert np.array_equal(b[0], r[0]) and np.array_equal(b[2], r[2])
    assert np.array_equal(b[1], c[1]) and np.array_equal(b[3], c[3])


def test_grouped_colwise_restarts_per_group(oracle_mod):
    """Colwise blocks restart at each group's first row and the tail block is
    short: the grouped result equals quantizing each group on its own."""
    rng = np.random.default_rng(13)
    splits = [31, 0, 33, 1, 64, 7]
    ro, bo = oracle_mod.splits_to_offsets(splits)
    M = int(ro[-1])
    x = rand_bf16(rng, (M, 64))
    _, cc, _, cs = oracle_mod.mx_quantize(x, oracle_mod.COL, ro)
    assert cs.shape == (int(bo[-1]), 64)
    for g in range(len(splits)):
        if splits[g] == 0:
            continue
        _, gc, _, gs = oracle_mod.mx_quantize(x[ro[g]:ro[g + 1]], oracle_mod.COL)
        assert np.array_equal(cc[ro[g]:ro[g + 1]], gc)
        assert np.array_equal(cs[bo[g]:bo[g + 1]], gs)


def test_short_tail_block_amax_over_present_rows(oracle_mod):
    x = np.zeros((33, 32), np.uint16)
    x[:32] = 0x3F80   # 1.0
    x[32] = 0x4000    # 2.0 alone in the tail block
    _, cc, _, cs = oracle_mod.mx_quantize(x, oracle_mod.COL)
    assert np.all(cs[0] == 119) and np.all(cs[1] == 120)
    assert np.all(cc[32] == 0x78)


def test_dequant_within_half_ulp(oracle_mod):
    rng = np.random.default_rng(14)
    x = rand_bf16(rng, (64, 128), 3.0)
    rc, cc, rs, cs = oracle_mod.mx_quantize(x, 3)
    v = R.bf16_bits_to_f64(x)
    for codes, sc in ((rc, np.repeat(rs, 32, axis=1)), (cc, np.repeat(cs, 32, axis=0))):
        s = np.exp2(sc.astype(np.float64) - 127)
        y = v / s
        dq = R.E4M3[codes]
        e = np.maximum(np.floor(np.log2(np.maximum(np.abs(y), 1e-300))), -6)
        assert np.all(np.abs(dq - y) <= 0.5 * np.exp2(e - 3))
        assert np.all(np.abs(y) <= 448)


def test_negative_zero_and_subnormal_tiny(oracle_mod):
    x = np.zeros((1, 32), np.uint16)
    x[0, 0] = 0x8000                   # -0
    x[0, 1] = 0x0008                   # 2^-130 = 8 * 2^-133: a bf16 subnormal
    rc, _, rs, _ = oracle_mod.mx_quantize(x, 1)
    case = GOLD["block"][0]
    assert rs[0, 0] == case["E"]
    assert rc[0, 0] == 0x80 and rc[0, 1] == case["code"]


# ---------------------------------------------------------------- offsets ---

@pytest.mark.parametrize("case", GOLD["offsets"])
def test_offsets_hand_cases(oracle_mod, case):
    ro, bo = oracle_mod.splits_to_offsets(case["splits"])
    assert list(ro) == case["row_off"] and list(bo) == case["block_off"]


def test_offsets_properties(oracle_mod):
    rng = np.random.default_rng(15)
    s = rng.integers(0, 200, 300)
    s[rng.integers(0, 300, 40)] = 0
    ro, bo = oracle_mod.splits_to_offsets(s)
    assert ro[0] == 0 and bo[0] == 0
    assert np.array_equal(np.diff(ro), s)
    assert np.array_equal(np.diff(bo), -(-s // 32))
