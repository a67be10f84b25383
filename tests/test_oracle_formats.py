"""Pins of the oracle's number formats and of the RCEIL scale rule.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel", Summary and Numerics and tests: E8M0 scales with RCEIL
rounding and E4M3 data, including zero, subnormal-tiny, NaN/Inf and
E4M3-boundary regimes.  The checks below are exhaustive or brute force against
the independent formulations in refmath.py, plus the hand cases in
tests/golden/hand_cases.json.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def _num(v):
    return float(v) if not isinstance(v, str) else float(v)


# ---------------------------------------------------------------- bf16 ---

def test_bf16_decode_exhaustive(oracle_mod):
    got = oracle_mod.bf16_to_double(R._ALL)
    ref = R._ALLV
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_bf16_roundtrip_all_patterns(oracle_mod):
    bits = R._ALL[~np.isnan(R._ALLV)]
    back = oracle_mod.double_to_bf16(R.bf16_bits_to_f64(bits))
    assert np.array_equal(back, bits)


def test_bf16_rounding_vs_exact_nearest(oracle_mod):
    rng = np.random.default_rng(1)
    # random magnitudes over the whole range, plus exact midpoints and +-1 ulp of them
    mags = np.exp2(rng.uniform(-140, 128, 3000)) * rng.choice([-1, 1], 3000)
    i = rng.integers(0, len(R.POS_BF16_VALS) - 1, 2000)
    mids = (R.POS_BF16_VALS[i] + R.POS_BF16_VALS[i + 1]) / 2
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    xs = np.concatenate([mags, near, -near[:500], [0.0, -0.0, 3.4e38, 3.39e38, 1e-45]])
    got = oracle_mod.double_to_bf16(xs)
    ref = np.array([R.nearest_bf16_exact(Fraction(float(x))) | (0x8000 if np.signbit(x) and x == 0 else 0)
                    for x in xs], dtype=np.uint16)
    assert np.array_equal(got, ref), xs[got != ref][:5]


def test_bf16_specials(oracle_mod):
    got = oracle_mod.double_to_bf16([np.inf, -np.inf, np.nan, -np.nan, 1e39])
    assert list(got[:2]) == [0x7F80, 0xFF80]
    assert (got[2] & 0x7FFF) > 0x7F80 and (got[3] & 0x8000)
    assert got[4] == 0x7F80


# ---------------------------------------------------------------- E4M3 ---

def test_e4m3_anchor_values():
    # facts of the OCP E4M3 ('fn') format, independent of any implementation
    T = R.E4M3
    assert T[0x7E] == 448.0 and T[0x08] == 2.0 ** -6 and T[0x01] == 2.0 ** -9
    assert T[0x07] == 0.875 * 2.0 ** -6 and T[0x38] == 1.0 and np.isnan(T[0x7F])
    assert np.all(np.diff(R.E4M3_POS) > 0)


def test_e4m3_decode_all_codes(oracle_mod):
    got = oracle_mod.e4m3_to_double(np.arange(256))
    same = (got == R.E4M3) | (np.isnan(got) & np.isnan(R.E4M3))
    assert same.all()


def test_e4m3_roundtrip_all_finite_codes(oracle_mod):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    assert len(codes) == 254
    back = oracle_mod.double_to_e4m3(R.E4M3[codes])
    assert np.array_equal(back, codes)


def test_e4m3_encode_bruteforce(oracle_mod):
    rng = np.random.default_rng(2)
    mids = (R.E4M3_POS[:-1] + R.E4M3_POS[1:]) / 2
    ys = np.concatenate([
        rng.uniform(-470, 470, 4000),
        np.exp2(rng.uniform(-14, 9, 4000)) * rng.choice([-1, 1], 4000),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, -0.0, 448.0, 448.0001, 464.0, 1e30, -1e30, np.inf, -np.inf],
    ])
    got = oracle_mod.double_to_e4m3(ys)
    ref = np.array([R.nearest_e4m3_bruteforce(y) for y in ys], dtype=np.uint8)
    assert np.array_equal(got, ref), ys[got != ref][:5]


def test_e4m3_half_ulp_bound(oracle_mod):
    rng = np.random.default_rng(3)
    ys = rng.uniform(-448, 448, 5000)
    codes = oracle_mod.double_to_e4m3(ys)
    dq = R.E4M3[codes]
    # quantum at |y|: 2^(max(floor(log2|y|), -6) - 3)
    e = np.maximum(np.floor(np.log2(np.abs(ys))), -6)
    assert np.all(np.abs(dq - ys) <= 0.5 * np.exp2(e - 3) + 1e-300)


def test_e4m3_nan(oracle_mod):
    got = oracle_mod.double_to_e4m3([np.nan])
    assert got[0] in (0x7F, 0xFF)


@pytest.mark.parametrize("case", GOLD["e4m3"])
def test_e4m3_hand_cases(oracle_mod, case):
    assert int(oracle_mod.double_to_e4m3([case["y"]])[0]) == case["code"]


# ---------------------------------------------------------------- E8M0 ---

@pytest.mark.parametrize("case", GOLD["e8m0"])
def test_e8m0_hand_cases(oracle_mod, case):
    assert int(oracle_mod.e8m0_from_amax([_num(case["amax"])])[0]) == case["E"]


def test_e8m0_minimal_over_all_bf16(oracle_mod):
    """For every positive finite bf16 amax: amax*2^(127-E) <= 448 and, where E
    is not clamped at 0, amax*2^(128-E) > 448 (E is the smallest such)."""
    a = R.POS_BF16_VALS[1:]  # skip +0
    E = oracle_mod.e8m0_from_amax(a).astype(np.int64)
    assert np.all(E <= 254)
    assert np.all(a * np.exp2(127.0 - E) <= 448.0)
    unclamped = E > 0
    assert np.all(a[unclamped] * np.exp2(128.0 - E[unclamped]) > 448.0)
    # the clamp only fires below 448 * 2^-127
    assert np.all(a[~unclamped] <= 448.0 * 2.0 ** -127)


def test_e8m0_bruteforce_sample(oracle_mod):
    rng = np.random.default_rng(4)
    a = np.concatenate([np.exp2(rng.uniform(-150, 127, 500)),
                        448.0 * np.exp2(np.arange(-130, 120)),
                        np.nextafter(448.0 * np.exp2(np.arange(-100, 100)), np.inf)])
    got = oracle_mod.e8m0_from_amax(a)
    ref = np.array([R.e8m0_bruteforce(v) for v in a], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_e8m0_ceil_log2_closed_form(oracle_mod):
    """E - 127 equals ceil(log2(amax / 448)) wherever that is not clamped; the
    closed form is evaluated in fp32 as the page's 'RCEIL' wording suggests,
    on amax values that are not within fp32 rounding of 448 * 2^k."""
    rng = np.random.default_rng(5)
    a = np.exp2(rng.uniform(-100, 100, 2000))
    e = np.ceil(np.log2((a / 448.0).astype(np.float32).astype(np.float64)))
    got = oracle_mod.e8m0_from_amax(a).astype(np.int64) - 127
    assert np.array_equal(got, e.astype(np.int64))


def test_e8m0_decode(oracle_mod):
    v = oracle_mod.e8m0_to_double(np.arange(255))
    assert np.array_equal(v, np.exp2(np.arange(255) - 127.0))
    assert np.isnan(oracle_mod.e8m0_to_double([255])[0])
