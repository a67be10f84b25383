"""Pins of the oracle's row-scaled (clamped) SwiGLU forward and backward.

Page ByteDance-Seed/VeOmni pull 1340, "What does this PR do?": SiLU is rounded
to the activation dtype before it multiplies up.  Page "Activation +
GroupedLinear Fusion for MOE and other MOE optimizations", Greptile Summary:
per-row-scaled SwiGLU and ClampedSwiGLU, and the gradient of the row scales.
Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel", API: the backward returns the packed [dGate | dUp].

The references here are exact: SiLU comes from 60-digit Decimal exp, its
derivative from a Decimal central difference (no closed form is retyped), and
every rounding to bf16 is decided by an exact comparison with the tie point.
"""
import json
import os
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import refmath as R

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


def bits(vals):
    return np.array([R.nearest_bf16_exact(Fraction(float(v))) for v in vals], dtype=np.uint16)


def f64(b):
    return R.bf16_bits_to_f64(b)


def test_silu_exhaustive_all_finite_bf16(oracle_mod):
    """bf16(silu(g)) for all 65,280 finite bf16 g (the domain the torchao page
    sweeps in its review discussion), against 60-digit Decimal exp with exact
    tie handling."""
    g = R.FINITE_BF16_BITS
    assert len(g) == 65280
    M = len(g)
    ones = np.full(M, 0x3F80, np.uint16)   # u = 1
    h = oracle_mod.swiglu_fwd(g.reshape(M, 1).repeat(32, 1)[:, :32],
                              ones.reshape(M, 1).repeat(32, 1))[:, 0]
    gv = f64(g)
    bad = []
    for i in range(M):
        d = R.silu_dec(Decimal(float(gv[i])))
        ref = R.nearest_bf16_exact(Fraction(d))
        if gv[i] == 0:
            ref = int(g[i])   # silu(+-0) = +-0: the sign of zero is kept
        if ref != h[i]:
            # only a value within 1e-15 of a tie may legitimately differ (fp64 silu)
            if R.bf16_tie_distance_rel(Fraction(d)) > Fraction(1, 10 ** 15):
                bad.append((gv[i], ref, h[i]))
    assert not bad, bad[:5]


@pytest.mark.parametrize("case", GOLD["silu_bf16"])
def test_silu_hand(oracle_mod, case):
    g = bits([case["g"]] * 32).reshape(1, 32)
    u = bits([1.0] * 32).reshape(1, 32)
    h = oracle_mod.swiglu_fwd(g, u)
    assert f64(h)[0, 0] == case["bf16"]


@pytest.mark.parametrize("case", GOLD["swiglu"])
def test_swiglu_hand(oracle_mod, case):
    g = bits([case["g"]] * 32).reshape(1, 32)
    u = bits([case["u"]] * 32).reshape(1, 32)
    h = oracle_mod.swiglu_fwd(g, u, np.array([case["s"]], np.float32))
    assert f64(h)[0, 0] == case["h"]


def test_gate_up_swap_breaks_equality(oracle_mod):
    rng = np.random.default_rng(20)
    g = bits(rng.standard_normal(64 * 32)).reshape(64, 32)
    u = bits(rng.standard_normal(64 * 32)).reshape(64, 32)
    assert not np.array_equal(oracle_mod.swiglu_fwd(g, u), oracle_mod.swiglu_fwd(u, g))


def test_row_scale_single_rounding_exact(oracle_mod):
    """h = bf16(a * u * s) with ONE rounding of the exact product, where
    a = bf16(silu(g)) (pinned above).  A double rounding (via bf16(a*u) or via
    fp32) would fail near ties; the inputs include products placed on and
    next to bf16 ties."""
    rng = np.random.default_rng(21)
    M, K = 64, 64
    g = bits(rng.standard_normal(M * K) * 2).reshape(M, K)
    u = bits(rng.standard_normal(M * K)).reshape(M, K)
    s = rng.uniform(0.5, 1.5, M).astype(np.float32)
    h = oracle_mod.swiglu_fwd(g, u, s)
    a = oracle_mod.swiglu_fwd(g, np.full((M, K), 0x3F80, np.uint16))  # bf16 silu, u = 1
    for r in range(M):
        for j in range(K):
            exact = Fraction(float(f64(a[r, j]))) * Fraction(float(f64(u[r, j]))) * Fraction(float(s[r]))
            assert h[r, j] == R.nearest_bf16_exact(exact)


def test_null_scale_is_one(oracle_mod):
    rng = np.random.default_rng(22)
    g = bits(rng.standard_normal(256)).reshape(8, 32)
    u = bits(rng.standard_normal(256)).reshape(8, 32)
    assert np.array_equal(oracle_mod.swiglu_fwd(g, u), oracle_mod.swiglu_fwd(g, u, np.ones(8, np.float32)))


def test_zero_scale_gives_zero(oracle_mod):
    rng = np.random.default_rng(23)
    g = bits(rng.standard_normal(256)).reshape(8, 32)
    u = bits(rng.standard_normal(256)).reshape(8, 32)
    h = oracle_mod.swiglu_fwd(g, u, np.zeros(8, np.float32))
    assert np.all((h & 0x7FFF) == 0)


def test_strided_views_equal_packed(oracle_mod):
    rng = np.random.default_rng(24)
    gu = bits(rng.standard_normal(16 * 128)).reshape(16, 128)
    h1 = oracle_mod.swiglu_fwd(gu[:, :64], gu[:, 64:])
    h2 = oracle_mod.swiglu_fwd(np.ascontiguousarray(gu[:, :64]), np.ascontiguousarray(gu[:, 64:]))
    assert np.array_equal(h1, h2)


# ---------------------------------------------------------------- clamped ---

def test_clamped_hand(oracle_mod):
    c0, c1, c2 = GOLD["clamped"]
    g = bits([c0["g"]] * 32).reshape(1, 32)
    u = bits([c0["u"]] * 32).reshape(1, 32)
    h = oracle_mod.swiglu_fwd(g, u, kind=oracle_mod.CLAMPED_SWIGLU)
    assert f64(h)[0, 0] == c0["a"]
    dh = bits([1.0] * 32).reshape(1, 32)
    dg, du, ds = oracle_mod.swiglu_bwd(dh, g, u, kind=oracle_mod.CLAMPED_SWIGLU)
    assert np.all((dg & 0x7FFF) == 0)
    for c in (c1, c2):
        g = bits([c["g"]] * 32).reshape(1, 32)
        u = bits([c["u"]] * 32).reshape(1, 32)
        dg, du, ds = oracle_mod.swiglu_bwd(dh, g, u, kind=oracle_mod.CLAMPED_SWIGLU)
        assert bool(np.all((du & 0x7FFF) == 0)) == c["dup_zero"]


def test_clamped_equals_plain_on_clamped_inputs(oracle_mod):
    """The clamped forward is the plain forward of min(g, 7), clamp(u, -7, 7)."""
    rng = np.random.default_rng(25)
    gv = rng.standard_normal(32 * 64) * 6
    uv = rng.standard_normal(32 * 64) * 6
    g = bits(gv).reshape(32, 64)
    u = bits(uv).reshape(32, 64)
    hc = oracle_mod.swiglu_fwd(g, u, kind=oracle_mod.CLAMPED_SWIGLU)
    gc = bits(np.minimum(f64(g).ravel(), 7.0)).reshape(32, 64)
    uc = bits(np.clip(f64(u).ravel(), -7.0, 7.0)).reshape(32, 64)
    hp = oracle_mod.swiglu_fwd(gc, uc)
    assert np.array_equal(hc, hp)


def test_clamped_nan_passes(oracle_mod):
    g = np.full((1, 32), 0x3F80, np.uint16)
    g[0, 0] = 0x7FC0
    u = np.full((1, 32), 0x3F80, np.uint16)
    h = oracle_mod.swiglu_fwd(g, u, kind=oracle_mod.CLAMPED_SWIGLU)
    assert (h[0, 0] & 0x7FFF) > 0x7F80


# ---------------------------------------------------------------- backward ---

@pytest.mark.parametrize("case", GOLD["bwd"])
def test_bwd_hand(oracle_mod, case):
    g = bits([case["g"]] * 32).reshape(1, 32)
    u = bits([case["u"]] * 32).reshape(1, 32)
    dh = bits([case["dh"]] + [0.0] * 31).reshape(1, 32)
    dg, du, ds = oracle_mod.swiglu_bwd(dh, g, u, np.array([case["s"]], np.float32))
    assert f64(du)[0, 0] == case["dup"] and f64(dg)[0, 0] == case["dgate"]
    assert ds[0] == np.float32(case["dscale"])


@pytest.mark.parametrize("kind", [0, 1])
def test_bwd_against_finite_differences(oracle_mod, kind):
    """dgate against u * s * dh * (d silu / dg) with the derivative taken by a
    60-digit central difference; dup against s * dh * a (a pinned above);
    both rounded exactly.  With the clamped variant, the masks zero the
    gradient strictly outside [-7, 7] (gate: above 7)."""
    rng = np.random.default_rng(26 + kind)
    M, K = 8, 32
    gv = rng.standard_normal(M * K) * (5 if kind else 2)
    uv = rng.standard_normal(M * K) * (5 if kind else 1)
    g = bits(gv).reshape(M, K)
    u = bits(uv).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    s = rng.uniform(0.5, 1.5, M).astype(np.float32)
    dg, du, ds = oracle_mod.swiglu_bwd(dh, g, u, s, kind=kind)
    a = oracle_mod.swiglu_fwd(g, np.full((M, K), 0x3F80, np.uint16), kind=kind)
    G, U, DH = f64(g), f64(u), f64(dh)
    for r in range(M):
        for j in range(K):
            gg, uu = G[r, j], U[r, j]
            mg = mu = 1
            if kind:
                if gg > 7:
                    gg, mg = 7.0, 0
                if uu > 7 or uu < -7:
                    uu, mu = float(np.clip(uu, -7, 7)), 0
            d = R.dsilu_dec_fd(gg)
            t = Decimal(float(DH[r, j])) * Decimal(float(s[r])) * Decimal(uu) * d * mg
            ref = R.nearest_bf16_exact(Fraction(t))
            if not mg:
                ref = int(dg[r, j])    # masked: checked as a zero below
            if ref != dg[r, j]:
                assert R.bf16_tie_distance_rel(Fraction(t)) < Fraction(1, 10 ** 12)
            t2 = Fraction(float(DH[r, j])) * Fraction(float(s[r])) * Fraction(float(f64(a[r, j])))
            if mu:
                assert du[r, j] == R.nearest_bf16_exact(t2)
            else:
                # the mask multiplies the gradient: a zero carrying the product's sign
                assert du[r, j] == (0x8000 if np.signbit(DH[r, j] * f64(a[r, j])) else 0)
            if not mg:
                assert dg[r, j] & 0x7FFF == 0


def test_dscale_properties(oracle_mod):
    """dscale = d/ds of sum_j dh*h: independent of s, linear in dh, and the
    row sum of dh*a*u (a checked two-column case and a zero-grad row)."""
    rng = np.random.default_rng(28)
    M, K = 4, 64
    g = bits(rng.standard_normal(M * K)).reshape(M, K)
    u = bits(rng.standard_normal(M * K)).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    _, _, d1 = oracle_mod.swiglu_bwd(dh, g, u, np.full(M, 1.0, np.float32))
    _, _, d2 = oracle_mod.swiglu_bwd(dh, g, u, np.full(M, 0.625, np.float32))
    assert np.array_equal(d1, d2)
    dh2 = bits(f64(dh).ravel() * 2).reshape(M, K)
    _, _, d3 = oracle_mod.swiglu_bwd(dh2, g, u)
    assert np.array_equal(d3, 2 * d1)
    dz = np.zeros((M, K), np.uint16)
    _, _, d4 = oracle_mod.swiglu_bwd(dz, g, u)
    assert np.all(d4 == 0)
    # two nonzero columns: exact sum of dh*a*u, rounded to fp32 once
    dhp = np.zeros((1, 64), np.uint16)
    dhp[0, 3] = bits([0.5])[0]
    dhp[0, 40] = bits([-0.25])[0]
    a = oracle_mod.swiglu_fwd(g[:1], np.full((1, K), 0x3F80, np.uint16))
    _, _, d5 = oracle_mod.swiglu_bwd(dhp, g[:1], u[:1])
    ex = (Fraction(0.5) * Fraction(float(f64(a[0, 3]))) * Fraction(float(f64(u[0, 3])))
          - Fraction(0.25) * Fraction(float(f64(a[0, 40]))) * Fraction(float(f64(u[0, 40]))))
    assert d5[0] == np.float32(float(ex))


def test_bwd_quantized_dact_layout(oracle_mod):
    """dact is the quantization of the packed (M, 2K) [dgate | dup]."""
    rng = np.random.default_rng(29)
    M, K = 40, 64
    g = bits(rng.standard_normal(M * K)).reshape(M, K)
    u = bits(rng.standard_normal(M * K)).reshape(M, K)
    dh = bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    out = oracle_mod.swiglu_quantize_bwd(dh, g, u, None, 3)
    rc, cc, rs, cs, dg, du, ds = out
    assert rc.shape == (M, 2 * K) and rs.shape == (M, 2 * K // 32) and cs.shape == (2, 2 * K)
    q = oracle_mod.mx_quantize(np.concatenate([dg, du], 1), 3)
    for x, y in zip(q, (rc, cc, rs, cs)):
        assert np.array_equal(x, y)
