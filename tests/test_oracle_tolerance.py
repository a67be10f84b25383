"""Pins of the oracle's tolerance helpers: the boundary-closeness flag of an
exact value (near_bf16_tie) and the tolerance of the fp32 dscale row sum.

Neither number is printed on the pages.  The parity contract (bit-exact
unless the exact value lies within 2 fp32 ulps of a rounding tie) names the
closeness rule; the dscale tolerance is a reading: the error bound of an fp32
summation in which no term passes through more than 63 additions, plus the
final rounding, plus the terms whose bf16 activation a correct fp32
evaluation may round the other way.  Page "Activation + GroupedLinear Fusion
for MOE and other MOE optimizations", Greptile Summary (the gradient of the
row scales); page "[mxfp8 training] Add a fused gated-activation (SwiGLU) +
MXFP8 quantization kernel", Numerics and tests (where fp32 evaluation may
differ from the exact one).

The references are exact rationals built independently of the oracle: tie
points from bf16 bit patterns, distances in binary32 ulps from numpy's
float32 nextafter, sums from Fractions.
"""
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import refmath as R
import workloads as W

ULP = Fraction(1, 1 << 24)


def _tie_cases():
    """(x, k): x = a bf16 rounding tie moved by k binary32 ulps, k in -3..3,
    for normal and subnormal bf16 neighbours of both signs."""
    rng = np.random.default_rng(31)
    normals = rng.integers(0x0080, 0x7F7F, 150).astype(np.uint16)
    subnormals = np.array([0x0001, 0x0002, 0x0033, 0x007E, 0x007F], np.uint16)
    cases = []
    for b in np.concatenate([normals, subnormals]):
        lo = np.float32(R.bf16_bits_to_f64(b))
        hi = np.float32(R.bf16_bits_to_f64(np.uint16(b + 1)))
        tie = np.float32((np.float64(lo) + np.float64(hi)) / 2)   # 9 significant bits: exact
        assert Fraction(float(tie)) == (Fraction(float(lo)) + Fraction(float(hi))) / 2
        for k in range(-3, 4):
            x = tie
            step = np.float32(np.inf) if k > 0 else np.float32(-np.inf)
            for _ in range(abs(k)):
                x = np.nextafter(x, step)
            for sgn in (1, -1):
                cases.append((sgn * float(x), k, float(tie), sgn))
    return cases


def test_near_bf16_tie_against_constructed_ulps(oracle_mod):
    """The flag is set exactly at 0, +-1 and +-2 fp32 ulps of a tie and clear at
    +-3, for normal and subnormal values; refmath's exact tie search agrees
    with the construction."""
    cases = _tie_cases()
    got = oracle_mod.near_bf16_tie(np.array([c[0] for c in cases]))
    for (x, k, tie, sgn), flag in zip(cases, got):
        assert flag == (abs(k) <= 2), (x, k, flag)
        # the exact distance to the nearest tie, from refmath's own search
        d = R.bf16_tie_distance_rel(Fraction(x)) * abs(Fraction(x))
        assert d == abs(Fraction(x) - sgn * Fraction(tie))


def test_near_bf16_tie_away_from_ties(oracle_mod):
    """bf16 values themselves, zero, and non-finite values are never close."""
    rng = np.random.default_rng(32)
    b = rng.integers(0x0001, 0x7F7F, 500).astype(np.uint16)
    v = R.bf16_bits_to_f64(b)
    assert not oracle_mod.near_bf16_tie(np.concatenate([v, -v])).any()
    assert not oracle_mod.near_bf16_tie(np.array([0.0, -0.0, np.inf, -np.inf, np.nan])).any()


def _bits(vals):
    return np.array([R.nearest_bf16_exact(Fraction(float(v))) for v in vals], dtype=np.uint16)


def _silu_close_gates(oracle_mod, n):
    """Gate values whose exact silu the oracle flags as boundary-close (scan of
    all finite bf16 g in [-20, 20])."""
    g = R.FINITE_BF16_BITS
    gv = R.bf16_bits_to_f64(g)
    g = g[np.abs(gv) <= 20]
    M = (len(g) // 32) * 32
    g = g[:M].reshape(-1, 32)
    _, close = oracle_mod.swiglu_fwd(g, np.full_like(g, 0x3F80), want_close=True)
    picked = g[(close & 1) != 0]
    assert len(picked) >= n, len(picked)
    return picked[:n]


def test_dscale_tol_equals_its_formula(oracle_mod):
    """dscale_tol = 64 * 2^-24 * sum|dh*a*u| + sum over silu-close columns of
    |dh*u| * ulp_bf16(a), evaluated here with Fractions and refmath's exact
    silu; the rows include silu-close gate values so the second term is live."""
    rng = np.random.default_rng(33)
    M, K = 6, 64
    g = _bits(rng.standard_normal(M * K) * 2).reshape(M, K)
    close_g = _silu_close_gates(oracle_mod, 12)
    g[:, :2] = close_g.reshape(M, 2)
    u = _bits(rng.standard_normal(M * K)).reshape(M, K)
    dh = _bits(rng.standard_normal(M * K) * 1e-2).reshape(M, K)
    s = rng.uniform(0.5, 1.5, M).astype(np.float32)
    _, _, _, close, tol = oracle_mod.swiglu_bwd(dh, g, u, s, want_close=True)
    G, U, D = (R.bf16_bits_to_f64(x) for x in (g, u, dh))
    for r in range(M):
        absum = Fraction(0)
        flip = Fraction(0)
        nflip = 0
        for j in range(K):
            t = R.silu_dec(Decimal(float(G[r, j])))
            a = Fraction(float(R.bf16_bits_to_f64(np.uint16(R.nearest_bf16_exact(Fraction(t))))))
            term = Fraction(float(D[r, j])) * a * Fraction(float(U[r, j]))
            absum += abs(term)
            if close[r, j] & 1:
                nflip += 1
                e = max(int(np.floor(np.log2(abs(float(a))))) if a != 0 else -126, -126)
                flip += abs(Fraction(float(D[r, j])) * Fraction(float(U[r, j]))) * Fraction(2) ** (e - 7)
        assert nflip >= 2
        ref = 64 * ULP * absum + flip
        assert abs(Fraction(float(tol[r])) - ref) <= ref * Fraction(1, 1 << 50), (r, float(tol[r]), float(ref))


def _c2_rows(K, n, seed):
    gu = W.packed_gate_up(n, K, seed=seed)
    sc = W.row_scale(n, seed=seed).numpy()
    dy = W.bf16_bits(W.grad_out(n, K, seed=seed))
    return dy, W.bf16_bits(gu[:, :K]), W.bf16_bits(gu[:, K:]), sc


def _blocked_sum(t, widths):
    """fp32 sum of the rows of t summed in nested blocks: sequential runs of
    widths[0] terms, then of widths[1] of those partial sums, ..., then the
    rest sequentially."""
    x = t.astype(np.float32)
    for w in widths:
        n = x.shape[1]
        nb = (n + w - 1) // w
        pad = np.zeros((x.shape[0], nb * w - n), np.float32)
        y = np.concatenate([x, pad], 1).reshape(x.shape[0], nb, w)
        acc = np.zeros((x.shape[0], nb), np.float32)
        for i in range(w):
            acc = (acc + y[:, :, i]).astype(np.float32)
        x = acc
    out = np.zeros(x.shape[0], np.float32)
    for i in range(x.shape[1]):
        out = (out + x[:, i]).astype(np.float32)
    return out


@pytest.mark.parametrize("K", [2048, 7168])
def test_dscale_tol_covers_shallow_fp32_sums(oracle_mod, K):
    """Every fp32 summation of the row whose terms pass through at most 63
    additions stays within the tolerance of the oracle's dscale: pairwise,
    the 8 x 8 x 8 blocking of a 512-column slab reduction followed by the slabs
    in order, and 32-term runs followed by the runs in order (K <= 2048)."""
    dy, g, u, sc = _c2_rows(K, 64, seed=34 + K)
    _, _, ds, close, tol = oracle_mod.swiglu_bwd(dy, g, u, sc, want_close=True)
    a = oracle_mod.swiglu_fwd(g, np.full_like(g, 0x3F80))
    t = R.bf16_bits_to_f64(dy) * R.bf16_bits_to_f64(a) * R.bf16_bits_to_f64(u)   # exact in fp64
    orders = {"slab": [8, 8, 8], "pairwise": [2] * 13}
    if K <= 2048:
        orders["runs32"] = [32]
    for name, w in orders.items():
        got = _blocked_sum(t, w).astype(np.float64)
        err = np.abs(got - ds.astype(np.float64))
        assert np.all(err <= tol), (name, float((err / tol).max()))


@pytest.mark.parametrize("K", [2048, 7168])
def test_dscale_tol_detects_a_dropped_term(oracle_mod, K):
    """On rows shaped like the benchmark's, the tolerance stays below 3 % of the
    mean |dh*a*u| term, so leaving out any one term larger than that (dh set to
    zero) moves dscale past the tolerance; at least 80 % of the columns hold
    such a term."""
    dy, g, u, sc = _c2_rows(K, 4, seed=35 + K)
    _, _, ds, _, tol = oracle_mod.swiglu_bwd(dy, g, u, sc, want_close=True)
    a = oracle_mod.swiglu_fwd(g, np.full_like(g, 0x3F80))
    t = np.abs(R.bf16_bits_to_f64(dy) * R.bf16_bits_to_f64(a) * R.bf16_bits_to_f64(u))
    mean = t.mean(axis=1)
    assert np.all(tol < 0.03 * mean), (tol / mean)
    rng = np.random.default_rng(36)
    big = total = 0
    for r in range(4):
        total += K
        big += int((t[r] >= 0.03 * mean[r]).sum())
        for j in rng.choice(np.flatnonzero(t[r] >= 0.03 * mean[r]), 40, replace=False):
            d2 = dy[r:r + 1].copy()
            d2[0, j] = 0
            _, _, ds2 = oracle_mod.swiglu_bwd(d2, g[r:r + 1], u[r:r + 1], sc[r:r + 1])
            assert abs(float(ds2[0]) - float(ds[r])) > tol[r], (r, j)
    assert big >= 0.80 * total, (big, total)
