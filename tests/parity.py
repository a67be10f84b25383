"""Parity rules between the HIP library and the CPU oracle (tests only).

The numeric contract: offsets, E8M0 scale bytes and E4M3 codes are bit-exact
wherever the element's value was not boundary-close (its exact pre-rounding
value lies within 2 fp32 ulps of a rounding tie, as flagged by the oracle);
elsewhere a code may differ by one step, on at most 1e-4 of the codes, and a
scale byte may differ by one only in a block whose amax element is
boundary-close.  bf16 outputs are within one bf16 ulp and bit-exact where not
boundary-close.  NaN outputs compare equal to NaN whatever their payload.
"""
import numpy as np


def e4m3_ordinal(c):
    c = np.asarray(c, np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def bf16_ordinal(b):
    b = np.asarray(b, np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_isnan(b):
    b = np.asarray(b, np.uint16)
    return (b & 0x7FFF) > 0x7F80


def compare_bf16(name, got, ref, close, report):
    """got/ref uint16 bit patterns, close bool (same shape)."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    nan_g, nan_r = bf16_isnan(got), bf16_isnan(ref)
    assert np.array_equal(nan_g, nan_r), f"{name}: NaN positions differ ({(nan_g != nan_r).sum()})"
    diff = (got != ref) & ~nan_g
    # +0 and -0: the sign of zero is part of the contract, so they differ
    n = int(diff.sum())
    report[name] = n
    if n:
        bad = diff & ~close
        assert not bad.any(), f"{name}: {int(bad.sum())} non-boundary-close bf16 mismatches, e.g. at {np.argwhere(bad)[:3].tolist()}"
        d = np.abs(bf16_ordinal(got[diff]) - bf16_ordinal(ref[diff]))
        assert d.max() <= 1, f"{name}: bf16 mismatch of {d.max()} ulps"


def compare_mx(name, gc, gs, rc, rs, close, rowwise, rowblock=None, report=None, max_frac=1e-4):
    """Codes gc/rc (M, K) uint8; scales gs/rs (rowwise (M, K/32), colwise (B, K));
    close (M, K) bool; rowblock (M,) colwise scale row of every row."""
    report = {} if report is None else report
    gc, gs, rc, rs = (np.asarray(x, np.uint8) for x in (gc, gs, rc, rs))
    M, K = rc.shape
    assert gc.shape == rc.shape, f"{name}: code shape {gc.shape} vs {rc.shape}"
    assert gs.shape == rs.shape, f"{name}: scale shape {gs.shape} vs {rs.shape}"
    if M == 0 or K == 0:
        return
    if rowwise:
        blk_close = close.reshape(M, K // 32, 32).any(axis=2)        # (M, K/32)
        sdiff = gs != rs
        exp_s = lambda s: np.repeat(s, 32, axis=1)
    else:
        nb = rs.shape[0]
        blk_close = np.zeros((nb, K), bool)
        np.logical_or.at(blk_close, rowblock, close)
        sdiff = gs != rs
        exp_s = lambda s: s[rowblock]
    ns = int(sdiff.sum())
    report[name + ".scales"] = ns
    if ns:
        bad = sdiff & ~blk_close
        assert not bad.any(), f"{name}: {int(bad.sum())} scale bytes differ in blocks with no boundary-close element"
        dE = np.abs(gs[sdiff].astype(int) - rs[sdiff].astype(int))
        assert dE.max() <= 1, f"{name}: scale byte off by {dE.max()}"
    same_scale = ~exp_s(sdiff)
    cdiff = (gc != rc) & same_scale
    nc = int(cdiff.sum())
    report[name + ".codes"] = nc
    if nc:
        bad = cdiff & ~close
        assert not bad.any(), (f"{name}: {int(bad.sum())} codes differ at non-boundary-close elements, "
                               f"e.g. {np.argwhere(bad)[:3].tolist()}")
        d = np.abs(e4m3_ordinal(gc[cdiff]) - e4m3_ordinal(rc[cdiff]))
        assert d.max() <= 1, f"{name}: code off by {d.max()} steps"
        assert nc <= max_frac * M * K + 1, f"{name}: {nc} codes differ (> {max_frac} of {M * K})"


def rowblock_of(M, row_off=None):
    """Colwise scale row of every row (blocks restart at each group)."""
    if row_off is None:
        return np.arange(M) // 32
    ro = np.asarray(row_off, np.int64)
    out = np.zeros(M, np.int64)
    b = 0
    for g in range(len(ro) - 1):
        n = ro[g + 1] - ro[g]
        out[ro[g]:ro[g + 1]] = b + np.arange(n) // 32
        b += (n + 31) // 32
    return out


def close_h(close_flags):
    """Forward closeness: either rounding (silu or h) may flip h."""
    return close_flags != 0


def rowmajor(x):
    """Row-major codes of a tensor the layer may hold K-blocked (a KBlocked of
    the package): the same bytes in (rows, K) order, for comparisons."""
    return x.to_rowmajor() if hasattr(x, "to_rowmajor") else x
