"""Every element of the fused forward and backward at full size, against the
oracle: (16384, 7168) and the bandwidth-stress workload (131072, 8192) with
its zero and outlier blocks, both directions, packed [gate | up], in the
launch configuration the benchmark times.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel" (Performance: the (16384, 7168) and (131072, 8192)
rows; Numerics and tests).  The oracle runs in 1024-row chunks (whole 32-row
colwise blocks) on the host's cores; each chunk's codes, scales and bf16
gradients must equal the GPU's bit for bit, and dscale must lie within the
oracle's error bound.  On a mismatch the tolerant comparison of the parity
rules reports where.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle as O
import workloads as W
from parity import compare_bf16, compare_mx, rowblock_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


def host(t):
    if t.dtype == torch.bfloat16:
        return W.bf16_bits(t)
    return t.cpu().numpy()


def check_chunk(r0, r1, K, g, u, d, s, f, b):
    """Oracle forward + backward on rows [r0, r1); returns mismatch counts."""
    rows = slice(r0, r1)
    blocks = slice(r0 // 32, (r1 + 31) // 32)
    rc, cc, rs, cs, h, close = O.swiglu_quantize_fwd(g[rows], u[rows], s[rows], 3, want_close=True)
    o = O.swiglu_quantize_bwd(d[rows], g[rows], u[rows], s[rows], 3, want_close=True)
    pairs = {"fwd.row.codes": (f[0][rows], rc), "fwd.col.codes": (f[1][rows], cc),
             "fwd.row.scales": (f[2][rows], rs), "fwd.col.scales": (f[3][blocks], cs),
             "bwd.row.codes": (b[0][rows], o[0]), "bwd.col.codes": (b[1][rows], o[1]),
             "bwd.row.scales": (b[2][rows], o[2]), "bwd.col.scales": (b[3][blocks], o[3]),
             "dgate": (b[4][rows, :K], o[4]), "dup": (b[4][rows, K:], o[5])}
    bad = {k: int((x != y).sum()) for k, (x, y) in pairs.items() if not np.array_equal(x, y)}
    if bad:
        # the tolerant comparison names the offending elements
        rep = {}
        n = r1 - r0
        compare_mx("fwd.row", f[0][rows], f[2][rows], rc, rs, close != 0, True, report=rep)
        compare_mx("fwd.col", f[1][rows], f[3][blocks], cc, cs, close != 0, False, rowblock_of(n), report=rep)
        closeb = o[7] != 0
        compare_mx("bwd.row", b[0][rows], b[2][rows], o[0], o[2], closeb, True, report=rep)
        compare_mx("bwd.col", b[1][rows], b[3][blocks], o[1], o[3], closeb, False, rowblock_of(n), report=rep)
        compare_bf16("dgate", b[4][rows, :K], o[4], closeb[:, :K], rep)
        compare_bf16("dup", b[4][rows, K:], o[5], closeb[:, K:], rep)
    err = np.abs(b[5][rows].astype(np.float64) - o[6].astype(np.float64))
    if not np.all(err <= o[8] + 1e-30):
        bad["dscale"] = int((err > o[8] + 1e-30).sum())
    return r0, bad


@pytest.mark.parametrize("shape,stress", [((16384, 7168), False), ((131072, 8192), True)])
def test_every_element_at_full_size(mxq, shape, stress):
    M, K = shape
    print("full size", shape, "stress" if stress else "", flush=True)
    if stress:
        gu, sc, dy = W.stress_inputs(M, K, seed=0, device="cuda", frac=1e-3)
    else:
        gu = W.packed_gate_up(M, K, seed=3, device="cuda")
        sc = W.row_scale(M, seed=3, device="cuda")
        dy = W.grad_out(M, K, seed=3, device="cuda")
    f = mxq.swiglu_quantize_fwd(gu[:, :K], gu[:, K:], sc, rowwise=True, colwise=True)
    b = mxq.swiglu_quantize_bwd(dy, gu[:, :K], gu[:, K:], sc, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    g, u, d, s = host(gu[:, :K]), host(gu[:, K:]), host(dy), sc.cpu().numpy()
    f = [host(x) for x in f]
    b = [host(x) for x in b]
    del gu, dy, sc
    torch.cuda.empty_cache()
    print("  GPU outputs on the host; oracle in 1024-row chunks", flush=True)
    chunk = 1024
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    bad = {}
    done = 0
    with ThreadPoolExecutor(max_workers=workers) as ex:
        futs = [ex.submit(check_chunk, r0, min(M, r0 + chunk), K, g, u, d, s, f, b) for r0 in range(0, M, chunk)]
        for fu in futs:
            r0, bd = fu.result()
            if bd:
                bad[r0] = bd
            done += 1
            if done % 16 == 0:
                print(f"  {done * chunk} of {M} rows checked", flush=True)
    assert not bad, f"chunks differing from the oracle (first row: counts): {dict(list(bad.items())[:5])}"
