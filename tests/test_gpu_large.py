"""GPU checks past the 32-bit boundaries: the fused forward and backward on
more than 2^31 elements (row offsets past 2^32 bytes), the MXFP8 NT grouped
GEMM with an operand of more than 4 GiB, and the bf16 K-grouped GEMM over a
group whose operand spans more than 2^31 bytes, each checked
against the oracle on rows or blocks lying past the boundary.

Page "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
quantization kernel" (Numerics and tests: the unfused definition);
NVIDIA/TransformerEngine pull 3224 (Greptile Summary: one grouped GEMM over
the experts' row groups).
"""
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


def bits(t):
    return W.bf16_bits(t)


def u8(t):
    return t.cpu().numpy()


def bf16_rows(M, K, seed, std=1.0):
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 65536):   # in slices, to bound the fp32 temporary
        r1 = min(M, r0 + 65536)
        x[r0:r1] = (torch.randn((r1 - r0, K), generator=g, device="cuda") * std).to(torch.bfloat16)
    return x


def test_fused_past_2_31_elements(mxq):
    """(262176, 8192): 2^31 + 262,144 elements per input; the last 32-row
    stripe starts at element 2^31 of gate (byte 2^33 of the packed buffer)."""
    M, K = 262144 + 32, 8192
    print("fused", M, K, flush=True)
    gu = bf16_rows(M, 2 * K, 61)
    sc = (torch.rand(M, generator=torch.Generator(device="cuda").manual_seed(62), device="cuda") + 0.5)
    dy = bf16_rows(M, K, 63, std=1e-2)
    f = mxq.swiglu_quantize_fwd(gu[:, :K], gu[:, K:], sc, rowwise=True, colwise=True)
    b = mxq.swiglu_quantize_bwd(dy, gu[:, :K], gu[:, K:], sc, rowwise=True, colwise=True)
    torch.cuda.synchronize()
    for stripe in (M // 64, M // 32 - 2, M // 32 - 1):
        r0, r1 = 32 * stripe, 32 * stripe + 32
        g_np, u_np, d_np = bits(gu[r0:r1, :K]), bits(gu[r0:r1, K:]), bits(dy[r0:r1])
        s_np = sc[r0:r1].cpu().numpy()
        rc, cc, rs, cs, h, close = O.swiglu_quantize_fwd(g_np, u_np, s_np, 3, want_close=True)
        rep = {}
        compare_mx("fwd.row", u8(f[0][r0:r1]), u8(f[2][r0:r1]), rc, rs, close != 0, True, report=rep)
        compare_mx("fwd.col", u8(f[1][r0:r1]), u8(f[3][stripe:stripe + 1]), cc, cs, close != 0, False,
                   rowblock_of(32), report=rep)
        o = O.swiglu_quantize_bwd(d_np, g_np, u_np, s_np, 3, want_close=True)
        closeb = o[7] != 0
        compare_mx("bwd.row", u8(b[0][r0:r1]), u8(b[2][r0:r1]), o[0], o[2], closeb, True, report=rep)
        compare_mx("bwd.col", u8(b[1][r0:r1]), u8(b[3][stripe:stripe + 1]), o[1], o[3], closeb, False,
                   rowblock_of(32), report=rep)
        dd = bits(b[4][r0:r1])
        compare_bf16("dgate", dd[:, :K], o[4], closeb[:, :K], rep)
        compare_bf16("dup", dd[:, K:], o[5], closeb[:, K:], rep)
        err = np.abs(b[5][r0:r1].cpu().numpy().astype(np.float64) - o[6].astype(np.float64))
        assert np.all(err <= o[8] + 1e-30)
        bad = {k: v for k, v in rep.items() if v}
        assert not bad, f"stripe {stripe}: {bad}"
        print("  stripe", stripe, "ok", flush=True)


def test_mxfp8_gemm_operand_past_4_gib(mxq):
    """NT MXFP8 with A of 1,114,112 x 4096 codes (4.25 GiB) in 3 groups; the
    oracle checks the last rows of every group (A offsets past 2^32 bytes)."""
    splits = [400000, 1, 714111]
    R, N, K, G = sum(splits), 256, 4096, len(splits)
    print("gemm", R, N, K, flush=True)
    ro, _, _ = mxq.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    ro_np = O.splits_to_offsets(splits)[0]
    gen = torch.Generator(device="cuda").manual_seed(71)
    A = torch.randint(0, 0x70, (R, K), dtype=torch.uint8, device="cuda", generator=gen)
    As = torch.randint(118, 130, (R, K // 32), dtype=torch.uint8, device="cuda", generator=gen)
    B = torch.randint(0, 0x70, (G, N, K), dtype=torch.uint8, device="cuda", generator=gen)
    Bs = torch.randint(118, 130, (G, N, K // 32), dtype=torch.uint8, device="cuda", generator=gen)
    out = torch.empty((R, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_NT, ro, A, B, out, As, Bs)
    e4m3 = O.e4m3_to_double(np.arange(256))     # decode tables from the oracle
    e8m0 = O.e8m0_to_double(np.arange(256))
    torch.cuda.synchronize()
    for g in range(G):
        r1 = int(ro_np[g + 1])
        rows = np.arange(max(int(ro_np[g]), r1 - 3), r1)
        idx = torch.as_tensor(rows, device="cuda")
        a, as_ = u8(A[idx]), u8(As[idx])
        bb, bs = u8(B[g]), u8(Bs[g])
        ref = O.grouped_gemm("m", np.array([0, len(rows)], np.int64), 0, N, K,
                             O.Operand("mxfp8", a, 0, K, 1, as_, 0, K // 32, 1),
                             O.Operand("mxfp8", bb, 0, K, 1, bs, 0, K // 32, 1), "f32")
        got = out[idx].cpu().numpy().astype(np.float64)
        # the block-scaled MFMA's adder: within 1e-3 of the sum of |terms| (random codes over E4M3's range)
        da = e4m3[a] * np.repeat(e8m0[as_], 32, axis=1)
        db = e4m3[bb] * np.repeat(e8m0[bs], 32, axis=1)
        bound = 1e-3 * (np.abs(da) @ np.abs(db).T) + 1e-30
        assert np.all(np.abs(got - ref.astype(np.float64)) <= bound), f"group {g}"
        print("  group", g, "ok", flush=True)


def small_ints(M, K, seed):
    """bf16 integers in [-2, 2] (exact), in slices."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, M, 262144):
        r1 = min(M, r0 + 262144)
        x[r0:r1] = torch.randint(-2, 3, (r1 - r0, K), generator=g, device="cuda").to(torch.bfloat16)
    return x


def test_bf16_wgrad_group_past_2_31_bytes(mxq):
    """bf16 K-grouped (TN) over a group of 300,000 rows of 4096 columns
    (2.3 GiB for that operand, contraction offsets past 2^31 bytes).  Inputs
    are integers in [-2, 2], so every partial sum (at most 1.2e6 < 2^24) is
    exact in fp32 and the result equals the oracle's bit for bit in any
    order: a 64 x 64 block of the weight gradient, summed over every row."""
    splits = [3, 300000, 0]
    R, M, N, G = sum(splits), 4096, 256, len(splits)
    print("bf16 wgrad", R, flush=True)
    ro, _, _ = mxq.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
    A = small_ints(R, M, 81)
    B = small_ints(R, N, 82)
    out = torch.empty((G, M, N), dtype=torch.float32, device="cuda")
    mxq.grouped_gemm(mxq.GEMM_TN, ro, A, B, out)
    torch.cuda.synchronize()
    ms, ns = slice(4032, 4096), slice(192, 256)
    a = np.ascontiguousarray(bits(A[3:3 + 300000, ms]))
    bb = np.ascontiguousarray(bits(B[3:3 + 300000, ns]))
    ref = O.grouped_gemm("k", np.array([0, 300000], np.int64), 64, 64, 0, O.Operand("bf16", a, 0, 1, 64),
                         O.Operand("bf16", bb, 0, 1, 64), "f32")[0]
    got = out[1, ms, ns].cpu().numpy()
    assert np.array_equal(got, ref)
    assert torch.all(out[2] == 0)
