"""GPU check of the allocation-free backward (mxq_swiglu_quantize_bwd_noalloc,
for callers that cannot allocate): through the C ABI, its outputs equal
those of mxq_swiglu_quantize_bwd with a caller workspace, bit for bit, on two
calls in a row with the second on a smaller input (the library's scratch
keeps the first call's partial sums, which the second must not see); and a
call too large for the scratch is refused before it touches the device."""
import numpy as np
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


def run(m, M, K, dirs, noalloc, splits=None, seed=0):
    gu = W.packed_gate_up(M, K, seed=seed, device="cuda")
    sc = W.row_scale(M, seed=seed, device="cuda")
    dy = W.grad_out(M, K, seed=seed, device="cuda")
    groups, ncb = None, (M + 31) // 32
    if splits is not None:
        ro, bo, _ = m.splits_to_offsets(torch.tensor(splits, dtype=torch.int64, device="cuda"))
        groups = m.make_groups(ro, bo)
        ncb = sum((s + 31) // 32 for s in splits)
    rc, cc, rs, cs = m._alloc_mx(M, 2 * K, dirs, ncb, "cuda")
    ro_, co_ = m._outs(rc, cc, rs, cs, dirs)
    dd = torch.empty((M, 2 * K), dtype=torch.bfloat16, device="cuda")
    ds = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    act = m.make_act()
    if noalloc:
        st = m.mxq_swiglu_quantize_bwd_noalloc(act, dy, gu[:, :K], gu[:, K:], sc, groups, dd[:, :K], dd[:, K:], ds,
                                               dirs, ro_, co_)
    else:
        nws = m.mxq_swiglu_quantize_bwd_workspace(M, K, dirs)
        ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
        st = m.mxq_swiglu_quantize_bwd(act, dy, gu[:, :K], gu[:, K:], sc, groups, dd[:, :K], dd[:, K:], ds, dirs,
                                       ro_, co_, ws)
    m.check(st)
    torch.cuda.synchronize()
    return [t.cpu() for t in (rc, cc, rs, cs, dd.view(torch.int16), ds)]


@pytest.mark.parametrize("first,second", [((4096, 7168, None), (1000, 2048, None)),
                                          ((2048, 4096, [700, 0, 1348]), (96, 1024, [33, 63]))])
def test_noalloc_matches_workspace_entry(mxq, first, second):
    for i, (M, K, splits) in enumerate((first, second)):
        print("noalloc case", i, M, K, splits, flush=True)
        a = run(mxq, M, K, 3, noalloc=True, splits=splits, seed=i)
        b = run(mxq, M, K, 3, noalloc=False, splits=splits, seed=i)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
        assert not torch.isnan(a[5]).any()


def test_noalloc_without_dscale_and_too_large(mxq):
    """dscale NULL needs no scratch; a dscale call beyond the scratch is refused
    with MXQ_ERR_WORKSPACE and nothing runs."""
    M, K = 512, 2048
    gu = W.packed_gate_up(M, K, seed=3, device="cuda")
    dy = W.grad_out(M, K, seed=3, device="cuda")
    rc, cc, rs, cs = mxq._alloc_mx(M, 2 * K, 1, (M + 31) // 32, "cuda")
    ro_, _ = mxq._outs(rc, cc, rs, cs, 1)
    mxq.check(mxq.mxq_swiglu_quantize_bwd_noalloc(mxq.make_act(), dy, gu[:, :K], gu[:, K:], None, None, None,
                                                  None, None, 1, ro_, None))
    ref = mxq.swiglu_quantize_bwd(dy, gu[:, :K], gu[:, K:], None, rowwise=True, dense=False, want_dscale=False)
    torch.cuda.synchronize()
    assert torch.equal(rc, ref[0]) and torch.equal(rs, ref[2])
    # 2^20 rows at K = 8192: 2^20 * 16 partials * 4 B = 64 MiB > 16 MiB; the
    # pointers are never dereferenced because validation refuses first
    big = ctypes_call_too_large(mxq)
    assert big == 8 and "scratch" in mxq.last_error()


def ctypes_call_too_large(m):
    import ctypes
    fake = ctypes.c_void_p(0x7F0000000000)
    return m.lib.mxq_swiglu_quantize_bwd_noalloc(None, 1 << 20, 8192, fake, 16384, fake, 16384, fake, 16384, None,
                                                 None, None, 0, None, 0, fake, 1, None, None, None)
