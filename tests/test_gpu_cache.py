"""GPU checks of the graph-safe weight quantization (mxq_quantize_noop): the
caller-owned outputs are filled in place, a non-zero device no-op flag leaves
them untouched, and a HIP graph holding the call replays correctly whatever
the flag holds at replay time; and the expert layer's weight cache.

Page NVIDIA/TransformerEngine pull 3224, Greptile Summary: grouped
quantization of the weights into a reused output with a no-op flag, so a
graph-captured weight quantization replays in place without pointer changes.
Page "[PyTorch] GroupedTensor integration", review discussion: an optional
no-op tensor for graph capture.
"""
import numpy as np
import pytest
import torch

import oracle as O
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


def u8(t):
    return t.cpu().numpy()


def weight(G, rows, cols, seed):
    return W._normal((G * rows, cols), 0.02, seed, 40, "cuda")


def outputs(G, rows, cols):
    z = dict(dtype=torch.uint8, device="cuda")
    return (torch.empty((G * rows, cols), **z), torch.empty((G * rows, cols), **z),
            torch.empty((G * rows, cols // 32), **z), torch.empty((G * rows // 32, cols), **z))


def expect(x, G, rows):
    ro = np.arange(G + 1, dtype=np.int64) * rows
    return O.mx_quantize(W.bf16_bits(x), 3, ro)


def same(outs, ref):
    for got, r in zip(outs, ref):
        assert np.array_equal(u8(got), r)


def test_noop_flag_in_place(mxq):
    """flag 0: the outputs are the quantization of the weight; flag 1: a later
    call on a changed weight leaves them bit-identical."""
    G, rows, cols = 4, 96, 256
    ro, bo = mxq.splits_to_offsets(torch.full((G,), rows, dtype=torch.int64, device="cuda"))[:2]
    x = weight(G, rows, cols, 1)
    rc, cc, rs, cs = outputs(G, rows, cols)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    mxq.quantize_into(x, rc, cc, rs, cs, flag, ro, bo)
    torch.cuda.synchronize()
    ref = expect(x, G, rows)
    same((rc, cc, rs, cs), ref)
    flag.fill_(1)
    x.mul_(3.0)
    mxq.quantize_into(x, rc, cc, rs, cs, flag, ro, bo)
    torch.cuda.synchronize()
    same((rc, cc, rs, cs), ref)
    flag.zero_()
    mxq.quantize_into(x, rc, cc, rs, cs, flag, ro, bo)
    torch.cuda.synchronize()
    same((rc, cc, rs, cs), expect(x, G, rows))
    # without a flag: the same as the plain quantizer
    x2 = weight(G, rows, cols, 2)
    mxq.quantize_into(x2, rc, cc, rs, cs, None, ro, bo)
    q = mxq.quantize(x2, rowwise=True, colwise=True, row_off=ro, block_off=bo, n_col_blocks=G * rows // 32)
    torch.cuda.synchronize()
    for a, b in zip((rc, cc, rs, cs), q):
        assert torch.equal(a, b)


def test_noop_flag_graph_replay(mxq):
    """A graph captured with the flag at 0 replays as the flag says at replay
    time: it re-quantizes a changed weight with the flag at 0 and leaves the
    cache alone with the flag at 1.  Eager work and synchronizations run
    between replays, and every replay is checked."""
    G, rows, cols = 8, 128, 512
    ro, bo = mxq.splits_to_offsets(torch.full((G,), rows, dtype=torch.int64, device="cuda"))[:2]
    x = weight(G, rows, cols, 3)
    rc, cc, rs, cs = outputs(G, rows, cols)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mxq.quantize_into(x, rc, cc, rs, cs, flag, ro, bo)   # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.quantize_into(x, rc, cc, rs, cs, flag, ro, bo)
    torch.cuda.synchronize()
    for step in range(6):
        fresh = step % 2 == 0
        flag.fill_(0 if fresh else 1)
        before = [t.clone() for t in (rc, cc, rs, cs)]
        x.copy_(weight(G, rows, cols, 10 + step))             # the optimizer changed the weight
        junk = torch.randn(1 << 20, device="cuda").sum()      # unrelated eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        if fresh:
            same((rc, cc, rs, cs), expect(x, G, rows))
        else:
            for a, b in zip((rc, cc, rs, cs), before):
                assert torch.equal(a, b), f"replay {step}: the flag was set but the cache changed"


def test_layer_weight_cache(mxq):
    """The expert layer re-quantizes its weights on every call until told the
    cache is current; then a changed weight is not picked up (by design) until
    the layer is told the weights changed."""
    from swiglu_mxfp8_quant_amd.moe import Layer
    T, H, E, k, I = 64, 128, 8, 2, 64
    moe = W.moe_layer(5, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    R = int(moe["splits"].sum())
    layer = Layer(moe["splits"].cuda(), moe["w13"].cuda(), moe["w2"].cuda())
    x, sc = moe["x_perm"].cuda(), moe["scale"].cuda()
    dy = W.moe_grad(R, H, seed=5).cuda()
    y0 = layer.forward(x, sc).clone()
    layer.backward(dy)
    torch.cuda.synchronize()
    w2b = W.bf16_bits(moe["w2"]).reshape(E * H, I)
    q = O.mx_quantize(w2b, 3, np.arange(E + 1, dtype=np.int64) * H)
    assert np.array_equal(u8(layer.w2q).reshape(E * H, I), q[0])
    assert np.array_equal(u8(layer.w2cs).reshape(E * H // 32, I), q[3])
    layer.mark_weights_current()
    layer.w2.mul_(2.0)                 # not seen while the cache is marked current
    y1 = layer.forward(x, sc)
    layer.backward(dy)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    layer.mark_weights_changed()
    y2 = layer.forward(x, sc)
    torch.cuda.synchronize()
    q2 = O.mx_quantize(W.bf16_bits(layer.w2).reshape(E * H, I), 1)
    assert np.array_equal(u8(layer.w2q).reshape(E * H, I), q2[0])
    assert not torch.equal(y0, y2)
