"""GPU check of the expert layer captured into a HIP graph
(swiglu_mxfp8_quant_amd.moe.capture_step): every launch of a forward +
backward (grouped GEMMs with their tile counter reset kernel, fused
activation, quantizers under the weight-cache flag) replays in place.

Each replay is compared bit for bit with an eager step on the same inputs;
eager work and synchronizations run between replays, new inputs are copied
in before some of them, and the weight-cache flag is set between replays.
Page NVIDIA/TransformerEngine pull 3224 (Greptile Summary: the grouped
quantization and GEMM path kept capturable for graph replay).
"""
import pytest
import torch

import workloads as W
from parity import rowmajor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mxq():
    assert torch.cuda.is_available(), "GPU tests need the MI355X"
    import swiglu_mxfp8_quant_amd as m
    return m


KEYS = ("da", "dd", "dq_r", "dqs_r", "dq_c", "dx", "dw2", "dw13", "dscale")


def snapshot(layer, y):
    out = {"y": y.clone()}
    for k in KEYS:
        out[k] = rowmajor(layer.grads[k]).clone()
    for k in ("h13", "a_r", "as_r"):
        out[k] = rowmajor(layer.saved[k]).clone()
    return out


def same(a, b, what):
    for k in a:
        x, y = a[k], b[k]
        if x.dtype != torch.uint8:
            x, y = x.view(torch.uint8), y.view(torch.uint8)
        assert torch.equal(x, y), f"{what}: {k} differs"


@pytest.mark.parametrize("skewed,fused", [(False, False), (True, False), (True, True)])
def test_layer_graph_replay(mxq, skewed, fused):
    from swiglu_mxfp8_quant_amd.moe import Layer, capture_step
    T, H, E, k, I = 128, 256, 16, 2, 256
    moe = W.moe_layer(11, skewed=skewed, tokens=T, hidden=H, experts=E, topk=k, inter=I)
    R = int(moe["splits"].sum())
    splits, w13, w2 = moe["splits"].cuda(), moe["w13"].cuda(), moe["w2"].cuda()
    x, sc = moe["x_perm"].cuda(), moe["scale"].cuda()
    dy = W.moe_grad(R, H, seed=11).cuda()
    ref_layer = Layer(splits, w13, w2, fused_fc1=fused)
    layer = Layer(splits, w13, w2, fused_fc1=fused)
    graph, y = capture_step(layer, x, sc, dy)
    torch.cuda.synchronize()
    for step in range(5):
        if step in (2, 4):   # new inputs, copied into the captured ones
            x.copy_(W.moe_layer(20 + step, skewed=skewed, tokens=T, hidden=H, experts=E, topk=k, inter=I,
                                weights=False)["x_perm"].cuda())
            dy.copy_(W.moe_grad(R, H, seed=20 + step).cuda())
        if step == 3:        # the weights have not changed since the last step
            layer.mark_weights_current()
        junk = torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        got = snapshot(layer, y)
        ry = ref_layer.forward(x, sc)
        ref_layer.backward(dy)
        torch.cuda.synchronize()
        same(got, snapshot(ref_layer, ry), f"replay {step}")
