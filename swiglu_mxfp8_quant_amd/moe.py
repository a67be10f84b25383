"""The MoE expert-MLP hot path as a sequence of libmxq calls (forward and
backward of one grouped expert layer).  Every step runs in the library's HIP
kernels; this module only allocates outputs and passes pointers.

Pages: "Activation + GroupedLinear Fusion for MOE and other MOE
optimizations" (Sequence Diagram: grouped FC1, the fused row-scaled SwiGLU
with MXFP8 quantization, grouped FC2; backward: quantized dY, FC2 dgrad and
wgrad, the fused dSwiGLU with the routing-weight gradient, FC1 dgrad and
wgrad); NVIDIA/TransformerEngine pull 3224 (Greptile Summary: one grouped GEMM
over the experts' row groups with device-side offsets).

Layouts (R routed rows sorted by expert, H hidden, I expert intermediate,
G experts):
  x_perm (R, H) bf16, row scale (R,) fp32 (routing weights),
  w13 (G, 2I, H) bf16 with rows 0..I-1 = gate and I..2I-1 = up,
  w2 (G, H, I) bf16.
Forward: H13 = FC1(x_perm) (R, 2I) bf16 [gate | up]; A = MXFP8(SwiGLU(H13) * s)
rowwise and colwise (per expert); Y = FC2(A) (R, H) bf16.
Backward from dY (R, H): dA = dY . W2_g (MXFP8 NN), dW2_g = dY_g^T A_g (MXFP8
TN), [dgate | dup], dscale and MXFP8 dact from the fused backward,
dX = dact . W13_g (MXFP8 NN), dW13_g = dact_g^T X_g (MXFP8 TN).
"""
import torch

from . import (GEMM_NN, GEMM_NT, GEMM_TN, grouped_gemm, quantize, splits_to_offsets,
               swiglu_quantize_bwd, swiglu_quantize_fwd)


def weight_offsets(G, rows, device):
    """Device offsets of G equal groups of `rows` rows (a stacked weight)."""
    return splits_to_offsets(torch.full((G,), rows, dtype=torch.int64, device=device))[:2]


def quantize_weight_both(w, offs):
    """(G, K, N) bf16 -> rowwise codes (G, K, N) and scales (G, K, N/32) (1x32
    blocks along N, for a contraction over N), and colwise codes (G, K, N) and
    scales (G, K/32, N) (32x1 blocks along each expert's K rows, for a
    contraction over K), from one read of the weight."""
    G, K, N = w.shape
    ro, bo = offs
    rc, cc, rs, cs = quantize(w.reshape(G * K, N), rowwise=True, colwise=True, row_off=ro, block_off=bo,
                              n_col_blocks=G * K // 32)
    return rc.view(G, K, N), rs.view(G, K, N // 32), cc.view(G, K, N), cs.view(G, K // 32, N)


def quantize_weight_colwise(w, offs):
    """(G, K, N) bf16 -> codes (G, K, N), scales (G, K/32, N): 32x1 blocks
    along each expert's K rows (K a multiple of 32)."""
    G, K, N = w.shape
    ro, bo = offs
    _, cc, _, cs = quantize(w.reshape(G * K, N), rowwise=False, colwise=True, row_off=ro, block_off=bo,
                            n_col_blocks=G * K // 32)
    return cc.view(G, K, N), cs.view(G, K // 32, N)


class Layer:
    """One grouped expert layer; `forward` keeps what `backward` needs."""

    def __init__(self, splits, w13, w2, clamped=False, limit=7.0):
        self.splits = splits
        self.w13, self.w2 = w13, w2
        self.G, self.I2, self.H = w13.shape
        self.I = self.I2 // 2
        self.clamped, self.limit = clamped, limit
        self.row_off, self.block_off, self.err = splits_to_offsets(splits)

    def forward(self, x_perm, scale):
        R, I, H = x_perm.shape[0], self.I, self.H
        dev = x_perm.device
        ro, bo = self.row_off, self.block_off
        h13 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NT, ro, x_perm, self.w13, h13)
        a_r, a_c, as_r, as_c = swiglu_quantize_fwd(h13[:, :I], h13[:, I:], scale, rowwise=True, colwise=True,
                                                   row_off=ro, block_off=bo, clamped=self.clamped,
                                                   limit=self.limit)
        # W2 in both directions from one read: rowwise along I for FC2, and
        # colwise along H (per expert) for FC2's dgrad in the backward
        w2q, w2s, w2c, w2cs = quantize_weight_both(self.w2, weight_offsets(self.G, H, dev))
        y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NT, ro, a_r, w2q, y, as_r, w2s)
        self.saved = dict(x_perm=x_perm, scale=scale, h13=h13, a_r=a_r, a_c=a_c, as_r=as_r, as_c=as_c,
                          w2q=w2q, w2s=w2s, w2c=w2c, w2cs=w2cs)
        return y

    def backward(self, dy):
        s = self.saved
        R, I, H, G = dy.shape[0], self.I, self.H, self.G
        dev = dy.device
        ro, bo = self.row_off, self.block_off
        dy_r, dy_c, dys_r, dys_c = quantize(dy, rowwise=True, colwise=True, row_off=ro, block_off=bo)
        w2c, w2cs = s["w2c"], s["w2cs"]
        da = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NN, ro, dy_r, w2c, da, dys_r, w2cs)
        dw2 = torch.empty((G, H, I), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_TN, ro, dy_c, s["a_c"], dw2, dys_c, s["as_c"], block_off=bo)
        h13 = s["h13"]
        dq_r, dq_c, dqs_r, dqs_c, dd, dscale = swiglu_quantize_bwd(
            da, h13[:, :I], h13[:, I:], s["scale"], rowwise=True, colwise=True, row_off=ro, block_off=bo,
            clamped=self.clamped, limit=self.limit)
        w13c, w13cs = quantize_weight_colwise(self.w13, weight_offsets(G, 2 * I, dev))
        dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NN, ro, dq_r, w13c, dx, dqs_r, w13cs)
        _, x_c, _, xs_c = quantize(s["x_perm"], rowwise=False, colwise=True, row_off=ro, block_off=bo)
        dw13 = torch.empty((G, 2 * I, H), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_TN, ro, dq_c, x_c, dw13, dqs_c, xs_c, block_off=bo)
        self.grads = dict(dy_r=dy_r, dy_c=dy_c, dys_r=dys_r, dys_c=dys_c, w2c=w2c, w2cs=w2cs, da=da, dw2=dw2,
                          dq_r=dq_r, dq_c=dq_c, dqs_r=dqs_r, dqs_c=dqs_c, dd=dd, dscale=dscale, w13c=w13c,
                          w13cs=w13cs, dx=dx, x_c=x_c, xs_c=xs_c, dw13=dw13)
        return dx, dw13, dw2, dscale


def gemm_flops(R, H, I, G=None):
    """FLOPs of the six grouped GEMMs of one forward + backward (2 per MAC)."""
    fc1 = 2 * R * (2 * I) * H
    fc2 = 2 * R * H * I
    return {"fc1_fwd": fc1, "fc2_fwd": fc2, "fc2_dgrad": fc2, "fc2_wgrad": fc2, "fc1_dgrad": fc1,
            "fc1_wgrad": fc1}
