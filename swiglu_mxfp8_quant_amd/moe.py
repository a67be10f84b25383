"""The MoE expert-MLP hot path as a sequence of libmxq calls (forward and
backward of one grouped expert layer).  Every step runs in the library's HIP
kernels; this module only allocates outputs and passes pointers.

Pages: "Activation + GroupedLinear Fusion for MOE and other MOE
optimizations" (Sequence Diagram: grouped FC1, the fused row-scaled SwiGLU
with MXFP8 quantization, grouped FC2; backward: quantized dY, FC2 dgrad and
wgrad, the fused dSwiGLU with the routing-weight gradient, FC1 dgrad and
wgrad); NVIDIA/TransformerEngine pull 3224 (Greptile Summary: one grouped GEMM
over the experts' row groups with device-side offsets; the MXFP8 weights
cached in place and re-quantized under a device no-op flag, so a captured
step replays with unchanged pointers).

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
The BF16-wgrad recipe (page "[mxfp8 training] Add a fused gated-activation
(SwiGLU) + MXFP8 quantization kernel", Performance: rowwise-only casts, the
activation recomputed in bf16 for the two wgrad GEMMs) casts A, dY and dact
rowwise only, recomputes A in bf16 from H13 in the backward, and runs both
wgrads as bf16 TN GEMMs: dW2_g = dY_g^T A_bf16_g, dW13_g = [dgate | dup]_g^T
X_g.
The MXFP8 weights (W2 rowwise along I and colwise along H, W13 colwise along
2I) live in buffers the layer owns and are re-quantized in place on every
call unless the layer's device flag says the cache holds the current weights.
"""
import torch

from . import (GEMM_NN, GEMM_NT, GEMM_TN, grouped_gemm, grouped_gemm_swiglu, interleave_rows, quantize,
               quantize_into, splits_to_offsets, swiglu_bf16, swiglu_quantize_bwd, swiglu_quantize_fwd)


def weight_offsets(G, rows, device):
    """Device offsets of G equal groups of `rows` rows (a stacked weight)."""
    return splits_to_offsets(torch.full((G,), rows, dtype=torch.int64, device=device))[:2]


class Layer:
    """One grouped expert layer; `forward` keeps what `backward` needs."""

    def __init__(self, splits, w13, w2, clamped=False, limit=7.0, fused_fc1=False, recipe="mxfp8", kblock=True):
        if recipe not in ("mxfp8", "bf16_wgrad"):
            raise ValueError(f"unknown recipe {recipe!r}")
        self.recipe = recipe
        # kblock: the rowwise codes that feed a GEMM along the contraction
        # (the activation for FC2, dY and dact for the dgrads) are written
        # K-blocked by 64 (KBlocked), so that the GEMM's stage loads cover
        # whole cache lines; the results are the same bits either way
        self.kblock = kblock
        I_, H_ = w13.shape[1] // 2, w13.shape[2]
        self.kb_a, self.kb_dy, self.kb_dq = (kblock and I_ % 64 == 0, kblock and H_ % 64 == 0,
                                             kblock and (2 * I_) % 64 == 0)
        self.splits = splits
        self.G, self.I2, self.H = w13.shape
        self.I = self.I2 // 2
        # fused_fc1: FC1 computes the activation and its MXFP8 form in its
        # epilogue; the layer then keeps W13 with gate and up rows interleaved
        # in blocks of 128 (a one-time layout change), H13 and [dgate | dup]
        # take that interleaved column order, and so do dW13's rows
        self.fused_fc1 = fused_fc1
        self.il = 128 if fused_fc1 else 0
        self.w13 = interleave_rows(w13, 128) if fused_fc1 else w13
        self.w2 = w2
        self.clamped, self.limit = clamped, limit
        self.row_off, self.block_off, self.err = splits_to_offsets(splits)
        G, H, I, dev = self.G, self.H, self.I, w13.device
        u8 = dict(dtype=torch.uint8, device=dev)
        # the MXFP8 weight cache: W2 rowwise (1x32 along I, for FC2) and
        # colwise (32x1 along each expert's H rows, for FC2's dgrad); W13
        # colwise (32x1 along each expert's 2I rows, for FC1's dgrad)
        self.w2q, self.w2s = torch.empty((G, H, I), **u8), torch.empty((G, H, I // 32), **u8)
        self.w2c, self.w2cs = torch.empty((G, H, I), **u8), torch.empty((G, H // 32, I), **u8)
        self.w13c, self.w13cs = torch.empty((G, 2 * I, H), **u8), torch.empty((G, 2 * I // 32, H), **u8)
        self.w2_offs = weight_offsets(G, H, dev)
        self.w13_offs = weight_offsets(G, 2 * I, dev)
        # device flag: non-zero = the cache holds the current weights (the
        # quantizations then do nothing); read by the kernels, never the host
        self.weights_current = torch.zeros(1, dtype=torch.int32, device=dev)

    def mark_weights_changed(self):
        """The next forward / backward re-quantize the weights into the cache."""
        self.weights_current.zero_()

    def mark_weights_current(self):
        """The cache holds the current weights (after a forward and a backward
        since they last changed): the quantizations are skipped on the device."""
        self.weights_current.fill_(1)

    def _quantize_w2(self):
        G, H, I = self.G, self.H, self.I
        quantize_into(self.w2.reshape(G * H, I), self.w2q.view(G * H, I), self.w2c.view(G * H, I),
                      self.w2s.view(G * H, I // 32), self.w2cs.view(G * H // 32, I),
                      noop_flag=self.weights_current, row_off=self.w2_offs[0], block_off=self.w2_offs[1])

    def _quantize_w13(self):
        G, H, I = self.G, self.H, self.I
        quantize_into(self.w13.reshape(G * 2 * I, H), None, self.w13c.view(G * 2 * I, H), None,
                      self.w13cs.view(G * 2 * I // 32, H), noop_flag=self.weights_current,
                      row_off=self.w13_offs[0], block_off=self.w13_offs[1])

    def forward(self, x_perm, scale):
        R, I, H = x_perm.shape[0], self.I, self.H
        dev = x_perm.device
        ro, bo = self.row_off, self.block_off
        h13 = torch.empty((R, 2 * I), dtype=torch.bfloat16, device=dev)
        col = self.recipe == "mxfp8"   # the colwise cast feeds the MXFP8 FC2 wgrad only
        if self.fused_fc1:
            a_r, a_c, as_r, as_c = grouped_gemm_swiglu(ro, x_perm, self.w13, h13, scale, rowwise=True, colwise=col,
                                                       block_off=bo, clamped=self.clamped, limit=self.limit)
        else:
            grouped_gemm(GEMM_NT, ro, x_perm, self.w13, h13)
            a_r, a_c, as_r, as_c = swiglu_quantize_fwd(h13[:, :I], h13[:, I:], scale, rowwise=True, colwise=col,
                                                       row_off=ro, block_off=bo, clamped=self.clamped,
                                                       limit=self.limit, kblock=self.kb_a)
        # W2 in both directions from one read (the colwise copy is kept for
        # the backward's FC2 dgrad)
        self._quantize_w2()
        y = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NT, ro, a_r, self.w2q, y, as_r, self.w2s)
        self.saved = dict(x_perm=x_perm, scale=scale, h13=h13, a_r=a_r, a_c=a_c, as_r=as_r, as_c=as_c,
                          w2q=self.w2q, w2s=self.w2s, w2c=self.w2c, w2cs=self.w2cs)
        return y

    def backward(self, dy):
        s = self.saved
        R, I, H, G = dy.shape[0], self.I, self.H, self.G
        dev = dy.device
        ro, bo = self.row_off, self.block_off
        mx = self.recipe == "mxfp8"
        dy_r, dy_c, dys_r, dys_c = quantize(dy, rowwise=True, colwise=mx, row_off=ro, block_off=bo,
                                            kblock=self.kb_dy)
        w2c, w2cs = s["w2c"], s["w2cs"]
        da = torch.empty((R, I), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NN, ro, dy_r, w2c, da, dys_r, w2cs)
        dw2 = torch.empty((G, H, I), dtype=torch.bfloat16, device=dev)
        h13 = s["h13"]
        uo = self.il if self.il else I   # up's first column in H13
        gate, up = h13[:, :I], h13[:, uo:uo + I]
        a_bf16 = None
        if mx:
            grouped_gemm(GEMM_TN, ro, dy_c, s["a_c"], dw2, dys_c, s["as_c"], block_off=bo)
        else:
            # the activation recomputed in bf16 for the FC2 wgrad
            a_bf16 = swiglu_bf16(gate, up, s["scale"], clamped=self.clamped, limit=self.limit,
                                 interleave=self.il)[0]
            grouped_gemm(GEMM_TN, ro, dy, a_bf16, dw2)
        dq_r, dq_c, dqs_r, dqs_c, dd, dscale = swiglu_quantize_bwd(
            da, gate, up, s["scale"], rowwise=True, colwise=mx, row_off=ro, block_off=bo,
            clamped=self.clamped, limit=self.limit, interleave=self.il, kblock=self.kb_dq)
        self._quantize_w13()
        w13c, w13cs = self.w13c, self.w13cs
        dx = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
        grouped_gemm(GEMM_NN, ro, dq_r, w13c, dx, dqs_r, w13cs)
        dw13 = torch.empty((G, 2 * I, H), dtype=torch.bfloat16, device=dev)
        x_c = xs_c = None
        if mx:
            _, x_c, _, xs_c = quantize(s["x_perm"], rowwise=False, colwise=True, row_off=ro, block_off=bo)
            grouped_gemm(GEMM_TN, ro, dq_c, x_c, dw13, dqs_c, xs_c, block_off=bo)
        else:
            grouped_gemm(GEMM_TN, ro, dd, s["x_perm"], dw13)
        self.grads = dict(dy_r=dy_r, dy_c=dy_c, dys_r=dys_r, dys_c=dys_c, w2c=w2c, w2cs=w2cs, da=da, dw2=dw2,
                          dq_r=dq_r, dq_c=dq_c, dqs_r=dqs_r, dqs_c=dqs_c, dd=dd, dscale=dscale, w13c=w13c,
                          w13cs=w13cs, dx=dx, x_c=x_c, xs_c=xs_c, dw13=dw13, a_bf16=a_bf16)
        return dx, dw13, dw2, dscale


def capture_step(layer, x_perm, scale, dy):
    """One forward + backward of `layer` captured into a HIP graph through
    torch's graph API: the library's launches go to the capturing stream, and
    the outputs and workspaces the calls allocate come from the graph's memory
    pool, so every replay recomputes them in place (reachable afterwards as
    layer.saved, layer.grads and the returned y).  x_perm, scale and dy are
    read where they lie: new data is copied into them before a replay.  The
    weight quantizations stay under the layer's device flag, so replays after
    mark_weights_current() skip them.  One untimed step runs on a side stream
    first, as graph capture asks.  Returns (graph, y)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x_perm, scale)
        layer.backward(dy)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y = layer.forward(x_perm, scale)
        layer.backward(dy)
    return graph, y


def gemm_flops(R, H, I, G=None):
    """FLOPs of the six grouped GEMMs of one forward + backward (2 per MAC)."""
    fc1 = 2 * R * (2 * I) * H
    fc2 = 2 * R * H * I
    return {"fc1_fwd": fc1, "fc2_fwd": fc2, "fc2_dgrad": fc2, "fc2_wgrad": fc2, "fc1_dgrad": fc1,
            "fc1_wgrad": fc1}
