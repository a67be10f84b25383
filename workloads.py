"""Seeded synthetic inputs for the fused SwiGLU + MXFP8 path and the MoE layer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic, so both the CPU oracle and the HIP library can be fed from
it.  Every tensor draws from its own torch.Generator seeded with
(seed, stream id), so any tensor can be regenerated on its own, on the CPU or
directly on the GPU (the CPU and GPU streams differ; a test that compares the
two sides generates once and copies the same bytes to both).

Shapes and distributions follow the workloads the pages measure:
  * gate/up (M, K) bf16 ~ N(0, 1), passed as views of one packed (M, 2K)
    buffer [gate | up] (the layout a fused w13 projection produces; page
    "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
    quantization kernel", API), row scale fp32 ~ U(0.5, 1.5), grad bf16
    ~ N(0, 1e-2);
  * a stress variant with 0.1 % all-zero 32-blocks and 0.1 % blocks holding
    one ~N(0, 1e3) outlier;
  * a Qwen3-MoE-shaped expert layer (hidden 2048, expert intermediate 768,
    128 experts, top-8; page ByteDance-Seed/VeOmni pull 1340, Test) with
    softmax top-8 routing, or a skewed Zipf(1.2) routing that leaves 8
    experts empty.
bf16 tensors are torch.bfloat16 (round-to-nearest-even from the fp32 draw).
"""
from __future__ import annotations

import torch

# stream ids: one per tensor role
_S_GATEUP, _S_SCALE, _S_GRAD = 1, 2, 3
_S_ZERO_R, _S_ZERO_C, _S_OUT_R, _S_OUT_C, _S_OUT_V, _S_GZERO_R, _S_GZERO_C = range(10, 17)
_S_LOGITS, _S_X, _S_W13, _S_W2, _S_DY, _S_PERM, _S_GUMBEL, _S_WLOGITS = range(20, 28)


def generator(seed: int, stream: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + int(stream))
    return g


def _normal(shape, std, seed, stream, device, dtype=torch.bfloat16):
    g = generator(seed, stream, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def packed_gate_up(M: int, K: int, seed: int = 0, device="cpu", std: float = 1.0):
    """(M, 2K) bf16 [gate | up]; gate = [:, :K], up = [:, K:]."""
    return _normal((M, 2 * K), std, seed, _S_GATEUP, device)


def row_scale(M: int, seed: int = 0, device="cpu"):
    """fp32 per-row scale ~ U(0.5, 1.5)."""
    g = generator(seed, _S_SCALE, device)
    return torch.rand((M,), generator=g, device=device, dtype=torch.float32).add_(0.5)


def grad_out(M: int, K: int, seed: int = 0, device="cpu"):
    """bf16 (M, K) ~ N(0, 1e-2) (the 1e-2 is the standard deviation)."""
    return _normal((M, K), 1e-2, seed, _S_GRAD, device)


def _block_mask_rows(M, K, frac, seed, stream, device):
    """Boolean (M/1, K/32) mask selecting a fraction of aligned 1x32 blocks."""
    g = generator(seed, stream, device)
    return torch.rand((M, K // 32), generator=g, device=device) < frac


def _block_mask_cols(M, K, frac, seed, stream, device):
    """Boolean (ceil(M/32), K) mask selecting a fraction of aligned 32x1 blocks."""
    g = generator(seed, stream, device)
    return torch.rand(((M + 31) // 32, K), generator=g, device=device) < frac


def _expand_row_mask(mask, M, K):
    return mask.repeat_interleave(32, dim=1)[:, :K]


def _expand_col_mask(mask, M, K):
    return mask.repeat_interleave(32, dim=0)[:M, :]


def stress_inputs(M: int, K: int, seed: int = 0, device="cpu", frac: float = 1e-3):
    """Bandwidth-stress inputs: packed [gate | up], scale and grad, with
    frac of aligned 1x32 and of 32x1 blocks of gate (and of grad) set to zero
    and frac of 1x32 and 32x1 blocks of gate and of up each given one element
    drawn from N(0, 1e3).  Returns (gate_up, scale, grad)."""
    gu = packed_gate_up(M, K, seed, device)
    sc = row_scale(M, seed, device)
    gr = grad_out(M, K, seed, device)
    gate = gu[:, :K]
    zr = _expand_row_mask(_block_mask_rows(M, K, frac, seed, _S_ZERO_R, device), M, K)
    zc = _expand_col_mask(_block_mask_cols(M, K, frac, seed, _S_ZERO_C, device), M, K)
    gate.masked_fill_(zr | zc, 0.0)
    gzr = _expand_row_mask(_block_mask_rows(M, K, frac, seed, _S_GZERO_R, device), M, K)
    gzc = _expand_col_mask(_block_mask_cols(M, K, frac, seed, _S_GZERO_C, device), M, K)
    gr.masked_fill_(gzr | gzc, 0.0)
    # outliers: one element per selected block, position and value seeded
    gpos = generator(seed, _S_OUT_V, device)
    for half in (0, 1):
        view = gu[:, half * K:(half + 1) * K]
        rmask = _block_mask_rows(M, K, frac, seed, _S_OUT_R + 100 * half, device)
        cmask = _block_mask_cols(M, K, frac, seed, _S_OUT_C + 100 * half, device)
        rr, bb = torch.nonzero(rmask, as_tuple=True)
        if rr.numel():
            off = torch.randint(0, 32, (rr.numel(),), generator=gpos, device=device)
            val = torch.randn((rr.numel(),), generator=gpos, device=device) * 1e3
            view[rr, bb * 32 + off] = val.to(torch.bfloat16)
        sb, cc = torch.nonzero(cmask, as_tuple=True)
        if sb.numel():
            off = torch.randint(0, 32, (sb.numel(),), generator=gpos, device=device)
            rows = torch.clamp(sb * 32 + off, max=M - 1)
            val = torch.randn((sb.numel(),), generator=gpos, device=device) * 1e3
            view[rows, cc] = val.to(torch.bfloat16)
    return gu, sc, gr


# ------------------------------------------------------------- MoE layer ---

QWEN3_MOE = dict(tokens=8192, hidden=2048, experts=128, topk=8, inter=768)


def _route_topk(logits: torch.Tensor, topk: int):
    """softmax over experts, top-k (ties -> lower expert id), weights = the
    softmax values (not renormalised)."""
    p = torch.softmax(logits.double(), dim=-1)
    T, E = p.shape
    # stable order: sort by (-p, expert id)
    order = torch.argsort(-p, dim=-1, stable=True)[:, :topk]
    w = torch.gather(p, 1, order)
    return order, w.float()


def _route_zipf(T: int, E: int, topk: int, seed: int, device, empty: int = 8, alpha: float = 1.2):
    """Skewed routing: experts ranked by a seeded permutation, p(rank r) ~ r^-alpha
    for the first E-empty ranks and 0 for the last `empty`; each token draws
    topk distinct experts by Gumbel-top-k on log p; weights = softmax of
    N(0,1) logits over the chosen experts."""
    gp = generator(seed, _S_PERM, "cpu")
    perm = torch.randperm(E, generator=gp)
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    p = ranks.pow(-alpha)
    p[E - empty:] = 0.0
    logp_rank = torch.log(p / p.sum())
    logp = torch.empty(E, dtype=torch.float64)
    logp[perm] = logp_rank          # expert perm[r] has rank r
    gg = generator(seed, _S_GUMBEL, "cpu")
    u = torch.rand((T, E), generator=gg, dtype=torch.float64).clamp_(1e-300, 1.0)
    gumbel = -torch.log(-torch.log(u))
    key = logp.unsqueeze(0) + gumbel
    order = torch.argsort(-key, dim=-1, stable=True)[:, :topk]
    gw = generator(seed, _S_WLOGITS, "cpu")
    wl = torch.randn((T, topk), generator=gw, dtype=torch.float64)
    w = torch.softmax(wl, dim=-1).float()
    return order.to(device), w.to(device)


def moe_layer(seed: int = 0, device="cpu", skewed: bool = False, tokens=None,
              hidden=None, experts=None, topk=None, inter=None, weights=True):
    """A Qwen3-MoE-shaped expert layer on synthetic data.

    Returns a dict with
      splits  int64 [G]             rows routed to each expert
      x_perm  bf16 (R, H)           token rows gathered in (expert, token) order
      scale   fp32 [R]              routing weight of each routed row
      token   int64 [R]             source token of each routed row
      w13     bf16 (G, 2I, H)       rows 0..I-1 = gate, I..2I-1 = up   (if weights)
      w2      bf16 (G, H, I)                                            (if weights)
    """
    cfg = dict(QWEN3_MOE)
    for k, v in dict(tokens=tokens, hidden=hidden, experts=experts, topk=topk, inter=inter).items():
        if v is not None:
            cfg[k] = v
    T, H, E, k, I = cfg["tokens"], cfg["hidden"], cfg["experts"], cfg["topk"], cfg["inter"]
    if skewed:
        order, w = _route_zipf(T, E, k, seed, "cpu")
    else:
        gl = generator(seed, _S_LOGITS, "cpu")
        logits = torch.randn((T, E), generator=gl, dtype=torch.float32)
        order, w = _route_topk(logits, k)
    expert = order.reshape(-1)
    token = torch.arange(T).repeat_interleave(k)
    wflat = w.reshape(-1)
    # sort routed rows by (expert, token)
    key = expert * T + token
    idx = torch.argsort(key, stable=True)
    expert, token, wflat = expert[idx], token[idx], wflat[idx]
    splits = torch.bincount(expert, minlength=E).to(torch.int64)
    x = _normal((T, H), 1.0, seed, _S_X, device)
    token_d = token.to(device)
    out = dict(cfg=cfg, splits=splits.to(device), token=token_d,
               x_perm=x.index_select(0, token_d), scale=wflat.to(device))
    if weights:
        out["w13"] = _normal((E, 2 * I, H), 0.02, seed, _S_W13, device)
        out["w2"] = _normal((E, H, I), 0.02, seed, _S_W2, device)
    return out


def moe_grad(R: int, H: int, seed: int = 0, device="cpu"):
    """dY (R, H) bf16 ~ N(0, 1e-2)."""
    return _normal((R, H), 1e-2, seed, _S_DY, device)


def bf16_bits(t: torch.Tensor):
    """A bf16 tensor's bit patterns as a numpy uint16 array (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def from_bits(bits, device="cpu"):
    """numpy uint16 bit patterns -> torch.bfloat16 tensor."""
    import numpy as np
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)

