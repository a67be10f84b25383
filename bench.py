"""Benchmark of the fused SwiGLU + MXFP8 path and the grouped GEMM on one MI355X.

One step = the bandwidth-stress workload: the fused row-scaled SwiGLU + MXFP8
forward and backward, both scale directions, at gate/up (131072, 8192) bf16
~N(0,1) passed as views of one packed [gate | up] buffer, fp32 row scale
~U(0.5,1.5), bf16 grad ~N(0,1e-2), with 0.1 % of aligned 1x32 and 32x1 blocks
of gate (and of grad) set to zero and 0.1 % of blocks of gate and of up holding
one ~N(0,1e3) outlier (page "[mxfp8 training] Add a fused gated-activation
(SwiGLU) + MXFP8 quantization kernel", Performance: the (131072, 8192) rows).
The backward writes the bf16 dgate/dup and the fp32 dscale besides the MXFP8
[dgate | dup].  value = algorithmic bytes of the step / step time, in GB/s
(inputs read once, outputs written once: forward 4 + n_dir*(1 + 1/32) B per
element + 4 B per row, backward 10 + 2*n_dir*(1 + 1/32) B per element + 8 B per
row).

Outside the timed region, for the record:
  * per_cell: every cell of the (4096, 2048), (4096, 7168), (16384, 7168)
    shapes and of (131072, 8192), forward and backward x rowwise / colwise /
    both, and the backward without dense outputs or dscale (the layout the
    torchao page times: 6 + 2*n_dir*(1 + 1/32) B per element + 4 B per row);
    p10 / median / p90 of device times with the caches flushed before each;
  * gemm: the expert-layer workload (Qwen3-MoE-like: 8192 tokens, hidden 2048,
    128 experts, top-8, intermediate 768) forward + backward through
    swiglu_mxfp8_quant_amd.moe with uniform softmax top-8 routing and plain
    SwiGLU, and with skewed Zipf(1.2) routing (8 empty experts) and the plain
    and the clamped SwiGLU: the whole layer's wall time (plain, with FC1's
    fused activation epilogue, and under the BF16-wgrad recipe, timed in
    turn; and the plain layer with its MXFP8 weight cache valid), each
    grouped GEMM's median time and TFLOP/s, the recipe's bf16 wgrads, and
    FC1 + activation unfused against fused; and (gemm.graph) the plain layer
    eager against a HIP-graph replay of the same step;
  * gemm_supplementary: a compute-bound grouped GEMM outside the workload
    configurations, labelled as such (row-major and K-blocked operands);
  * fused_expert: the fused forward and backward at the expert layer's width
    (65,536 rows of 768 columns in 128 groups, and 65,536 / 131,072 /
    262,144 rows in one group), timed like per_cell;
  * clocks: the GPU's current sclk / mclk as rocm-smi reports them;
  * cpu_baseline: the CPU oracle on a bounded sample of the step's workload,
    on one host thread and on all of the process's host cores, and the
    oracle's grouped GEMM on an FC2-shaped slice.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-moe]
Prints one JSON line.
"""
import argparse
import collections
import csv
import json
import os
import re
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

STRESS = (131072, 8192)
C2_SHAPES = [(4096, 2048), (4096, 7168), (16384, 7168)]
DIRS = [("row", 1), ("col", 2), ("both", 3)]
HBM_PEAK_GBS = 8000.0
STEP_CELLS = [("fwd", "both", STRESS, "dense"), ("bwd", "both", STRESS, "dense")]
DOMINANT = ("bwd", "both", STRESS, "dense")


def fwd_bytes(M, K, nd):
    return M * K * (4 + nd * (1 + 1 / 32)) + 4 * M


def bwd_bytes(M, K, nd, dense=True):
    if dense:
        return M * K * (10 + 2 * nd * (1 + 1 / 32)) + 8 * M
    return M * K * (6 + 2 * nd * (1 + 1 / 32)) + 4 * M


def ndir(d):
    return (d & 1) + ((d >> 1) & 1)


class Cell:
    """One (pass, direction, shape, output mode) call with its outputs
    preallocated.  mode "dense": the backward writes dgate/dup and dscale too;
    "codes": only the MXFP8 outputs (the forward is always "dense")."""

    def __init__(self, m, torch, data, kind, dname, dirs, shape, mode="dense"):
        M, K = shape
        self.kind, self.dname, self.dirs, self.shape, self.mode = kind, dname, dirs, shape, mode
        gu, sc, dy = data[shape]
        g, u = gu[:, :K], gu[:, K:]
        act = m.make_act()
        if kind == "fwd":
            rc, cc, rs, cs = m._alloc_mx(M, K, dirs, (M + 31) // 32, "cuda")
            ro, co = m._outs(rc, cc, rs, cs, dirs)
            self.keep = (rc, cc, rs, cs, ro, co, act)
            self.fn = lambda: m.mxq_swiglu_quantize_fwd(act, g, u, sc, None, dirs, ro, co)
            self.bytes = fwd_bytes(M, K, ndir(dirs))
        else:
            dense = mode == "dense"
            rc, cc, rs, cs = m._alloc_mx(M, 2 * K, dirs, (M + 31) // 32, "cuda")
            ro, co = m._outs(rc, cc, rs, cs, dirs)
            dd = torch.empty((M, 2 * K), dtype=torch.bfloat16, device="cuda") if dense else None
            ds = torch.empty(M, dtype=torch.float32, device="cuda") if dense else None
            nws = m.mxq_swiglu_quantize_bwd_workspace(M, K, dirs) if dense else 0
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if dense else None
            self.keep = (rc, cc, rs, cs, ro, co, dd, ds, ws, act)
            self.fn = lambda: m.mxq_swiglu_quantize_bwd(act, dy, g, u, sc, None,
                                                        dd[:, :K] if dense else None,
                                                        dd[:, K:] if dense else None, ds, dirs, ro, co, ws)
            self.bytes = bwd_bytes(M, K, ndir(dirs), dense)

    def key(self):
        return (self.kind, self.dname, self.shape, self.mode)

    def label(self):
        s = f"{self.kind}.{self.dname}.{self.shape[0]}x{self.shape[1]}"
        return s if self.mode == "dense" else s + ".codes_only"


def make_data(torch, W, shapes):
    data = {}
    for (M, K) in shapes:
        if (M, K) == STRESS:
            data[(M, K)] = W.stress_inputs(M, K, seed=0, device="cuda", frac=1e-3)
        else:
            data[(M, K)] = (W.packed_gate_up(M, K, seed=0, device="cuda"), W.row_scale(M, seed=0, device="cuda"),
                            W.grad_out(M, K, seed=0, device="cuda"))
    return data


def record_cells(m, torch, data):
    """Every cell outside the timed step (per_cell timings)."""
    cells = []
    for shape in C2_SHAPES + [STRESS]:
        for kind in ("fwd", "bwd"):
            for dname, d in DIRS:
                cells.append(Cell(m, torch, data, kind, dname, d, shape))
        for dname, d in DIRS:
            if shape in ((16384, 7168), STRESS):
                cells.append(Cell(m, torch, data, "bwd", dname, d, shape, "codes"))
    return cells


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (profiles/traffic.json), or None when the kernel source has
    changed since the counters were taken."""
    import hashlib
    tf = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(tf))["bwd_both_131072x8192"]
        src = b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])
        if hashlib.sha256(src).hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def percentiles(ts):
    ts = sorted(ts)
    q = lambda p: ts[min(len(ts) - 1, max(0, round(p * (len(ts) - 1))))]
    return q(0.1), q(0.5), q(0.9)


def gpu_clocks():
    """sclk / mclk of card 0 as rocm-smi reports them (strings), or the error."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=30)
        js = json.loads(r.stdout[r.stdout.index("{"):])
        card = js[sorted(js)[0]]
        return {k: v for k, v in card.items() if "sclk" in k or "mclk" in k or "fclk" in k}
    except Exception as e:  # the record only; never fails the benchmark
        return {"error": f"{type(e).__name__}: {e}"[:200]}


FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
MOE_VARIANTS = (("uniform_plain", False, False), ("zipf_plain", True, False), ("zipf_clamped", True, True))
GEMM_INNER = 4   # back-to-back calls per timing of a single GEMM (timed_alt)


def timed_alt(torch, fns, reps, inner=1):
    """Medians (us) of `reps` rounds that time each of fns, in turn, on the
    current stream (alternating, so that clock drift over the run falls on
    every variant alike).  Each timing covers `inner` calls back to back and
    reports the time per call: the host's time to issue the first call lies
    between the events, and over several calls it is a small share (the
    later calls are issued while the GPU runs the earlier ones)."""
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = [[] for _ in fns]
    for _ in range(reps):
        for i, fn in enumerate(fns):
            e0.record(stream)
            for _ in range(inner):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts[i].append(e0.elapsed_time(e1) * 1e3 / inner)
    return [sorted(t)[len(t) // 2] for t in ts]


def moe_section(m, torch, W, reps=5):
    """Expert-layer forward + backward: whole-layer timings (plain, with the
    fused FC1 epilogue, with the weight cache valid), per-GEMM timings, and
    FC1 + activation unfused against fused."""
    from swiglu_mxfp8_quant_amd.moe import Layer, gemm_flops
    out = {}
    for name, skewed, clamped in MOE_VARIANTS:
        moe = W.moe_layer(0, device="cuda", skewed=skewed)
        cfg = moe["cfg"]
        H, I, G = cfg["hidden"], cfg["inter"], cfg["experts"]
        R = int(moe["splits"].sum())
        layer = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped)
        # the same layer with FC1's fused epilogue (its W13 rows interleaved
        # in blocks of 128), and under the BF16-wgrad recipe
        fl = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped, fused_fc1=True)
        bl = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped, recipe="bf16_wgrad")
        # the recipe with the fused FC1 (its epilogue then writes the rowwise
        # cast only)
        fbl = Layer(moe["splits"], moe["w13"], moe["w2"], clamped=clamped, fused_fc1=True, recipe="bf16_wgrad")
        dy = W.moe_grad(R, H, seed=0, device="cuda")
        xs, sc = moe["x_perm"], moe["scale"]

        def full():
            layer.forward(xs, sc)
            layer.backward(dy)

        def full_fused():
            fl.forward(xs, sc)
            fl.backward(dy)

        def full_bf16():
            bl.forward(xs, sc)
            bl.backward(dy)

        def full_bf16_fused():
            fbl.forward(xs, sc)
            fbl.backward(dy)
        full()
        full_fused()
        full_bf16()
        full_bf16_fused()
        torch.cuda.synchronize()
        layer_us, fused_us, bf16_us, bf16_fused_us = timed_alt(torch, [full, full_fused, full_bf16, full_bf16_fused],
                                                                reps)
        # the plain layer with the MXFP8 weight cache valid (the device flag
        # skips the weight quantizations, as on the micro-batches after a
        # weight update)
        layer.mark_weights_current()
        cached_us, = timed_alt(torch, [full], reps)
        layer.mark_weights_changed()
        s, gr, ro, bo = layer.saved, layer.grads, layer.row_off, layer.block_off
        h13 = torch.empty_like(s["h13"])
        y = torch.empty((R, H), dtype=torch.bfloat16, device="cuda")
        da, dx = torch.empty_like(gr["da"]), torch.empty_like(gr["dx"])
        dw2, dw13 = torch.empty_like(gr["dw2"]), torch.empty_like(gr["dw13"])
        calls = {
            "fc1_fwd": (lambda: m.grouped_gemm(m.GEMM_NT, ro, xs, moe["w13"], h13), "bf16"),
            "fc2_fwd": (lambda: m.grouped_gemm(m.GEMM_NT, ro, s["a_r"], s["w2q"], y, s["as_r"], s["w2s"]), "fp8"),
            "fc2_dgrad": (lambda: m.grouped_gemm(m.GEMM_NN, ro, gr["dy_r"], gr["w2c"], da, gr["dys_r"], gr["w2cs"]),
                          "fp8"),
            "fc2_wgrad": (lambda: m.grouped_gemm(m.GEMM_TN, ro, gr["dy_c"], s["a_c"], dw2, gr["dys_c"], s["as_c"],
                                                 block_off=bo), "fp8"),
            "fc1_dgrad": (lambda: m.grouped_gemm(m.GEMM_NN, ro, gr["dq_r"], gr["w13c"], dx, gr["dqs_r"],
                                                 gr["w13cs"]), "fp8"),
            "fc1_wgrad": (lambda: m.grouped_gemm(m.GEMM_TN, ro, gr["dq_c"], gr["x_c"], dw13, gr["dqs_c"], gr["xs_c"],
                                                 block_off=bo), "fp8"),
        }
        flops = gemm_flops(R, H, I, G)
        per, tot_fl, tot_us = {}, 0.0, 0.0
        for k, (fn, dt) in calls.items():
            fn()
            us, = timed_alt(torch, [fn], reps, inner=GEMM_INNER)
            tf = flops[k] / us / 1e6
            peak = BF16_PEAK_TFLOPS if dt.startswith("bf16") else FP8_PEAK_TFLOPS
            per[k] = {"us": round(us, 1), "TFLOPs": round(tf, 1), "dtype": dt, "frac_peak": round(tf / peak, 4)}
            tot_fl += flops[k]
            tot_us += us
        # the recipe's two bf16 wgrads
        bs, bg = bl.saved, bl.grads
        bcalls = {
            "fc2_wgrad_bf16": lambda: m.grouped_gemm(m.GEMM_TN, ro, dy, bg["a_bf16"], dw2),
            "fc1_wgrad_bf16": lambda: m.grouped_gemm(m.GEMM_TN, ro, bg["dd"], bs["x_perm"], dw13),
        }
        per_bf16 = {}
        for k, fn in bcalls.items():
            fn()
            us, = timed_alt(torch, [fn], reps, inner=GEMM_INNER)
            tf = flops[k[:-5]] / us / 1e6
            per_bf16[k] = {"us": round(us, 1), "TFLOPs": round(tf, 1), "dtype": "bf16",
                           "frac_peak": round(tf / BF16_PEAK_TFLOPS, 4)}
        # FC1 + the activation's MXFP8 both ways: the bf16 FC1, then the fused
        # activation kernel, against FC1 with the activation in its epilogue
        unfused = lambda: (m.grouped_gemm(m.GEMM_NT, ro, xs, moe["w13"], h13),
                           m.swiglu_quantize_fwd(h13[:, :I], h13[:, I:], sc, True, True, ro, bo,
                                                 clamped=clamped, limit=layer.limit))
        fused = lambda: m.grouped_gemm_swiglu(ro, xs, fl.w13, h13, sc, True, True, block_off=bo,
                                              clamped=clamped, limit=layer.limit)
        # rowwise only (the BF16-wgrad recipe's cast)
        unfused_r = lambda: (m.grouped_gemm(m.GEMM_NT, ro, xs, moe["w13"], h13),
                             m.swiglu_quantize_fwd(h13[:, :I], h13[:, I:], sc, True, False,
                                                   clamped=clamped, limit=layer.limit))
        fused_r = lambda: m.grouped_gemm_swiglu(ro, xs, fl.w13, h13, sc, True, False, clamped=clamped,
                                                limit=layer.limit)
        for fn in (unfused, fused, unfused_r, fused_r):
            fn()
        fc1_act_us = [round(v, 1) for v in timed_alt(torch, [unfused, fused, unfused_r, fused_r], reps)]
        out[name] = {"routed_rows": R, "layer_fwd_bwd_us": round(layer_us, 1),
                     "layer_fwd_bwd_fused_fc1_us": round(fused_us, 1),
                     "layer_fwd_bwd_bf16_wgrad_recipe_us": round(bf16_us, 1),
                     "layer_fwd_bwd_bf16_wgrad_recipe_fused_fc1_us": round(bf16_fused_us, 1),
                     "layer_fwd_bwd_cached_weights_us": round(cached_us, 1),
                     "fc1_plus_activation_fwd_us": {"unfused": fc1_act_us[0], "fused": fc1_act_us[1],
                                                    "unfused_rowwise": fc1_act_us[2],
                                                    "fused_rowwise": fc1_act_us[3]},
                     "gemm_total_us": round(tot_us, 1), "gemm_TFLOPs": round(tot_fl / tot_us / 1e6, 1),
                     "per_gemm": per, "per_gemm_bf16_wgrad_recipe": per_bf16}
        del layer, fl, bl, fbl, moe, dy
        torch.cuda.empty_cache()
    return out


def graph_section(torch, W, reps=10):
    """The plain expert layer (uniform routing), forward + backward, eager
    against one HIP-graph replay of the same step (moe.capture_step), timed
    in turn; with the weight cache invalid (re-quantized every step) and
    valid."""
    from swiglu_mxfp8_quant_amd.moe import Layer, capture_step
    moe = W.moe_layer(0, device="cuda")
    H = moe["cfg"]["hidden"]
    R = int(moe["splits"].sum())
    dy = W.moe_grad(R, H, seed=0, device="cuda")
    eager = Layer(moe["splits"], moe["w13"], moe["w2"])
    captured = Layer(moe["splits"], moe["w13"], moe["w2"])
    graph, _ = capture_step(captured, moe["x_perm"], moe["scale"], dy)

    def step():
        eager.forward(moe["x_perm"], moe["scale"])
        eager.backward(dy)
    step()
    graph.replay()
    torch.cuda.synchronize()
    e_us, g_us = timed_alt(torch, [step, graph.replay], reps)
    eager.mark_weights_current()
    captured.mark_weights_current()
    ec_us, gc_us = timed_alt(torch, [step, graph.replay], reps)
    out = {"routing": "uniform_plain", "layer_fwd_bwd_eager_us": round(e_us, 1),
           "layer_fwd_bwd_graph_us": round(g_us, 1), "cached_weights_eager_us": round(ec_us, 1),
           "cached_weights_graph_us": round(gc_us, 1)}
    del graph, eager, captured, moe, dy
    torch.cuda.empty_cache()
    return out


def supplementary_gemm(m, torch, reps=5):
    """A compute-bound grouped shape, outside the workload's configurations
    (labelled as such): 8 equal groups of 4096 rows, N = K = 8192, NT, in
    MXFP8 (random finite E4M3 codes, unit-range E8M0 scales) and in bf16,
    each with row-major operands and with the same operands K-blocked by 64
    bytes (the layout change itself is not timed).  It shows the
    matrix-core rate the kernel reaches when the contraction is long and the
    output small against the flops."""
    G, rows, N, K = 8, 4096, 8192, 8192
    dev = "cuda"
    sp = torch.full((G,), rows, dtype=torch.int64, device=dev)
    ro, _bo, _ = m.splits_to_offsets(sp)
    R = G * rows
    out = torch.empty((R, N), dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    res = {"shape": f"{G} groups x {rows} rows, N = K = {N}, NT", "configuration": "supplementary, not a workload config"}
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for dt in ("fp8", "fp8_kblock", "bf16", "bf16_kblock"):
        if dt == "fp8":
            A = torch.randint(0, 0x70, (R, K), dtype=torch.uint8, device=dev, generator=g)
            B = torch.randint(0, 0x70, (G, N, K), dtype=torch.uint8, device=dev, generator=g)
            As = torch.full((R, K // 32), 120, dtype=torch.uint8, device=dev)
            Bs = torch.full((G, N, K // 32), 120, dtype=torch.uint8, device=dev)
            fn = lambda: m.grouped_gemm(m.GEMM_NT, ro, A, B, out, As, Bs)
        elif dt == "fp8_kblock":
            # the same codes K-blocked by 64 (the layout the quantizers can
            # write directly): every stage load covers whole cache lines
            Ak, Bk = m.KBlocked.from_rowmajor(A), m.KBlocked.from_rowmajor(B)
            A = B = None
            fn = lambda: m.grouped_gemm(m.GEMM_NT, ro, Ak, Bk, out, As, Bs)
        elif dt == "bf16":
            A = torch.randn((R, K), device=dev, generator=g).to(torch.bfloat16)
            B = torch.randn((G, N, K), device=dev, generator=g).to(torch.bfloat16)
            fn = lambda: m.grouped_gemm(m.GEMM_NT, ro, A, B, out)
        else:
            Ak, Bk = m.KBlocked.from_rowmajor(A), m.KBlocked.from_rowmajor(B)
            A = B = None
            fn = lambda: m.grouped_gemm(m.GEMM_NT, ro, Ak, Bk, out)
        fn()
        fn()
        ts = []
        for _ in range(reps):
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        us = sorted(ts)[len(ts) // 2]
        tf = 2.0 * R * N * K / us / 1e6
        peak = BF16_PEAK_TFLOPS if dt.startswith("bf16") else FP8_PEAK_TFLOPS
        res[dt] = {"us": round(us, 1), "TFLOPs": round(tf, 1), "frac_peak": round(tf / peak, 4)}
        fn = None
        if dt == "fp8_kblock":
            del Ak, Bk, As, Bs
        elif dt == "bf16_kblock":
            del Ak, Bk
    del out
    torch.cuda.empty_cache()
    return res


def fused_expert_section(m, torch, W, reps=9):
    """The fused forward and backward (plain SwiGLU, both directions, outputs
    preallocated) at the expert layer's width K = 768: 65,536 rows in 128
    equal groups (the layer's shape: the fused kernels of the configurations'
    expert layer) and 65,536 / 131,072 / 262,144 rows in one group; each
    call once untimed, then `reps` single calls timed like the per-cell
    record (caches flushed before each; the flush also covers the host's
    time to issue the call); medians and p10 / p90.  Shows how the launch's
    fixed cost spreads as M grows."""
    K, out = 768, {}
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        ts = []
        for _ in range(reps):
            flush.zero_()
            e0.record(stream)
            m.check(fn())
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        return percentiles(ts)

    act = m.make_act()
    for M, G in ((65536, 128), (65536, 0), (131072, 0), (262144, 0)):
        gu = W.packed_gate_up(M, K, seed=0, device="cuda")
        sc = W.row_scale(M, seed=0, device="cuda")
        dy = W.grad_out(M, K, seed=0, device="cuda")
        g, u = gu[:, :K], gu[:, K:]
        groups, ncb = None, (M + 31) // 32
        if G:
            ro, bo, _ = m.splits_to_offsets(torch.full((G,), M // G, dtype=torch.int64, device="cuda"))
            groups, ncb = m.make_groups(ro, bo), m.colwise_scale_rows_bound(M, G)
        fo = m._alloc_mx(M, K, 3, ncb, "cuda")
        f_row, f_col = m._outs(*fo, 3)
        bo_ = m._alloc_mx(M, 2 * K, 3, ncb, "cuda")
        b_row, b_col = m._outs(*bo_, 3)
        dd = torch.empty((M, 2 * K), dtype=torch.bfloat16, device="cuda")
        ds = torch.empty(M, dtype=torch.float32, device="cuda")
        ws = torch.empty(max(m.mxq_swiglu_quantize_bwd_workspace(M, K, 3), 1), dtype=torch.uint8, device="cuda")
        fwd = lambda: m.mxq_swiglu_quantize_fwd(act, g, u, sc, groups, 3, f_row, f_col)
        bwd = lambda: m.mxq_swiglu_quantize_bwd(act, dy, g, u, sc, groups, dd[:, :K], dd[:, K:], ds, 3, b_row, b_col,
                                                ws)
        m.check(fwd())
        m.check(bwd())
        torch.cuda.synchronize()
        (f10, f50, f90), (b10, b50, b90) = timed(fwd), timed(bwd)
        bf = M * K * (4 + 2 * (1 + 1 / 32)) + 4 * M
        bb = M * K * (10 + 4 * (1 + 1 / 32)) + 8 * M
        out[f"{M}x{K}" + (f"_G{G}" if G else "")] = {
            "fwd_both_us": round(f50, 1), "fwd_p10_us": round(f10, 1), "fwd_p90_us": round(f90, 1),
            "fwd_pct_hbm": round(bf / f50 / 1e3 / HBM_PEAK_GBS * 100, 1),
            "bwd_both_us": round(b50, 1), "bwd_p10_us": round(b10, 1), "bwd_p90_us": round(b90, 1),
            "bwd_pct_hbm": round(bb / b50 / 1e3 / HBM_PEAK_GBS * 100, 1)}
        del gu, dy, fo, bo_, dd, ds, ws
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(rows1=2048, rows_per_thread=1024, gemm_rows=64):
    """The CPU oracle (plain C in fp64, one element at a time) over a bounded
    sample of the step's workload: forward both + backward both of stress-
    structured rows of width 8192 (the same generators, at a smaller height),
    on one host thread, then on every host core the process may use (32-row
    stripes handed to a thread pool; the oracle's C calls release the GIL).
    Also the oracle's grouped GEMM on an FC2-shaped slice (gemm_rows rows of
    one expert, N = 2048, K = 768, MXFP8)."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle as O
    import workloads as W
    K = STRESS[1]
    cores = min(16, len(os.sched_getaffinity(0)))   # a GPU's share of the host

    def sample(rows):
        gu, sc, dy = W.stress_inputs(rows, K, seed=0, frac=1e-3)
        return W.bf16_bits(dy), W.bf16_bits(gu[:, :K]), W.bf16_bits(gu[:, K:]), sc.numpy()

    def run(part):
        d, g, u, s = part
        O.swiglu_quantize_fwd(g, u, s, 3)
        O.swiglu_quantize_bwd(d, g, u, s, 3)

    per_row = fwd_bytes(1, K, 2) + bwd_bytes(1, K, 2)
    d, g, u, s = sample(rows1)
    t0 = time.perf_counter()
    run((d, g, u, s))
    t1 = time.perf_counter() - t0
    rows_n = rows_per_thread * cores
    d, g, u, s = sample(rows_n)
    parts = [(d[i:i + 32], g[i:i + 32], u[i:i + 32], s[i:i + 32]) for i in range(0, rows_n, 32)]
    with ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(run, parts))
        tn = time.perf_counter() - t0
    # the oracle's GEMM: FC2 forward of one expert, MXFP8 NT
    rng = np.random.default_rng(0)
    N, KK = 2048, 768
    A = rng.integers(0, 0x70, (gemm_rows, KK)).astype(np.uint8)
    As = np.full((gemm_rows, KK // 32), 120, np.uint8)
    B = rng.integers(0, 0x70, (N, KK)).astype(np.uint8)
    Bs = np.full((N, KK // 32), 120, np.uint8)
    opB = O.Operand("mxfp8", B, 0, KK, 1, Bs, 0, KK // 32, 1)
    t0 = time.perf_counter()
    O.grouped_gemm("m", np.array([0, gemm_rows]), 0, N, KK, O.Operand("mxfp8", A, 0, KK, 1, As, 0, KK // 32, 1),
                   opB, "bf16")
    tg1 = time.perf_counter() - t0
    stripes = [(A[i:i + 8], As[i:i + 8]) for i in range(0, gemm_rows, 8)]
    gemm_one = lambda p: O.grouped_gemm("m", np.array([0, len(p[0])]), 0, N, KK,
                                        O.Operand("mxfp8", p[0], 0, KK, 1, p[1], 0, KK // 32, 1), opB, "bf16")
    with ThreadPoolExecutor(max_workers=cores) as ex:
        t0 = time.perf_counter()
        list(ex.map(gemm_one, stripes))
        tgn = time.perf_counter() - t0
    gfl = 2.0 * gemm_rows * N * KK
    return {"value": round(rows_n * per_row / tn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": (f"fused fwd both + bwd both over stress-structured rows of width {K}: {rows_n} rows "
                       f"({rows_n * per_row / 1e6:.0f} MB algorithmic) on {cores} threads in {tn:.1f} s; "
                       f"{rows1} rows on 1 thread in {t1:.1f} s"),
            "single_thread": {"value": round(rows1 * per_row / t1 / 1e9, 4), "unit": "GB/s", "cores": 1},
            "nproc": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model(),
            "gemm_oracle": {"shape": f"FC2 forward slice: {gemm_rows} x {N} x {KK} MXFP8",
                            "TFLOPs_1_thread": round(gfl / tg1 / 1e12, 8),
                            f"TFLOPs_{cores}_threads": round(gfl / tgn / 1e12, 8)}}


# ------------------------------------------------------------------ GEMM profile summary
# `--summarize-gemm-profile DIR`: the per-GEMM table of the grouped-GEMM
# profile from a rocprofv3 kernel trace (DIR/trace) and TCC_HIT/TCC_MISS
# (DIR/tcc) and FETCH_SIZE (DIR/fetch) counter runs of `--moe-only`.
# Dispatches are labelled by the kernel's template arguments (mode, dtype):
# NT bf16 is FC1 forward and NT MXFP8 FC2 forward; the NN (dgrad) and TN
# (wgrad) launches of FC2 and FC1 share a template, and `--moe-only` issues
# them in a fixed interleaving that the labeller checks dispatch by dispatch
# (a run in any other order stops with an error instead of mislabelling).

GP_ORDER = ["FC1 forward", "FC2 forward", "FC2 dgrad", "FC2 wgrad", "FC1 dgrad", "FC1 wgrad"]
GP_MODE = {"FC1 forward": "NT bf16", "FC2 forward": "NT MXFP8", "FC2 dgrad": "NN MXFP8", "FC2 wgrad": "TN MXFP8",
           "FC1 dgrad": "NN MXFP8", "FC1 wgrad": "TN MXFP8"}
GP_TEMPLATE = {"FC1 forward": "0, 0", "FC2 forward": "0, 1", "FC2 dgrad": "1, 1", "FC2 wgrad": "2, 1",
               "FC1 dgrad": "1, 1", "FC1 wgrad": "2, 1", "FC1 forward + act": "0, 0"}
# FC1 with the SwiGLU + MXFP8 epilogue: the same (mode, dtype), a non-zero
# epilogue argument (the last template argument; 1 SwiGLU, 2 clamped)
GP_FUSED = "FC1 forward + act"
GP_MODE[GP_FUSED] = "NT bf16 + act epilogue"
GP_FUSED_ORDER = [GP_FUSED] + GP_ORDER[1:]
# the same epilogue writing the rowwise cast only (the BF16-wgrad recipe's)
GP_FUSED_ROW = "FC1 forward + rowwise act"
GP_MODE[GP_FUSED_ROW] = "NT bf16 + rowwise act epilogue"
GP_TEMPLATE[GP_FUSED_ROW] = "0, 0"
# the BF16-wgrad recipe's wgrads: bf16 TN
GP_BF16_WGRADS = ["FC2 wgrad bf16", "FC1 wgrad bf16"]
GP_BF16_ORDER = GP_ORDER[:3] + [GP_BF16_WGRADS[0], GP_ORDER[4], GP_BF16_WGRADS[1]]
GP_BF16_FUSED_ORDER = [GP_FUSED_ROW] + GP_BF16_ORDER[1:]
for _g in GP_BF16_WGRADS:
    GP_MODE[_g] = "TN bf16"
    GP_TEMPLATE[_g] = "2, 0"
_FC1, _FC2 = 2 * 65536 * 2 * 768 * 2048, 2 * 65536 * 2048 * 768   # 65,536 routed rows, hidden 2048, intermediate 768
GP_FL = {"FC1 forward": _FC1, "FC2 forward": _FC2, "FC2 dgrad": _FC2, "FC2 wgrad": _FC2, "FC1 dgrad": _FC1,
         "FC1 wgrad": _FC1, GP_FUSED: _FC1, GP_FUSED_ROW: _FC1, "FC2 wgrad bf16": _FC2, "FC1 wgrad bf16": _FC1}
# algorithmic bytes of each GEMM: operands and their E8M0 scales read once, bf16 output written once
GP_BY = {"FC1 forward": 1275e6, "FC2 forward": 528e6, "FC2 dgrad": 447e6, "FC2 wgrad": 593e6, "FC1 dgrad": 787e6,
         "FC1 wgrad": 1048e6,
         # + the MXFP8 activation both ways (codes and E8M0 scales) and the row scale
         GP_FUSED: 1379e6,
         # + the rowwise MXFP8 activation and the row scale
         GP_FUSED_ROW: 1327e6,
         # bf16 operands (dY and the recomputed A; [dgate | dup] and X) and the bf16 dW
         "FC2 wgrad bf16": 771e6, "FC1 wgrad bf16": 1275e6}
GP_PEAK = {"NT bf16": 2500.0, "NT bf16 + act epilogue": 2500.0, "NT bf16 + rowwise act epilogue": 2500.0,
           "TN bf16": 2500.0}
GP_FETCH_SCALE = 2.0   # FETCH_SIZE calibration against a plain copy of known size
MOE_ONLY_REPS = 2


def _expected_gemm_sequence():
    """GEMM labels in the order `--moe-only` dispatches them: per routing, the
    plain layer, the layer with the fused FC1, the layer under the BF16-wgrad
    recipe and the recipe with the fused FC1 in turn, once untimed and
    MOE_ONLY_REPS times timed (each the six GEMMs in layer order), the plain
    layer MOE_ONLY_REPS times with the weight cache valid, each GEMM of the
    plain layer and then each bf16 wgrad once untimed and MOE_ONLY_REPS times
    timed (GEMM_INNER calls each), then FC1 + the activation unfused and
    fused, both directions and rowwise only, in turn, once untimed and
    MOE_ONLY_REPS times."""
    one = []
    for _ in range(1 + MOE_ONLY_REPS):
        one += GP_ORDER + GP_FUSED_ORDER + GP_BF16_ORDER + GP_BF16_FUSED_ORDER
    for _ in range(MOE_ONLY_REPS):
        one += GP_ORDER
    for g in GP_ORDER + GP_BF16_WGRADS:
        one += [g] * (1 + MOE_ONLY_REPS * GEMM_INNER)
    one += ["FC1 forward", GP_FUSED, "FC1 forward", GP_FUSED_ROW] * (1 + MOE_ONLY_REPS)
    return one * len(MOE_VARIANTS)


def _gemm_labels(rows):
    """Dispatch id -> GEMM label for the gemm_kernel rows of a trace (any
    order); checks every dispatch's template arguments against its label."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    seq = _expected_gemm_sequence()
    if len(rows) != len(seq):
        raise SystemExit(f"GEMM profile: {len(rows)} gemm_kernel dispatches, expected {len(seq)}")
    out = {}
    for r, lab in zip(rows, seq):
        t = re.search(r"gemm_kernel<(\d+), (\d+),[^>]*?(\d+)>", r["Kernel_Name"])
        if (t is None or f"{t.group(1)}, {t.group(2)}" != GP_TEMPLATE[lab]
                or (t.group(3) != "0") != (lab in (GP_FUSED, GP_FUSED_ROW))):
            raise SystemExit(f"GEMM profile: dispatch {r['Dispatch_Id']} ({r['Kernel_Name'][:60]}) is not {lab}")
        out[int(r["Dispatch_Id"])] = lab
    return out


def summarize_gemm_profile(base):
    tr = [r for r in csv.DictReader(open(f"{base}/trace/moe_kernel_trace.csv")) if "gemm_kernel" in r["Kernel_Name"]]
    lab = _gemm_labels(tr)
    dur = collections.defaultdict(list)
    for r in tr:
        dur[lab[int(r["Dispatch_Id"])]].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)

    def counters(path, names):
        rows = [r for r in csv.DictReader(open(path)) if "gemm_kernel" in r["Kernel_Name"]]
        first = {}
        for r in rows:
            first.setdefault(int(r["Dispatch_Id"]), r)
        lb = _gemm_labels(list(first.values()))
        acc = collections.defaultdict(lambda: collections.defaultdict(float))
        for r in rows:
            if r["Counter_Name"] in names:
                acc[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        per = collections.defaultdict(list)
        for d, v in acc.items():
            per[lb[d]].append(v)
        return per

    tcc = counters(f"{base}/tcc/moe_counter_collection.csv", {"TCC_HIT_sum", "TCC_MISS_sum"})
    fet = counters(f"{base}/fetch/moe_counter_collection.csv", {"FETCH_SIZE"})
    # optional: rocprofv3's derived MfmaUtil (matrix-core busy cycles over all SIMDs' cycles)
    mpath = f"{base}/mfma/moe_counter_collection.csv"
    mfu = counters(mpath, {"MfmaUtil"}) if os.path.exists(mpath) else None
    print("| GEMM | mode | dispatches | median us | TFLOP/s | % of dense peak | algorithmic bytes | flop/B |"
          " roofline-attainable TFLOP/s | % of attainable | L2 hit rate | HBM read MB |"
          + (" MFMA busy % |" if mfu else ""))
    print("|---|---|---|---|---|---|---|---|---|---|---|---|" + ("---|" if mfu else ""))
    for g in GP_ORDER + [GP_FUSED, GP_FUSED_ROW] + GP_BF16_WGRADS:
        us = statistics.median(dur[g])
        tf = GP_FL[g] / us / 1e6
        peak = GP_PEAK.get(GP_MODE[g], 5000.0)
        ai = GP_FL[g] / GP_BY[g]
        att = min(peak, ai * 8.0)   # flop/B x 8 TB/s, in TFLOP/s
        hits = statistics.median(v["TCC_HIT_sum"] / max(1.0, v["TCC_HIT_sum"] + v["TCC_MISS_sum"]) for v in tcc[g])
        mb = statistics.median(v["FETCH_SIZE"] for v in fet[g]) * 1024 * GP_FETCH_SCALE / 1e6
        busy = f" {statistics.median(v['MfmaUtil'] for v in mfu[g]):.1f} |" if mfu else ""
        print(f"| {g} | {GP_MODE[g]} | {len(dur[g])} | {us:.1f} | {tf:.0f} | {100 * tf / peak:.1f} | {GP_BY[g] / 1e6:.0f} MB |"
              f" {ai:.0f} | {att:.0f} | {100 * tf / att:.1f} | {100 * hits:.1f} % | {mb:.0f} |" + busy)


def time_cell(torch, m, c, flush, reps):
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ts = []
    for _ in range(reps):
        flush.zero_()   # evict the 256 MB Infinity Cache and the L2s
        e0.record(stream)
        m.check(c.fn())
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3)
    p10, p50, p90 = percentiles(ts)
    return {"us": round(p50, 2), "p10_us": round(p10, 2), "p90_us": round(p90, 2),
            "GBps": round(c.bytes / p50 / 1e3, 1), "pct_hbm": round(c.bytes / p50 / 1e3 / HBM_PEAK_GBS * 100, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-moe", action="store_true", help="skip the expert-layer (grouped GEMM) section")
    ap.add_argument("--no-cells", action="store_true", help="skip the per-cell record")
    ap.add_argument("--cell-reps", type=int, default=10)
    ap.add_argument("--fused-expert-only", action="store_true",
                    help="run only the fused forward/backward at the expert layer's width (for profiling)")
    ap.add_argument("--supp-only", action="store_true",
                    help="run only the compute-bound supplementary GEMM shape (for profiling) and print it")
    ap.add_argument("--moe-only", action="store_true",
                    help="only run the expert-layer section once and print its record (for profiling the GEMMs)")
    ap.add_argument("--summarize-gemm-profile", metavar="DIR",
                    help="print the per-GEMM table of a --moe-only profile (CPU only, no GPU run)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run the dominant call 3 times and a 1 GiB device copy 3 times "
                         "(for the HBM byte counters of rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.summarize_gemm_profile:
        summarize_gemm_profile(args.summarize_gemm_profile)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (--gpus {args.gpus} requested); "
              "the fused path shards by rows with no exchange, see the design notes", file=sys.stderr)
        sys.exit(2)

    import torch
    import swiglu_mxfp8_quant_amd as m
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    if args.moe_only:
        print(json.dumps({"gemm": moe_section(m, torch, W, reps=MOE_ONLY_REPS)}), flush=True)
        return
    if args.supp_only:
        print(json.dumps({"gemm_supplementary": supplementary_gemm(m, torch)}), flush=True)
        return
    if args.fused_expert_only:
        print(json.dumps({"fused_expert": fused_expert_section(m, torch, W)}), flush=True)
        return
    data = make_data(torch, W, [STRESS])
    cells = [Cell(m, torch, data, k, dn, dict(DIRS)[dn], sh, mo) for (k, dn, sh, mo) in STEP_CELLS]
    stream = torch.cuda.current_stream()
    dom = [c for c in cells if c.key() == DOMINANT][0]
    if args.traffic_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            m.check(dom.fn())
        for _ in range(3):
            dst.copy_(src)   # reference kernel: reads 1 GiB and writes 1 GiB
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe": True, "dominant_bytes": int(dom.bytes), "copy_bytes_each_way": 1 << 30}))
        return

    def step(ev=None):
        for c in cells:
            if c is dom and ev is not None:
                ev[0].record(stream)
                m.check(c.fn())
                ev[1].record(stream)
            else:
                m.check(c.fn())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"bench: {args.warmup} warm-up steps done", file=sys.stderr, flush=True)

    # the timed region: exactly `steps` steps, synchronized on both sides;
    # the dominant kernel is bracketed by events on its own stream
    dom_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(dom_ev[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    dom_ts = [a.elapsed_time(b) * 1e3 for a, b in dom_ev]
    dom_us = sum(dom_ts) / args.steps
    clocks = gpu_clocks()
    print(f"bench: {args.steps} timed steps done", file=sys.stderr, flush=True)

    step_bytes = sum(c.bytes for c in cells)
    ms_per_step = dt / args.steps * 1e3
    value = step_bytes / (dt / args.steps) / 1e9
    achieved = dom.bytes / dom_us / 1e3
    traffic = measured_traffic()
    p10, p50, p90 = percentiles(dom_ts)
    out = {
        "metric": "fused SwiGLU+MXFP8 quant GB/s (% HBM peak); grouped GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bandwidth stress: fused row-scaled SwiGLU + MXFP8 forward and backward, both "
                               "directions, gate/up (131072, 8192) packed [gate|up], 0.1% zero and 0.1% outlier "
                               "32-blocks; the backward also writes bf16 dgate/dup and fp32 dscale",
                   "cells": [c.label() for c in cells], "step_bytes": int(step_bytes),
                   "pct_hbm_peak": round(value / HBM_PEAK_GBS * 100, 1)},
        "roofline": {"kernel": "mxq_swiglu_quantize_bwd both (131072, 8192)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": int(dom.bytes), "avg_launch_us": round(dom_us, 2),
                     "p10_launch_us": round(p10, 2), "p90_launch_us": round(p90, 2)},
        "clocks": clocks,
    }
    del cells, dom
    torch.cuda.empty_cache()
    if not args.no_cells:
        data.update(make_data(torch, W, C2_SHAPES))
        rec = record_cells(m, torch, data)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        per_cell = {}
        for c in rec:
            m.check(c.fn())
            per_cell[c.label()] = time_cell(torch, m, c, flush, args.cell_reps)
        out["per_cell"] = per_cell
        del rec, flush
        print("bench: per-cell record done", file=sys.stderr, flush=True)
    del data
    torch.cuda.empty_cache()
    if not args.no_moe:
        out["gemm"] = moe_section(m, torch, W)
        out["gemm"]["graph"] = graph_section(torch, W)
        out["gemm_supplementary"] = supplementary_gemm(m, torch)
        out["fused_expert"] = fused_expert_section(m, torch, W)
        print("bench: grouped GEMM record done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
