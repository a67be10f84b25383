// act_quant.hip -- fused row-scaled SwiGLU + MXFP8 block quantization on gfx950:
// forward, backward (dgate, dup, dscale and the quantized [dgate | dup]) and the
// plain quantizer (identity activation); the row-scaled SReLU through the same
// kernels (unary: x in place of gate, dx in place of [dgate | dup]); gate and
// up either packed or interleaved in blocks of a multiple of 32 columns.
//
// Pages (cited by title; each defines what is computed here):
//   TAO4743 "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
//           quantization kernel": Summary (gate/up read once, the bf16
//           activation never stored, 1x32 and/or 32x1 RCEIL scales from one
//           pass), API (packed [gate | up], backward returns [dGate | dUp]),
//           Numerics and tests (bitwise match with the unfused definition).
//   TE3238  "Activation + GroupedLinear Fusion for MOE and other MOE
//           optimizations": Greptile Summary (per-row-scaled SReLU, SwiGLU and
//           ClampedSwiGLU; gradient of the scales), Important Files Changed
//           (the GLU interleave handled inside the scaled SwiGLU kernels).
//   VEO1340 ByteDance-Seed/VeOmni pull 1340, "What does this PR do?": SiLU is
//           rounded to the activation dtype before it multiplies up.
//
// Design (MI355X-first; the pages' CuTe DSL kernel for GB200 is prior art only):
//   * A workgroup owns one row tile (a colwise 32-row block, restarting at
//     every group) and a column slab: the forward splits the 32 rows over
//     4 waves of 8, the backward over 8 waves of 4; each lane owns 8
//     consecutive columns (a 512-column slab, 16-byte coalesced loads of gate
//     and up, and grad), or 4 (a 256-column slab, 8-byte loads) when the last
//     512-column slab would be at most half full; all rows' loads before any
//     arithmetic.  Work items are laid out so that each XCD takes a
//     contiguous range of them.
//   * Colwise: each wave keeps its rows' bf16 results in registers and the
//     32x1 amax combines the waves' partial maxima through LDS, so no second
//     HBM pass.  Rowwise: the 1x32 amax is a DPP max over the 4 (or 8) lanes
//     of the block.
//   * amax is an integer max of |bf16| bit patterns (NaN/Inf patterns sort
//     above every finite value), the scale byte comes straight from the amax
//     exponent bits, and gfx950's v_cvt_scalef32_pk_fp8_bf16 converts bf16
//     pairs to E4M3 with the block scale (exact RNE, probed over all bf16
//     inputs and scale bytes).  Codes and bf16 gradients leave with
//     nontemporal stores.
//   * Exactness: SiLU runs on v_exp_f32 / v_rcp_f32; an element whose fp32
//     result lies within a measured error margin of a bf16 rounding tie (or is
//     out of the range where the margin was measured, or involves a non-normal
//     fp32 value) is recomputed in fp64 the way the definition reads, so
//     results match the exact definition except within ~1e-15 of a tie.
#include "mxq_internal.h"
#include "act_math.h"

#include <math.h>

#include <mutex>

namespace mxq {
namespace {

// ------------------------------------------------------------------ loads

template <int CPT>
struct Vec;
template <>
struct Vec<8> {
    uint32_t w[4];
};
template <>
struct Vec<4> {
    uint32_t w[2];
};

// One row's CPT columns of a lane, nontemporal, through a buffer resource
// made from wave-uniform values only: `row` is the row's first element,
// `row_ok` whether the row lies inside the tile, `off` the lane's byte offset
// (kOffOut for lanes past the columns).  Rows and lanes outside load zeros
// (the resource's range is 0, or the offset lies past it) with no vector
// instruction spent on addresses or zero fills.
constexpr uint32_t kOffOut = 0x80000000u;   // past every range below
template <int CPT>
__device__ __forceinline__ Vec<CPT> load_row(const uint16_t *row, bool row_ok, uint32_t off) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(row), (short)0,
                                                                       row_ok ? 0x7FFFFFF0 : 0, 0x00020000);
    Vec<CPT> v;
    if constexpr (CPT == 8) {
        const u32x4_t q = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
        v.w[0] = q.x; v.w[1] = q.y; v.w[2] = q.z; v.w[3] = q.w;
    } else {
        const u32x2_t q = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 2));
        v.w[0] = q.x; v.w[1] = q.y;
    }
    return v;
}

// Stores through the same kind of resource: `row` wave-uniform, lanes with an
// offset of kOffOut (or rows with row_ok false) write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(void *row, bool row_ok) {
    return __builtin_amdgcn_make_buffer_rsrc(row, (short)0, row_ok ? 0x7FFFFFF0 : 0, 0x00020000);
}

// CPT bf16 (CPT / 2 packed words) at byte offset `off`, nontemporal
template <int CPT>
__device__ __forceinline__ void store_row_bf16(uint16_t *row, bool row_ok, uint32_t off, const uint32_t *w) {
    const __amdgpu_buffer_rsrc_t r = row_rsrc(row, row_ok);
    if constexpr (CPT == 8)
        __builtin_amdgcn_raw_buffer_store_b128(u32x4_t{w[0], w[1], w[2], w[3]}, r, off, 0, 2);
    else __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{w[0], w[1]}, r, off, 0, 2);
}

// CPT codes (CPT / 4 words) at byte offset `off`, nontemporal (NT), or
// through the cache: a K-blocked row's codes are 64-byte pieces, half lines
// whose other halves (the next row of the plane) the same wave writes next,
// which the L2 merges only if the stores go through it
template <int CPT, bool NT = true>
__device__ __forceinline__ void store_row_codes(uint8_t *row, bool row_ok, uint32_t off, const uint32_t *c) {
    const __amdgpu_buffer_rsrc_t r = row_rsrc(row, row_ok);
    constexpr int aux = NT ? 2 : 0;
    if constexpr (CPT == 8) __builtin_amdgcn_raw_buffer_store_b64(u32x2_t{c[0], c[1]}, r, off, 0, aux);
    else __builtin_amdgcn_raw_buffer_store_b32(c[0], r, off, 0, aux);
}

// Byte offset of column c's code from its row's start: c itself, or, with
// the codes K-blocked by 64 (row r's bytes k at (k / 64) plane + 64 r + k % 64,
// so the row's start is 64 r), (c / 64) plane + c % 64.  A lane's CPT
// columns never straddle a 64-column plane.
__device__ __forceinline__ uint32_t code_off(int c, int64_t plane) {
    return plane ? (uint32_t)((int64_t)(c >> 6) * plane + (c & 63)) : (uint32_t)c;
}

__device__ __forceinline__ void store_row_byte(uint8_t *row, uint32_t off, uint32_t v) {
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)v, row_rsrc(row, true), off, 0, 0);
}

template <int CPT>
__device__ __forceinline__ Vec<CPT> zero_vec() {
    Vec<CPT> v;
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) v.w[k] = 0u;
    return v;
}

// CPT/4 code dwords -> memory
template <int CPT>
__device__ __forceinline__ void store_codes(uint8_t *p, const uint32_t *c) {
    if constexpr (CPT == 8) __builtin_nontemporal_store(u32x2_t{c[0], c[1]}, reinterpret_cast<u32x2_t *>(p));
    else __builtin_nontemporal_store(c[0], reinterpret_cast<uint32_t *>(p));
}

// ------------------------------------------------------------------ tiles

// The dispatcher hands consecutive workgroups to the 8 XCDs in turn (block b
// runs on XCD b % 8, each with its own L2).  Grids are rounded up to a
// multiple of 8 and block b takes work item (b % 8) * (grid / 8) + b / 8, so
// each XCD owns a contiguous range of items: the column slabs of one row tile
// then share an L2, which merges their partial-line writes (the rowwise scale
// bytes of a row come from every slab) before they reach HBM.
constexpr int kXCD = 8;

__device__ __forceinline__ int64_t xcd_item(int64_t bid, int64_t grid) {
    return (bid % kXCD) * (grid / kXCD) + bid / kXCD;
}

inline int64_t xcd_grid(int64_t nwork) { return (nwork + kXCD - 1) / kXCD * kXCD; }

// The work item of block `bid`, or -1 for none.  A grouped colwise launch is
// sized for the bound on its 32-row blocks (one partial block per group on top
// of M / 32), but only block_off[G] of them exist: the items are spread over
// the XCDs by that count, so that the blocks left over are a few on every XCD
// rather than all on the last one, which would otherwise run the longest.
__device__ __forceinline__ int64_t work_item(int64_t bid, int64_t grid, int64_t nwork, int64_t nslabs,
                                             const Groups &gr, bool grouped) {
    if (!grouped) {
        const int64_t it = xcd_item(bid, grid);
        return it < nwork ? it : -1;
    }
    int64_t tiles = gr.block_off[gr.G];
    const int64_t bound = nwork / nslabs;
    tiles = tiles < 0 ? 0 : (tiles > bound ? bound : tiles);
    const int64_t n = tiles * nslabs, share = (n + kXCD - 1) / kXCD, i = bid / kXCD;
    const int64_t it = (bid % kXCD) * share + i;
    return (i < share && it < n) ? it : -1;
}

struct Tile {
    int64_t r0;    // first row
    int n;         // rows present (0 => nothing to do)
    int64_t srow;  // colwise scale row
};

// Row tile `t`: with groups, colwise tile t is global 32-row block t, found by a
// binary search of block_off (uniform, scalar loads); otherwise rows t*ROWS...
template <int ROWS>
__device__ __forceinline__ Tile tile_rows(int64_t t, int64_t M, const Groups &gr, bool grouped) {
    Tile T;
    T.srow = t;
    if (!grouped) {
        T.r0 = t * ROWS;
        const int64_t rem = M - T.r0;
        T.n = rem <= 0 ? 0 : (rem < ROWS ? (int)rem : ROWS);
        return T;
    }
    T.n = 0;
    T.r0 = 0;
    const int64_t G = gr.G;
    if (t >= gr.block_off[G] || t < 0) return T;
    int64_t lo = 0, hi = G;  // largest g with block_off[g] <= t
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (gr.block_off[mid] <= t) lo = mid;
        else hi = mid;
    }
    const int64_t r0 = gr.row_off[lo] + (t - gr.block_off[lo]) * 32;
    int64_t end = gr.row_off[lo + 1];
    if (end > M) end = M;
    const int64_t rem = end - r0;
    if (r0 < 0 || rem <= 0) return T;
    T.r0 = r0;
    T.n = rem < 32 ? (int)rem : 32;
    return T;
}

// ------------------------------------------------------------------ exact-path queue
//
// Pass 1 of every kernel below computes a row tile on the fast path and marks
// the elements whose result might differ from the exact definition in a
// per-lane bit mask (bit i * CPT + k for row i, column k).  Right after each
// row, if any lane of the wave marked an element of that row, every marking
// lane appends the element's bf16 inputs and position to its own LDS queue
// (kQ entries, stored slot-major so the lanes of a wave never conflict).
// After the tile, a rolled loop recomputes each lane's entries in fp64 (one
// copy of that code per kernel) and writes the results back into the queue;
// pass 2 merges them into the register tile, visiting only rows in which
// some lane has an entry.  A lane with more than kQ marked elements (only
// adversarial inputs get there) instead takes the slow path below, which
// walks its whole mask kQ elements at a time and re-reads their inputs from
// memory.

constexpr int kQ = 4;
constexpr int kFixQ = kQ;

__device__ __forceinline__ bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0ull; }

// low (hi = 0) or high half of a packed bf16 word
__device__ __forceinline__ uint32_t half16(uint32_t w, int hi) { return hi ? (w >> 16) : (w & 0xFFFFu); }

template <int ROWS, int CPT>
constexpr int risk_words() { return (ROWS * CPT + 31) / 32; }

template <int CPT>
__device__ __forceinline__ uint32_t row_bits(const uint32_t *risk, int i) {
    return (risk[(i * CPT) / 32] >> ((i * CPT) % 32)) & ((1u << CPT) - 1u);
}

// Slow path: gather the element indices of the set bits of rank
// [base, base + kFixQ) into q[0], q[QS], ... (a lane's column of the queue).
template <int NW, int QS>
__device__ __forceinline__ int fix_gather(const uint32_t *risk, int base, uint2 *q) {
    int rank = 0, nq = 0;
#pragma unroll
    for (int w = 0; w < NW; w++) {
        uint32_t bits = risk[w];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1u;
            if (rank >= base && nq < kFixQ) q[QS * nq++].x = (uint32_t)(w * 32 + b);
            rank++;
        }
    }
    return nq;
}

__device__ __forceinline__ uint32_t set_half(uint32_t w, int hi, uint32_t v) {
    return hi ? ((w & 0x0000FFFFu) | (v << 16)) : ((w & 0xFFFF0000u) | v);
}

__device__ __forceinline__ float bf16_at(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }


// ------------------------------------------------------------------ forward
//
// Work split: a workgroup of 4 waves owns one colwise block of up to 32 rows
// (restarting at every group) and a slab of 64 x CPT columns; wave w owns
// rows 8w..8w+7 of the block and each lane CPT consecutive columns (16-byte
// loads for CPT = 8, 8-byte for 4).  All 8 rows' loads are issued before any
// arithmetic.  The 1x32 amax is a DPP max over 32 / CPT lanes; the 32x1 amax
// is the max of the 4 waves' 8-row partial maxima, exchanged through LDS.

constexpr int RPW = 8;      // rows per wave
constexpr int NWAVE = 4;    // waves per workgroup
constexpr int TROWS = RPW * NWAVE;  // rows per tile (one colwise block)
// Columns per lane, CPT, is a template argument of the kernels: 8 (a 512-column
// slab per workgroup) or 4 (256 columns), chosen per launch (cols_per_lane).

constexpr int FNT = 64 * NWAVE;  // forward threads per workgroup

// Slow path for lanes whose marked elements overflowed the queue (their risk
// mask is passed; other lanes pass zeros); q is the lane's queue column; c0 is
// the lane's first column in the gate / up arrays (interleave applied).
template <int ACT, int CPT>
__device__ __forceinline__ void fwd_fix_slow(const FwdArgs &a, int64_t rbase, int c0, const uint32_t *risk,
                                          uint32_t (&h)[RPW][CPT / 2], uint2 *q) {
    constexpr int NWORDS = risk_words<RPW, CPT>();
    int total = 0;
#pragma unroll
    for (int w = 0; w < NWORDS; w++) total += __builtin_popcount(risk[w]);
    for (int base = 0; base < total; base += kFixQ) {
        const int nq = fix_gather<NWORDS, FNT>(risk, base, q);
#pragma unroll 1
        for (int j = 0; j < nq; j++) {
            const int idx = (int)q[FNT * j].x;
            const int64_t r = rbase + idx / CPT, c = c0 + idx % CPT;
            const float g = bf16_at(a.gate + r * a.ld_gate + c);
            const float u = gated<ACT>() ? bf16_at(a.up + r * a.ld_up + c) : 0.0f;
            const float s = a.row_scale != nullptr ? a.row_scale[r] : 1.0f;
            q[FNT * j].x = fwd_elem_f64(g, u, s, a.limit, ACT);
        }
        int rank = 0;
#pragma unroll
        for (int i = 0; i < RPW; i++) {
            const uint32_t rb = row_bits<CPT>(risk, i);
            if (rb) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    if (rb & (1u << k)) {
                        if (rank >= base && rank < base + nq) h[i][k >> 1] = set_half(h[i][k >> 1], k & 1, q[FNT * (rank - base)].x);
                        rank++;
                    }
                }
            }
        }
    }
}

// Is the row scale s safe for the fast product path (finite, normal or zero)?
__device__ __forceinline__ bool scale_ok(float s) { return normal_or_zero(s); }

// Scale bytes and NaN masks of CPT columns from their packed |bf16| maxima.
template <int CPT>
struct ColScales {
    uint32_t E[CPT];
    float s[CPT];
    uint32_t nan[CPT / 4];
};
template <int CPT>
__device__ __forceinline__ ColScales<CPT> col_scales(const uint32_t *cm) {
    ColScales<CPT> c;
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) {
        c.E[2 * k] = e8m0_from_amax_bits(cm[k] & 0xFFFFu);
        c.E[2 * k + 1] = e8m0_from_amax_bits(cm[k] >> 16);
    }
#pragma unroll
    for (int k = 0; k < CPT; k++) c.s[k] = scale_operand(c.E[k]);
#pragma unroll
    for (int q = 0; q < CPT / 4; q++) {
        c.nan[q] = 0u;
#pragma unroll
        for (int j = 0; j < 4; j++) c.nan[q] |= (c.E[4 * q + j] == 0xFFu ? 0xFFu : 0u) << (8 * j);
    }
    return c;
}

template <int CPT>
__device__ __forceinline__ void store_scale_bytes(uint8_t *p, const uint32_t *E) {
    uint32_t sb[CPT / 4];
#pragma unroll
    for (int q = 0; q < CPT / 4; q++)
        sb[q] = E[4 * q] | (E[4 * q + 1] << 8) | (E[4 * q + 2] << 16) | (E[4 * q + 3] << 24);
    store_codes<CPT>(p, sb);
}

// combine the 4 waves' partial column maxima (cmx[wave][lane][k]) for one lane
template <int CPT>
__device__ __forceinline__ void colmax_exchange(uint32_t (*cmx)[64][CPT / 2], int wave, int lane, uint32_t *cm) {
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) cmx[wave][lane][k] = cm[k];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) {
        uint32_t v = cmx[0][lane][k];
#pragma unroll
        for (int w = 1; w < NWAVE; w++) v = umax16x2(v, cmx[w][lane][k]);
        cm[k] = v;
    }
}

template <int ACT, int DIRS, int CPT>
__global__ void __launch_bounds__(FNT) fwd_kernel(FwdArgs a, int64_t nslabs, int64_t nwork) {
    constexpr int SLAB = 64 * CPT, NWORDS = risk_words<RPW, CPT>();
    __shared__ uint2 fq[kQ + 1][FNT];  // slot kQ takes the writes of lanes whose queue is full
    __shared__ uint32_t cmx[NWAVE][64][CPT / 2];
    const bool grouped = (DIRS & 2) && a.groups.G > 0;
    const int64_t item = work_item(blockIdx.x, gridDim.x, nwork, nslabs, a.groups, grouped);
    if (item < 0) return;  // grid padding (uniform over the workgroup)
    if (a.noop != nullptr && *a.noop != 0) return;  // a cached output that is still valid (uniform)
    const int64_t t = item / nslabs;
    const int64_t slab = item - t * nslabs;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int co = (int)(slab * SLAB) + lane * CPT;
    const bool active = co < a.K;
    // the lane's first column in the gate / up arrays: with gate and up
    // interleaved in blocks of il columns (il a multiple of 32, so a lane's 8
    // columns stay in one block), logical column j sits at 2 il (j / il) + j % il
    const int gco = a.il ? (co / a.il) * 2 * a.il + co % a.il : co;
    const Tile T = tile_rows<TROWS>(t, a.M, a.groups, grouped);
    if (T.n == 0) return;  // uniform over the workgroup
    const int nrow = min(max(T.n - wave * RPW, 0), RPW);  // rows of this wave (uniform per wave)
    const int64_t rbase = T.r0 + wave * RPW;
    const uint16_t *gate0 = a.gate + rbase * a.ld_gate;
    const uint16_t *up0 = gated<ACT>() ? a.up + rbase * a.ld_up : nullptr;

    // pass 1: all loads of the wave's rows, then the fast path
    Vec<CPT> gv[RPW], uv[RPW];
    const uint32_t goff = active ? (uint32_t)gco * 2u : kOffOut;
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        gv[i] = load_row<CPT>(gate0 + i * a.ld_gate, i < nrow, goff);
        if constexpr (gated<ACT>()) uv[i] = load_row<CPT>(up0 + i * a.ld_up, i < nrow, goff);
        else uv[i] = zero_vec<CPT>();
    }
    uint32_t h[RPW][CPT / 2];
    uint32_t risk[NWORDS];
    int nq = 0;  // this lane's marked elements (queued while nq <= kQ)
#pragma unroll
    for (int w = 0; w < NWORDS; w++) risk[w] = 0u;
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        float s = 1.0f;
        if constexpr (ACT != ACT_IDENTITY)
            if (a.row_scale != nullptr && i < nrow) s = a.row_scale[rbase + i];
        uint32_t bits = 0u;
#pragma unroll
        for (int k = CPT / 2 - 1; k >= 0; k--) {   // last pair first: its flags end in the top bits
            uint64_t m0, m1;
            fwd_pair_r<ACT>(gv[i].w[k], uv[i].w[k], s, a.limit, h[i][k], m0, m1);
            if constexpr (ACT != ACT_IDENTITY) bits = shift_in(shift_in(bits, m1), m0);
        }
        if constexpr (ACT != ACT_IDENTITY) {
            if (!scale_ok(s)) bits = (1u << CPT) - 1u;
            if (!active || i >= nrow) bits = 0u;
            risk[(i * CPT) / 32] |= bits << ((i * CPT) % 32);
            if (wave_any(bits != 0u)) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    const uint32_t c = (bits >> k) & 1u;
                    const int slot = c ? min(nq, kQ) : kQ;
                    fq[slot][tid] = make_uint2(half16(gv[i].w[k >> 1], k & 1) | (half16(uv[i].w[k >> 1], k & 1) << 16),
                                               (uint32_t)(i * CPT + k));
                    nq += (int)c;
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // the rare exact-path elements: queued ones in fp64, then the overflow lanes
    if constexpr (ACT != ACT_IDENTITY) {
        const int nfix = nq <= kQ ? nq : 0;
#pragma unroll 1
        for (int j = 0; j < nfix; j++) {
            const uint2 e = fq[j][tid];
            const float s = a.row_scale != nullptr ? a.row_scale[rbase + (int)e.y / CPT] : 1.0f;
            fq[j][tid].x = fwd_elem_f64(lo_f(e.x), hi_f(e.x), s, a.limit, ACT);
        }
        if (wave_any(nq > kQ)) {
            uint32_t rk[NWORDS];
#pragma unroll
            for (int w = 0; w < NWORDS; w++) rk[w] = nq > kQ ? risk[w] : 0u;
            fwd_fix_slow<ACT, CPT>(a, rbase, gco, rk, h, &fq[0][tid]);
        }
    }

    // pass 2: rowwise outputs and the wave's column maxima (rows past the
    // tile and lanes past K hold zeros; the latter form whole 32-column
    // groups of their own, so they never mix in)
    uint32_t cm[CPT / 2];
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) cm[k] = 0u;
    int rank = 0;
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        if constexpr (ACT != ACT_IDENTITY) {
            // merge this row's queued exact results
            const uint32_t rb = nq <= kQ ? row_bits<CPT>(risk, i) : 0u;
            if (wave_any(rb != 0u)) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    if (rb & (1u << k)) {
                        h[i][k >> 1] = set_half(h[i][k >> 1], k & 1, fq[rank][tid].x);
                        rank++;
                    }
                }
            }
        }
        if (a.h != nullptr) store_row_bf16<CPT>(a.h + (rbase + i) * a.ld_h, i < nrow, active ? (uint32_t)co * 2u : kOffOut, h[i]);
        uint32_t m = 0u;
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            const uint32_t mag = i < nrow ? (h[i][k] & 0x7FFF7FFFu) : 0u;
            if constexpr (DIRS & 2) cm[k] = umax16x2(cm[k], mag);
            m = umax16x2(m, mag);
        }
        if constexpr (DIRS & 1) {
            if (i < nrow) {
                m = block_max<32 / CPT>(max(m & 0xFFFFu, m >> 16));
                const uint32_t E = e8m0_from_amax_bits(m);
                uint32_t c[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) c[q] = cvt4_same(h[i][2 * q], h[i][2 * q + 1], E);
                const int64_t r = rbase + i;
                const uint32_t off = active ? code_off(co, a.row.plane) : kOffOut;
                if (a.row.plane) store_row_codes<CPT, false>(a.row.codes + r * a.row.ld_codes, true, off, c);
                else store_row_codes<CPT>(a.row.codes + r * a.row.ld_codes, true, off, c);
                store_row_byte(a.row.scales + r * a.row.ld_scales,
                               active && (lane & (32 / CPT - 1)) == 0 ? (uint32_t)co / 32u : kOffOut, E);
            }
        }
    }

    // pass 3: colwise outputs
    if constexpr (DIRS & 2) {
        colmax_exchange<CPT>(cmx, wave, lane, cm);
        if (!active) return;
        const ColScales<CPT> cs = col_scales<CPT>(cm);
        uint8_t *colc = a.col.codes + rbase * a.col.ld_codes;
#pragma unroll
        for (int i = 0; i < RPW; i++) {
            if (i < nrow) {
                uint32_t c[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) c[q] = cvt4_cols(h[i][2 * q], h[i][2 * q + 1], cs.s + 4 * q, cs.nan[q]);
                store_row_codes<CPT>(colc + i * a.col.ld_codes, true, (uint32_t)co, c);
            }
        }
        if (wave == 0) store_scale_bytes<CPT>(a.col.scales + T.srow * a.col.ld_scales + co, cs.E);
    }
}

// ------------------------------------------------------------------ backward

struct BwdPair {
    uint32_t dg, du;     // packed bf16 dgate / dup
    float dsum;          // dh*a*u of both elements
    uint64_t m[2];       // lanes whose low / high element needs the exact path
};

// Absolute error bound of the fast dgate tdg = fl(P * ds'), ds' =
// fl(sig' * fma(g, om', 1)) with P = fl(dh * u * s).  Measured against the
// exact silu'(g) for every bf16 g >= -80, |ds' - silu'(g)| stays below 0.51 of
//   sig * 2^-24 * (6 |1 + g (1 - sig)| + 3 |g| (1 - sig) (|g| + 3)),
// so that expression (a factor >= 1.98 of slack) bounds the silu' error; P
// and the final product add one rounding each, covered by 4 * 2^-24 |tdg|.
// Since |P| sig |1 + g (1 - sig)| is |tdg| up to two roundings, the bound is
//   2^-24 (10.5 |tdg| + 3 |P| sig |g| om (|g| + 3)).
__device__ __forceinline__ float dgate_err(float tdg, float P, float g, float sig, float om) {
    const float k = fabsf(g) * om;
    const float t3 = fmaf(fabsf(g), 3.0f * 0x1p-24f, 9.0f * 0x1p-24f);
    return fmaf(fabsf(tdg), 10.5f * 0x1p-24f, (fabsf(P) * sig) * (k * t3));
}

// Could an error of at most `bound` move t across a bf16 rounding tie?  The
// tie of t's own bf16 interval is tested directly; a bound that is not small
// against the bf16 quantum (2^-8 relative) is treated as risky outright, which
// covers the ties of the neighbouring intervals.  (Returns the lanes where it
// could.)
__device__ __forceinline__ uint64_t near_tie(float t, float bound) {
    const float tie = __uint_as_float((__float_as_uint(t) & 0xFFFF0000u) | 0x8000u);
    return lanes(fabsf(t - tie) <= bound) | lanes(bound > fabsf(t) * 0x1p-10f);
}

// SReLU backward of one element pair (x in gw): dx = bf16(dh * s * 2 v),
// v = max(x, 0), and dh * a (a = bf16(v^2)) for dscale.  dh * v and its double
// are exact in fp32 unless they leave the normal range; the product with s is
// the one rounding, so only its tie pattern (or a non-normal value) is risky.
__device__ __forceinline__ BwdPair bwd_pair_srelu(uint32_t dw, uint32_t gw, float s) {
    const float v[2] = {relu_f(lo_f(gw)), relu_f(hi_f(gw))};
    const float dh[2] = {lo_f(dw), hi_f(dw)};
    const float av[2] = {bf16_round(v[0] * v[0]), bf16_round(v[1] * v[1])};
    BwdPair out;
    float vdx[2];
    out.dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const float q2 = (dh[j] * v[j]) * 2.0f;   // exact
        const float tdx = q2 * s;                  // one rounding
        vdx[j] = tdx;
        out.dsum += dh[j] * av[j];                 // exact (8 x 8 bits)
        out.m[j] = product_risky(q2, tdx) | odd_lanes(v[j] * v[j]);
    }
    out.dg = pack_bf16(vdx[0], vdx[1]);
    out.du = 0u;
    return out;
}

template <int ACT>
__device__ __forceinline__ BwdPair bwd_pair(uint32_t dw, uint32_t gw, uint32_t uw, float s, float L) {
    if constexpr (ACT == ACT_SRELU) return bwd_pair_srelu(dw, gw, s);
    float g[2] = {lo_f(gw), hi_f(gw)}, u[2] = {lo_f(uw), hi_f(uw)};
    const float dh[2] = {lo_f(dw), hi_f(dw)};
    float mg[2] = {1.0f, 1.0f}, mu[2] = {1.0f, 1.0f};
    if constexpr (ACT == ACT_CLAMPED) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            mg[j] = g[j] > L ? 0.0f : 1.0f;
            mu[j] = (u[j] > L || u[j] < -L) ? 0.0f : 1.0f;
            g[j] = clamp_gate(g[j], L);
            u[j] = clamp_up(u[j], L);
        }
    }
    BwdPair out;
    float t[2], sg[2], om[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const Sig z = sig_fast(g[j]);
        sg[j] = z.sig;
        om[j] = z.e * z.sig;           // 1 - sigma without cancellation
        t[j] = g[j] * z.sig;
    }
    const float av[2] = {bf16_round(t[0]), bf16_round(t[1])};
    float vdg[2], vdu[2];
    out.dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const float q = dh[j] * av[j];          // exact (8 x 8 bits)
        const float qs = q * s;
        vdu[j] = qs * mu[j];
        out.dsum += q * u[j];                   // exact (24 bits) unless it underflows
        const float du_ = dh[j] * u[j];         // exact
        const float P = du_ * s;                // one rounding
        const float ds = sg[j] * (1.0f + g[j] * om[j]);
        const float tdg = P * ds * mg[j];
        vdg[j] = tdg;
        uint64_t m = silu_risky(g[j], t[j]) | product_risky(q, qs) | odd_lanes(du_) | odd_lanes(P) | odd_lanes(tdg);
        const uint64_t nt = near_tie(tdg, dgate_err(tdg, P, g[j], sg[j], om[j]));
        if constexpr (ACT == ACT_CLAMPED) m |= lanes(mg[j] != 0.0f) & nt;   // a clamped gate has dgate 0
        else m |= nt;
        out.m[j] = m;
    }
    out.dg = pack_bf16(vdg[0], vdg[1]);
    out.du = pack_bf16(vdu[0], vdu[1]);
    return out;
}

// fp64 recomputation of one backward element, in the definition's order.
// Returns dgate | dup << 16, and in *corr the change of dh*a*u caused by the
// exact a (the fast pass summed dh*a_fast*u into dscale).
template <int ACT>
__device__ __forceinline__ uint32_t bwd_elem_f64(float dhf, float gf, float uf, float s, float L, float *corr) {
    if constexpr (ACT == ACT_SRELU) {
        // dx = bf16(dh * s * 2 v) and a = bf16(v^2), v = max(x, 0): exact products in fp64
        const float vf = relu_f(gf);
        const double v = vf;
        const double a = (double)__uint_as_float(bf16_from_f64(v * v) << 16);
        const uint32_t dxb = bf16_from_f64((double)dhf * (double)s * 2.0 * v);
        const float af = lo_f(pack_bf16(vf * vf, 0.0f));   // the fast pass's a
        *corr = (float)a == af ? 0.0f : dhf * ((float)a - af);   // (an infinite a needs no correction)
        (void)uf;
        (void)L;
        return dxb;
    }
    double g = gf, u = uf;
    const double dh = dhf;
    double mg = 1.0, mu = 1.0;
    if (ACT == ACT_CLAMPED) {
        if (g > L) { mg = 0.0; g = L; }
        if (u > L || u < -L) { mu = 0.0; u = u > L ? (double)L : -(double)L; }
    }
    const double sg = sigmoid_f64(g);
    const uint32_t ab = bf16_from_f64(g * sg);
    const double a = (double)__uint_as_float(ab << 16);
    const double dsilu = sg * (1.0 + g * (1.0 - sg));
    const double sd = s;
    const uint32_t dgb = bf16_from_f64(dh * sd * u * dsilu * mg);
    const uint32_t dub = bf16_from_f64(dh * sd * a * mu);
    // the fast pass's a, recomputed with the same instructions
    const float gc = (float)g;
    const Sig z = sig_fast(gc);
    const float af = lo_f(pack_bf16(gc * z.sig, 0.0f));
    // (equal values, infinite ones included, need no correction: Inf - Inf would be NaN)
    *corr = (float)a == af ? 0.0f : (dhf * (float)u) * ((float)a - af);
    return dgb | (dub << 16);
}

// The backward splits a 32-row block over 8 waves of 4 rows (512 lanes): its
// per-element work is about twice the forward's, and 4 rows per wave keep it
// at ~100 VGPRs (4 waves per SIMD).
constexpr int BRPW = 4;
constexpr int BNWAVE = 8;

constexpr int BNT = 64 * BNWAVE;  // backward threads per workgroup

// Slow path for lanes whose marked elements overflowed the queue (see the
// forward's); the queue column's .x holds indices / results, .y corrections.
// c0 is the lane's first column of grad, gc0 of gate / up (interleave applied).
template <int ACT, int CPT>
__device__ __forceinline__ void bwd_fix_slow(const BwdArgs &a, int64_t rbase, int c0, int gc0, const uint32_t *risk,
                                             uint32_t (&hg)[BRPW][CPT / 2], uint32_t (&hu)[BRPW][CPT / 2],
                                             uint2 *q, float (&dsum)[BRPW]) {
    constexpr int BNWORDS = risk_words<BRPW, CPT>();
    int total = 0;
#pragma unroll
    for (int w = 0; w < BNWORDS; w++) total += __builtin_popcount(risk[w]);
    for (int base = 0; base < total; base += kFixQ) {
        const int nq = fix_gather<BNWORDS, BNT>(risk, base, q);
#pragma unroll 1
        for (int j = 0; j < nq; j++) {
            const int idx = (int)q[BNT * j].x;
            const int64_t r = rbase + idx / CPT, c = c0 + idx % CPT, gc = gc0 + idx % CPT;
            const float d = bf16_at(a.grad + r * a.ld_grad + c);
            const float g = bf16_at(a.gate + r * a.ld_gate + gc);
            const float u = gated<ACT>() ? bf16_at(a.up + r * a.ld_up + gc) : 0.0f;
            const float s = a.row_scale != nullptr ? a.row_scale[r] : 1.0f;
            float corr;
            q[BNT * j].x = bwd_elem_f64<ACT>(d, g, u, s, a.limit, &corr);
            q[BNT * j].y = __float_as_uint(corr);
        }
        int rank = 0;
#pragma unroll
        for (int i = 0; i < BRPW; i++) {
            const uint32_t rb = row_bits<CPT>(risk, i);
            if (rb) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    if (rb & (1u << k)) {
                        if (rank >= base && rank < base + nq) {
                            const uint2 v = q[BNT * (rank - base)];
                            hg[i][k >> 1] = set_half(hg[i][k >> 1], k & 1, v.x & 0xFFFFu);
                            hu[i][k >> 1] = set_half(hu[i][k >> 1], k & 1, v.x >> 16);
                            dsum[i] += __uint_as_float(v.y);
                        }
                        rank++;
                    }
                }
            }
        }
    }
}

// Backward over one tile x slab (8 waves of 4 rows, else as the forward).  Each lane
// owns CPT columns j of gate/up/grad and produces dgate (columns j of
// [dgate | dup]) and dup (columns K + j); with gate and up interleaved in
// blocks of il columns, the gradient takes the same layout (dgate at
// 2 il (j / il) + j % il, dup il columns on).  SReLU (unary) produces dx alone,
// at columns j of a (M x K) output.  dscale partials are reduced through LDS
// in a fixed order (deterministic) and written per (row, slab).
template <int ACT, int DIRS, int CPT>
__global__ void __launch_bounds__(BNT) bwd_kernel(BwdArgs a, int64_t nslabs, int64_t nwork) {
    constexpr int SLAB = 64 * CPT, BNWORDS = risk_words<BRPW, CPT>();
    __shared__ uint2 fq[kQ + 1][BNT];   // slot kQ takes the writes of lanes whose queue is full
    __shared__ uint32_t cmx[2][BNWAVE][64][CPT / 2];
    __shared__ float red[TROWS][65];
    __shared__ float red2[TROWS][9];
    const bool grouped = (DIRS & 2) && a.groups.G > 0;
    const int64_t item = work_item(blockIdx.x, gridDim.x, nwork, nslabs, a.groups, grouped);
    if (item < 0) return;  // grid padding (uniform over the workgroup)
    const int64_t t = item / nslabs;
    const int64_t slab = item - t * nslabs;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int co = (int)(slab * SLAB) + lane * CPT;
    const bool active = co < a.K;
    const int gco = a.il ? (co / a.il) * 2 * a.il + co % a.il : co;   // gate / up / dgate / dup column
    const int uoff = a.il ? a.il : (int)a.K;   // dup's columns of the MXFP8 [dgate | dup] lie this far on
    const Tile T = tile_rows<TROWS>(t, a.M, a.groups, grouped);
    if (T.n == 0) return;
    const int nrow = min(max(T.n - wave * BRPW, 0), BRPW);
    const int64_t rbase = T.r0 + wave * BRPW;
    const float L = a.limit;
    const bool dense = a.dgate != nullptr;
    const bool want_ds = a.dscale != nullptr;

    // pass 1: the fast path, PF rows of loads kept in flight
    constexpr int PF = 4;
    Vec<CPT> db[PF], gb[PF], ub[PF];
    const uint32_t doff = active ? (uint32_t)co * 2u : kOffOut, goff = active ? (uint32_t)gco * 2u : kOffOut;
    // output offsets: the codes of dgate / dup (bytes), and their rowwise scale bytes (one lane per 32 columns)
    const uint32_t coff_g = active ? (uint32_t)gco : kOffOut, coff_u = active ? (uint32_t)(gco + uoff) : kOffOut;
    const uint32_t rcoff_g = active ? code_off(gco, a.row.plane) : kOffOut;          // (rowwise codes, maybe K-blocked)
    const uint32_t rcoff_u = active ? code_off(gco + uoff, a.row.plane) : kOffOut;
    const bool scale_lane = active && (lane & (32 / CPT - 1)) == 0;
    const uint32_t soff_g = scale_lane ? (uint32_t)gco / 32u : kOffOut;
    const uint32_t soff_u = scale_lane ? (uint32_t)(gco + uoff) / 32u : kOffOut;
    const uint16_t *grad0 = a.grad + rbase * a.ld_grad, *gate0 = a.gate + rbase * a.ld_gate;
    const uint16_t *up0 = gated<ACT>() ? a.up + rbase * a.ld_up : nullptr;
    auto load3 = [&](int j, int i) {   // row i of the wave into prefetch slot j
        db[j] = load_row<CPT>(grad0 + i * a.ld_grad, i < nrow, doff);
        gb[j] = load_row<CPT>(gate0 + i * a.ld_gate, i < nrow, goff);
        if constexpr (gated<ACT>()) ub[j] = load_row<CPT>(up0 + i * a.ld_up, i < nrow, goff);
        else ub[j] = zero_vec<CPT>();
    };
#pragma unroll
    for (int i = 0; i < PF; i++) load3(i, i);
    uint32_t hg[BRPW][CPT / 2], hu[BRPW][CPT / 2];
    uint32_t risk[BNWORDS];
    float dsum[BRPW];
    int nq = 0;  // this lane's marked elements (queued while nq <= kQ)
#pragma unroll
    for (int w = 0; w < BNWORDS; w++) risk[w] = 0u;
#pragma unroll
    for (int i = 0; i < BRPW; i++) {
        const Vec<CPT> dv = db[i % PF], gv = gb[i % PF], uv = ub[i % PF];
        if (i + PF < BRPW) load3(i % PF, i + PF);
        const float s = (a.row_scale != nullptr && i < nrow) ? a.row_scale[rbase + i] : 1.0f;
        uint32_t bits = 0u;
        float ds = 0.0f;
        float pd[CPT / 2];
#pragma unroll
        for (int k = CPT / 2 - 1; k >= 0; k--) {   // last pair first: its flags end in the top bits
            const BwdPair p = bwd_pair<ACT>(dv.w[k], gv.w[k], uv.w[k], s, L);
            hg[i][k] = p.dg;
            hu[i][k] = p.du;
            pd[k] = p.dsum;
            bits = shift_in(shift_in(bits, p.m[1]), p.m[0]);
        }
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) ds += pd[k];   // the pairs' partial sums in column order
        if (!scale_ok(s)) bits = (1u << CPT) - 1u;
        if (!active || i >= nrow) {
            bits = 0u;
            ds = 0.0f;
        }
        risk[(i * CPT) / 32] |= bits << ((i * CPT) % 32);
        dsum[i] = ds;
        pin(dsum[i]);
        pin(risk[(i * CPT) / 32]);
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            pin(hg[i][k]);
            pin(hu[i][k]);
        }
        if (wave_any(bits != 0u)) {
#pragma unroll
            for (int k = 0; k < CPT; k++) {
                const uint32_t c = (bits >> k) & 1u;
                const int slot = c ? min(nq, kQ) : kQ;
                fq[slot][tid] = make_uint2(half16(gv.w[k >> 1], k & 1) | (half16(uv.w[k >> 1], k & 1) << 16),
                                          half16(dv.w[k >> 1], k & 1) | ((uint32_t)(i * CPT + k) << 16));
                nq += (int)c;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // the rare exact-path elements: queued ones in fp64, then the overflow lanes
    {
        const int nfix = nq <= kQ ? nq : 0;
#pragma unroll 1
        for (int j = 0; j < nfix; j++) {
            const uint2 e = fq[j][tid];
            const float s = a.row_scale != nullptr ? a.row_scale[rbase + (int)(e.y >> 16) / CPT] : 1.0f;
            float corr;
            const uint32_t v = bwd_elem_f64<ACT>(lo_f(e.y), lo_f(e.x), hi_f(e.x), s, L, &corr);
            fq[j][tid] = make_uint2(v, __float_as_uint(corr));
        }
        if (wave_any(nq > kQ)) {
            uint32_t rk[BNWORDS];
#pragma unroll
            for (int w = 0; w < BNWORDS; w++) rk[w] = nq > kQ ? risk[w] : 0u;
            bwd_fix_slow<ACT, CPT>(a, rbase, co, gco, rk, hg, hu, &fq[0][tid], dsum);
        }
    }

    // pass 2: dense outputs, rowwise outputs, the wave's column maxima
    uint32_t cmg[CPT / 2], cmu[CPT / 2];
#pragma unroll
    for (int k = 0; k < CPT / 2; k++) cmg[k] = cmu[k] = 0u;
    int rank = 0;
#pragma unroll
    for (int i = 0; i < BRPW; i++) {
        const int64_t r = rbase + i;
        {
            // merge this row's queued exact results
            const uint32_t rb = nq <= kQ ? row_bits<CPT>(risk, i) : 0u;
            if (wave_any(rb != 0u)) {
#pragma unroll
                for (int k = 0; k < CPT; k++) {
                    if (rb & (1u << k)) {
                        const uint2 v = fq[rank][tid];
                        hg[i][k >> 1] = set_half(hg[i][k >> 1], k & 1, v.x & 0xFFFFu);
                        hu[i][k >> 1] = set_half(hu[i][k >> 1], k & 1, v.x >> 16);
                        dsum[i] += __uint_as_float(v.y);
                        rank++;
                    }
                }
            }
        }
        if (dense) {
            store_row_bf16<CPT>(a.dgate + r * a.ld_dgate, i < nrow, goff, hg[i]);
            if constexpr (gated<ACT>()) store_row_bf16<CPT>(a.dup + r * a.ld_dup, i < nrow, goff, hu[i]);
        }
        uint32_t mg = 0u, mu = 0u;
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            const uint32_t ag = i < nrow ? (hg[i][k] & 0x7FFF7FFFu) : 0u;
            const uint32_t au = i < nrow ? (hu[i][k] & 0x7FFF7FFFu) : 0u;
            if constexpr (DIRS & 2) {
                cmg[k] = umax16x2(cmg[k], ag);
                cmu[k] = umax16x2(cmu[k], au);
            }
            mg = umax16x2(mg, ag);
            mu = umax16x2(mu, au);
        }
        if constexpr (DIRS & 1) {
            if (i < nrow) {
                mg = block_max<32 / CPT>(max(mg & 0xFFFFu, mg >> 16));
                mu = block_max<32 / CPT>(max(mu & 0xFFFFu, mu >> 16));
                const uint32_t Eg = e8m0_from_amax_bits(mg), Eu = e8m0_from_amax_bits(mu);
                uint32_t cg[CPT / 4], cu[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) {
                    cg[q] = cvt4_same(hg[i][2 * q], hg[i][2 * q + 1], Eg);
                    cu[q] = cvt4_same(hu[i][2 * q], hu[i][2 * q + 1], Eu);
                }
                uint8_t *rowc = a.row.codes + r * a.row.ld_codes;
                if (a.row.plane) {
                    store_row_codes<CPT, false>(rowc, true, rcoff_g, cg);
                    if constexpr (gated<ACT>()) store_row_codes<CPT, false>(rowc, true, rcoff_u, cu);
                } else {
                    store_row_codes<CPT>(rowc, true, rcoff_g, cg);
                    if constexpr (gated<ACT>()) store_row_codes<CPT>(rowc, true, rcoff_u, cu);
                }
                uint8_t *rs = a.row.scales + r * a.row.ld_scales;
                store_row_byte(rs, soff_g, Eg);
                if constexpr (gated<ACT>()) store_row_byte(rs, soff_u, Eu);
            }
        }
    }

    if (want_ds) {
        // this lane's dscale partials (corrected by the exact path) for the reduction
#pragma unroll
        for (int i = 0; i < BRPW; i++) red[wave * BRPW + i][lane] = dsum[i];
    }

    // pass 3: colwise outputs
    if constexpr (DIRS & 2) {
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            cmx[0][wave][lane][k] = cmg[k];
            cmx[1][wave][lane][k] = cmu[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            uint32_t vg = cmx[0][0][lane][k], vu = cmx[1][0][lane][k];
#pragma unroll
            for (int w = 1; w < BNWAVE; w++) {
                vg = umax16x2(vg, cmx[0][w][lane][k]);
                vu = umax16x2(vu, cmx[1][w][lane][k]);
            }
            cmg[k] = vg;
            cmu[k] = vu;
        }
        if (active) {
            const ColScales<CPT> sg = col_scales<CPT>(cmg), su = col_scales<CPT>(cmu);
            uint8_t *colc = a.col.codes + rbase * a.col.ld_codes;
#pragma unroll
            for (int i = 0; i < BRPW; i++) {
                if (i < nrow) {
                    uint32_t cg[CPT / 4], cu[CPT / 4];
#pragma unroll
                    for (int q = 0; q < CPT / 4; q++) {
                        cg[q] = cvt4_cols(hg[i][2 * q], hg[i][2 * q + 1], sg.s + 4 * q, sg.nan[q]);
                        cu[q] = cvt4_cols(hu[i][2 * q], hu[i][2 * q + 1], su.s + 4 * q, su.nan[q]);
                    }
                    store_row_codes<CPT>(colc + i * a.col.ld_codes, true, coff_g, cg);
                    if constexpr (gated<ACT>()) store_row_codes<CPT>(colc + i * a.col.ld_codes, true, coff_u, cu);
                }
            }
            if (wave == 0) {
                uint8_t *cs = a.col.scales + T.srow * a.col.ld_scales;
                store_scale_bytes<CPT>(cs + gco, sg.E);
                if constexpr (gated<ACT>()) store_scale_bytes<CPT>(cs + gco + uoff, su.E);
            }
        }
    }

    if (want_ds) {
        // deterministic reduction of the workgroup's dscale partials per row:
        // 8-lane segment sums in lane order, then the 8 segments in order
        __syncthreads();
        if (tid < 256) {
            const int row = tid >> 3, seg = tid & 7;
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++) acc += red[row][seg * 8 + j];
            red2[row][seg] = acc;
        }
        __syncthreads();
        if (tid < T.n) {
            float acc = 0.0f;
#pragma unroll
            for (int seg = 0; seg < 8; seg++) acc += red2[tid][seg];
            const int64_t r = T.r0 + tid;
            if (nslabs == 1) a.dscale[r] = acc;
            else a.partials[r * nslabs + slab] = acc;
        }
    }
}

// dscale[r] = sum over slabs of the partials, in slab order
__global__ void dscale_finish_kernel(const float *partials, int64_t nslabs, int64_t M, float *dscale) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= M) return;
    float acc = 0.0f;
    for (int64_t j = 0; j < nslabs; j++) acc += partials[r * nslabs + j];
    dscale[r] = acc;
}

// ------------------------------------------------------------------ launch

// Columns per lane of a launch: 8 (512-column slabs), or 4 (256-column slabs)
// when the last 512-column slab would be at most half full, as at K = 768
// (there the 4-column kernels take 11 % off the forward and 19 % off the
// backward; at K a multiple of 512 the 8-column ones are faster, by up to 8 %).
int cols_per_lane(int64_t K) {
    const int64_t r = K % 512;
    return (r != 0 && r <= 256) ? 4 : 8;
}

int64_t slabs_of(int64_t K) {
    const int64_t w = 64 * cols_per_lane(K);
    return (K + w - 1) / w;
}

int64_t tiles_of(int64_t M, const Groups &g, unsigned dirs) {
    const bool grouped = (dirs & 2) && g.G > 0;
    return grouped ? colwise_block_bound(M, g.G) : (M + TROWS - 1) / TROWS;
}

template <int ACT, int DIRS>
hipError_t fwd_launch(const FwdArgs &a, hipStream_t stream) {
    const int64_t ns = slabs_of(a.K);
    const int64_t nwork = tiles_of(a.M, a.groups, DIRS) * ns;
    if (nwork <= 0) return hipSuccess;
    if (cols_per_lane(a.K) == 4)
        hipLaunchKernelGGL((fwd_kernel<ACT, DIRS, 4>), dim3((unsigned)xcd_grid(nwork)), dim3(FNT), 0, stream, a, ns, nwork);
    else
        hipLaunchKernelGGL((fwd_kernel<ACT, DIRS, 8>), dim3((unsigned)xcd_grid(nwork)), dim3(FNT), 0, stream, a, ns, nwork);
    return hipGetLastError();
}

template <int ACT>
hipError_t fwd_dispatch(const FwdArgs &a, hipStream_t stream) {
    switch (a.dirs) {
        case 0: return fwd_launch<ACT, 0>(a, stream);   // the dense activation only
        case 1: return fwd_launch<ACT, 1>(a, stream);
        case 2: return fwd_launch<ACT, 2>(a, stream);
        default: return fwd_launch<ACT, 3>(a, stream);
    }
}

template <int ACT, int DIRS>
hipError_t bwd_launch(const BwdArgs &a, hipStream_t stream) {
    const int64_t ns = slabs_of(a.K);
    const int64_t nwork = tiles_of(a.M, a.groups, DIRS) * ns;
    if (nwork <= 0) return hipSuccess;
    if (cols_per_lane(a.K) == 4)
        hipLaunchKernelGGL((bwd_kernel<ACT, DIRS, 4>), dim3((unsigned)xcd_grid(nwork)), dim3(BNT), 0, stream, a, ns, nwork);
    else
        hipLaunchKernelGGL((bwd_kernel<ACT, DIRS, 8>), dim3((unsigned)xcd_grid(nwork)), dim3(BNT), 0, stream, a, ns, nwork);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dscale != nullptr && ns > 1) {
        const int64_t nb = (a.M + 255) / 256;
        hipLaunchKernelGGL(dscale_finish_kernel, dim3((unsigned)nb), dim3(256), 0, stream,
                           (const float *)a.partials, ns, a.M, a.dscale);
        e = hipGetLastError();
    }
    return e;
}

template <int ACT>
hipError_t bwd_dispatch(const BwdArgs &a, hipStream_t stream) {
    switch (a.dirs) {
        case 0: return bwd_launch<ACT, 0>(a, stream);
        case 1: return bwd_launch<ACT, 1>(a, stream);
        case 2: return bwd_launch<ACT, 2>(a, stream);
        default: return bwd_launch<ACT, 3>(a, stream);
    }
}

}  // namespace

hipError_t launch_act_quant_fwd(const FwdArgs &a, hipStream_t stream) {
    switch (a.act) {
        case ACT_SWIGLU: return fwd_dispatch<ACT_SWIGLU>(a, stream);
        case ACT_CLAMPED: return fwd_dispatch<ACT_CLAMPED>(a, stream);
        case ACT_SRELU: return fwd_dispatch<ACT_SRELU>(a, stream);
        default: return fwd_dispatch<ACT_IDENTITY>(a, stream);
    }
}

hipError_t launch_act_quant_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.act == ACT_CLAMPED) return bwd_dispatch<ACT_CLAMPED>(a, stream);
    if (a.act == ACT_SRELU) return bwd_dispatch<ACT_SRELU>(a, stream);
    return bwd_dispatch<ACT_SWIGLU>(a, stream);
}

int64_t act_quant_launch_threads(int64_t M, int64_t K, int64_t G, bool grouped_colwise, bool backward) {
    const int64_t tiles = grouped_colwise ? colwise_block_bound(M, G) : (M + TROWS - 1) / TROWS;
    return xcd_grid(tiles * slabs_of(K)) * (backward ? BNT : FNT);
}

size_t bwd_workspace_bytes(int64_t M, int64_t K) {
    const int64_t ns = slabs_of(K);
    return ns > 1 ? (size_t)M * (size_t)ns * sizeof(float) : 0;
}

// Scratch of the allocation-free backward: the per-(row, column slab) dscale
// partials, written in full by the backward kernel before the finisher reads
// them, so nothing needs clearing.  Each GPU the library runs on holds one
// copy until the process ends; calls that overlap on one GPU race on it.  In
// host code `scratch` names a host-side stand-in: only the address that
// hipGetSymbolAddress returns for the current device may reach a kernel.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

size_t bwd_scratch_capacity() { return kScratchBytes; }

hipError_t bwd_scratch(float **ptr) {
    static std::mutex mu;
    static float *addr[64] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<float *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace mxq
