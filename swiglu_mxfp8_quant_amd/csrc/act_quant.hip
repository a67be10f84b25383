// act_quant.hip -- fused row-scaled SwiGLU + MXFP8 block quantization on gfx950:
// forward, backward (dgate, dup, dscale and the quantized [dgate | dup]) and the
// plain quantizer (identity activation).
//
// Pages (cited by title; each defines what is computed here):
//   TAO4743 "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
//           quantization kernel": Summary (gate/up read once, the bf16
//           activation never stored, 1x32 and/or 32x1 RCEIL scales from one
//           pass), API (packed [gate | up], backward returns [dGate | dUp]),
//           Numerics and tests (bitwise match with the unfused definition).
//   TE3238  "Activation + GroupedLinear Fusion for MOE and other MOE
//           optimizations": Greptile Summary (per-row-scaled SwiGLU and
//           ClampedSwiGLU; gradient of the scales).
//   VEO1340 ByteDance-Seed/VeOmni pull 1340, "What does this PR do?": SiLU is
//           rounded to the activation dtype before it multiplies up.
//
// Design (MI355X-first; the pages' CuTe DSL kernel for GB200 is prior art only):
//   * A workgroup owns one row tile (a colwise 32-row block, restarting at
//     every group) and a 512-column slab: the forward splits the 32 rows over
//     4 waves of 8, the backward over 8 waves of 4; each lane owns 8
//     consecutive columns and issues 16-byte coalesced loads of gate and up
//     (and grad), all rows' loads before any arithmetic.  Work items are laid
//     out so that each XCD takes a contiguous range of them.
//   * Colwise: each wave keeps its rows' bf16 results in registers and the
//     32x1 amax combines the waves' partial maxima through LDS, so no second
//     HBM pass.  Rowwise: the 1x32 amax is a DPP max over the 4 lanes of the
//     block.
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

#include <math.h>

namespace mxq {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// fp32 classes {-normal, -zero, +zero, +normal} for v_cmp_class_f32
constexpr int kNormalOrZero = 0x168;

__device__ __forceinline__ bool normal_or_zero(float x) { return __builtin_amdgcn_classf(x, kNormalOrZero); }

__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2_t v;
    v.x = (__bf16)lo;
    v.y = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// Materialize x here: keeps the compiler from sinking the packing of a result
// word past later code (which would keep two fp32 values live instead of one word).
__device__ __forceinline__ void pin(uint32_t &x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(float &x) { asm volatile("" : "+v"(x)); }

__device__ __forceinline__ uint32_t umax16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}

// ------------------------------------------------------------------ fp64 path
//
// Used only for the rare elements whose fast fp32 result might round to a
// different bf16 than the exact value (see silu_risky / product_risky /
// near_tie below).  Evaluated in the order the definition reads, in fp64.

// double -> bf16 bits, round to nearest even: round to odd into fp32 (24 bits >=
// 8 + 2, so the second rounding is innocuous), then RNE to bf16.
__device__ __forceinline__ uint32_t bf16_from_f64(double d) {
    float f = (float)d;
    uint32_t b = __float_as_uint(f);
    if (d != d) return ((b >> 16) & 0x8000u) | 0x7FC0u;
    if ((double)f != d) {
        if (fabs((double)f) > fabs(d)) b -= 1u;
        b |= 1u;
    }
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ double sigmoid_f64(double g) { return 1.0 / (1.0 + exp(-g)); }

// ------------------------------------------------------------------ fast path

__device__ __forceinline__ float clamp_gate(float g, float L) { return g > L ? L : g; }
__device__ __forceinline__ float clamp_up(float u, float L) { return u > L ? L : (u < -L ? -L : u); }

// sigma(g) and its complement factor e = e^-g (1 - sigma = e * sigma)
struct Sig {
    float e, sig;
};
__device__ __forceinline__ Sig sig_fast(float g) {
    Sig r;
    r.e = __builtin_amdgcn_exp2f(g * -kLog2e);
    r.sig = __builtin_amdgcn_rcpf(1.0f + r.e);
    return r;
}

// May the fast fp32 silu t of g round to bf16 differently from the exact
// silu?  Measured against the exact silu for every bf16 g >= -80, the fast
// value is within 2.03 fp32 ulps for g >= 0 and within 2.25 + 0.7|g| ulps for
// g < 0 (the relative error of e^-g, which grows with |g|, reaches sigma only
// when e^-g is large); the margin 4 + 2 max(-g, 0) ulps covers that with a
// factor >= 1.78.  t's distance to the tie of its bf16 interval is
// 32768 - |low 16 bits of t read as int16| ulps, so the test below is
// "distance <= margin" rearranged into one add and one subtract (their own
// rounding, under 2^-7 ulp, is inside the slack).  For g < -80 (e^-g near
// overflow, sigma near the subnormal range) the element always takes the
// exact path.  Tiny g needs no special case: there sigma = 1/2 exactly and
// t = g/2 is exact, which is either a bf16 number that the exact silu
// (larger by ~g^2/4) also rounds to, or sits exactly on a tie (distance 0).
// For g > 80 the fast value is g itself, also the correctly rounded one.
__device__ __forceinline__ bool silu_risky(float g, float t) {
    const float z = fabsf((float)(short)__float_as_uint(t));
    return (bool)((int)(g < -80.0f) | (int)((z + fabsf(g)) - g >= 32764.0f));
}

// May bf16(hs), hs = fl32(p * s) with p exact, differ from the bf16 rounding of
// the exact product?  Only if hs sits exactly on a bf16 tie, or p / hs are not
// normal-or-zero (underflow, overflow, NaN/Inf inputs).
__device__ __forceinline__ bool product_risky(float p, float hs) {
    const bool tie = (__float_as_uint(hs) & 0xFFFFu) == 0x8000u;
    return (bool)((int)tie | (int)!normal_or_zero(p) | (int)!normal_or_zero(hs));
}

// ------------------------------------------------------------------ quantizer

// E8M0 byte from the largest |bf16| bit pattern m of a block (RCEIL).
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t m) {
    const int e = (int)((m + 0x1Fu) >> 7) - 8;  // mantissa > 0x60 (i.e. > 1.75) rounds the exponent up
    return m >= 0x7F80u ? 0xFFu : (e < 0 ? 0u : (uint32_t)e);
}

__device__ __forceinline__ float scale_operand(uint32_t E) { return __uint_as_float(E << 23); }

// Four bf16 (two packed words) -> four E4M3 codes with one block scale.
__device__ __forceinline__ uint32_t cvt4_same(uint32_t h01, uint32_t h23, uint32_t E) {
    const float s = scale_operand(E);
    short2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, h01), s, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, h23), s, true);
    const uint32_t c = __builtin_bit_cast(uint32_t, r);
    return E == 0xFFu ? 0x7F7F7F7Fu : c;
}

// Four bf16 of four different columns -> four codes, one scale per column.
__device__ __forceinline__ uint32_t cvt4_cols(uint32_t h01, uint32_t h23, const float *s,
                                              uint32_t nanmask) {
    short2_t x = {0, 0}, y = {0, 0};
    x = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(x, __builtin_bit_cast(bf16x2_t, h01), s[0], false);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(x, __builtin_bit_cast(bf16x2_t, h23), s[2], true);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(y, __builtin_bit_cast(bf16x2_t, h01), s[1], false);
    y = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(y, __builtin_bit_cast(bf16x2_t, h23), s[3], true);
    const uint32_t c = (__builtin_bit_cast(uint32_t, y) & 0xFF00FF00u) |
                       (__builtin_bit_cast(uint32_t, x) & 0x00FF00FFu);
    return (c & ~nanmask) | (0x7F7F7F7Fu & nanmask);
}

// max over the LPB lanes that share a 1x32 block (LPB = 32 / CPT, aligned groups)
template <int LPB>
__device__ __forceinline__ uint32_t block_max(uint32_t m) {
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, true));  // lane ^ 1
    m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, true));  // lane ^ 2
    // quads now hold their max; mirroring within each 8-lane half row pairs quad 0 with quad 1
    if (LPB == 8) m = max(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x141, 0xF, 0xF, true));
    return m;
}

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

template <int CPT>
__device__ __forceinline__ Vec<CPT> load_vec(const uint16_t *p) {
    Vec<CPT> v;
    if constexpr (CPT == 8) {
        const u32x4_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
        v.w[0] = q.x; v.w[1] = q.y; v.w[2] = q.z; v.w[3] = q.w;
    } else {
        const u32x2_t q = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p));
        v.w[0] = q.x; v.w[1] = q.y;
    }
    return v;
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

template <int CPT>
__device__ __forceinline__ void store_bf16(uint16_t *p, const uint32_t *w) {
    if constexpr (CPT == 8) __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_t *>(p));
    else __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t *>(p));
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
// (restarting at every group) and a slab of 512 columns; wave w owns rows
// 8w..8w+7 of the block and each lane 8 consecutive columns (16-byte loads).
// All 8 rows' loads are issued before any arithmetic, so a wave keeps 16 KB
// in flight.  The 1x32 amax is a DPP max over 4 lanes; the 32x1 amax is the
// max of the 4 waves' 8-row partial maxima, exchanged through LDS.

constexpr int CPT = 8;      // columns per lane
constexpr int RPW = 8;      // rows per wave
constexpr int NWAVE = 4;    // waves per workgroup
constexpr int TROWS = RPW * NWAVE;  // rows per tile (one colwise block)
constexpr int SLAB = 64 * CPT;      // columns per workgroup
constexpr int NWORDS = RPW * CPT / 32;  // risk mask words per lane

// One element pair of the forward: packed gate / up words -> packed h word.
// Returns a 2-bit mask of the elements that need the exact path.
template <int ACT>
__device__ __forceinline__ uint32_t fwd_pair(uint32_t gw, uint32_t uw, float s, float L, uint32_t &hw) {
    if constexpr (ACT == ACT_IDENTITY) {
        hw = gw;
        return 0u;
    } else {
        float g0 = lo_f(gw), g1 = hi_f(gw), u0 = lo_f(uw), u1 = hi_f(uw);
        if constexpr (ACT == ACT_CLAMPED) {
            g0 = clamp_gate(g0, L); g1 = clamp_gate(g1, L);
            u0 = clamp_up(u0, L);   u1 = clamp_up(u1, L);
        }
        const Sig s0 = sig_fast(g0), s1 = sig_fast(g1);
        const float t0 = g0 * s0.sig, t1 = g1 * s1.sig;
        const uint32_t aw = pack_bf16(t0, t1);
        const float p0 = lo_f(aw) * u0, p1 = hi_f(aw) * u1;
        const float h0 = p0 * s, h1 = p1 * s;
        hw = pack_bf16(h0, h1);
        uint32_t risky = 0u;
        risky |= (uint32_t)silu_risky(g0, t0) | (uint32_t)product_risky(p0, h0);
        risky |= ((uint32_t)silu_risky(g1, t1) | (uint32_t)product_risky(p1, h1)) << 1;
        return risky;
    }
}

// h = bf16( bf16(silu(g)) * u * s ) in fp64 (the product is exact in fp64)
__device__ __forceinline__ uint32_t fwd_elem_f64(float g, float u, float s, float L, int act) {
    if (act == ACT_CLAMPED) {
        g = clamp_gate(g, L);
        u = clamp_up(u, L);
    }
    const double gd = (double)g;
    const float a = __uint_as_float(bf16_from_f64(gd * sigmoid_f64(gd)) << 16);
    return bf16_from_f64((double)a * (double)u * (double)s);
}

constexpr int FNT = 64 * NWAVE;  // forward threads per workgroup

// Slow path for lanes whose marked elements overflowed the queue (their risk
// mask is passed; other lanes pass zeros); q is the lane's queue column.
template <int ACT>
__device__ __forceinline__ void fwd_fix_slow(const FwdArgs &a, int64_t rbase, int c0, const uint32_t *risk,
                                          uint32_t (&h)[RPW][CPT / 2], uint2 *q) {
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
            const float u = bf16_at(a.up + r * a.ld_up + c);
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
struct ColScales {
    uint32_t E[CPT];
    float s[CPT];
    uint32_t nan[CPT / 4];
};
__device__ __forceinline__ ColScales col_scales(const uint32_t *cm) {
    ColScales c;
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

__device__ __forceinline__ void store_scale_bytes(uint8_t *p, const uint32_t *E) {
    uint32_t sb[CPT / 4];
#pragma unroll
    for (int q = 0; q < CPT / 4; q++)
        sb[q] = E[4 * q] | (E[4 * q + 1] << 8) | (E[4 * q + 2] << 16) | (E[4 * q + 3] << 24);
    store_codes<CPT>(p, sb);
}

// combine the 4 waves' partial column maxima (cmx[wave][lane][k]) for one lane
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

template <int ACT, int DIRS>
__global__ void __launch_bounds__(FNT) fwd_kernel(FwdArgs a, int64_t nslabs, int64_t nwork) {
    __shared__ uint2 fq[kQ + 1][FNT];  // slot kQ takes the writes of lanes whose queue is full
    __shared__ uint32_t cmx[NWAVE][64][CPT / 2];
    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    if (item >= nwork) return;  // grid padding (uniform over the workgroup)
    const int64_t t = item / nslabs;
    const int64_t slab = item - t * nslabs;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int co = (int)(slab * SLAB) + lane * CPT;
    const bool active = co < a.K;
    const Tile T = tile_rows<TROWS>(t, a.M, a.groups, (DIRS & 2) && a.groups.G > 0);
    if (T.n == 0) return;  // uniform over the workgroup
    const int nrow = min(max(T.n - wave * RPW, 0), RPW);  // rows of this wave (uniform per wave)
    const int64_t rbase = T.r0 + wave * RPW;
    const uint16_t *gate0 = a.gate + rbase * a.ld_gate;
    const uint16_t *up0 = a.up + rbase * a.ld_up;

    // pass 1: all loads of the wave's rows, then the fast path
    Vec<CPT> gv[RPW], uv[RPW];
#pragma unroll
    for (int i = 0; i < RPW; i++) {
        gv[i] = zero_vec<CPT>();
        uv[i] = zero_vec<CPT>();
        if (i < nrow && active) {
            gv[i] = load_vec<CPT>(gate0 + i * a.ld_gate + co);
            if constexpr (ACT != ACT_IDENTITY) uv[i] = load_vec<CPT>(up0 + i * a.ld_up + co);
        }
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
        for (int k = 0; k < CPT / 2; k++) bits |= fwd_pair<ACT>(gv[i].w[k], uv[i].w[k], s, a.limit, h[i][k]) << (2 * k);
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
            fwd_fix_slow<ACT>(a, rbase, co, rk, h, &fq[0][tid]);
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
        uint32_t m = 0u;
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            const uint32_t mag = i < nrow ? (h[i][k] & 0x7FFF7FFFu) : 0u;
            if constexpr (DIRS & 2) cm[k] = umax16x2(cm[k], mag);
            m = umax16x2(m, mag);
        }
        if constexpr (DIRS & 1) {
            if (i < nrow) {
                m = block_max<4>(max(m & 0xFFFFu, m >> 16));
                const uint32_t E = e8m0_from_amax_bits(m);
                uint32_t c[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) c[q] = cvt4_same(h[i][2 * q], h[i][2 * q + 1], E);
                if (active) {
                    const int64_t r = rbase + i;
                    store_codes<CPT>(a.row.codes + r * a.row.ld_codes + co, c);
                    if ((lane & 3) == 0) a.row.scales[r * a.row.ld_scales + co / 32] = (uint8_t)E;
                }
            }
        }
    }

    // pass 3: colwise outputs
    if constexpr (DIRS & 2) {
        colmax_exchange(cmx, wave, lane, cm);
        if (!active) return;
        const ColScales cs = col_scales(cm);
        uint8_t *colc = a.col.codes + rbase * a.col.ld_codes;
#pragma unroll
        for (int i = 0; i < RPW; i++) {
            if (i < nrow) {
                uint32_t c[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) c[q] = cvt4_cols(h[i][2 * q], h[i][2 * q + 1], cs.s + 4 * q, cs.nan[q]);
                store_codes<CPT>(colc + i * a.col.ld_codes + co, c);
            }
        }
        if (wave == 0) store_scale_bytes(a.col.scales + T.srow * a.col.ld_scales + co, cs.E);
    }
}

// ------------------------------------------------------------------ backward

struct BwdPair {
    uint32_t dg, du;     // packed bf16 dgate / dup
    float dsum;          // dh*a*u of both elements
    uint32_t risky;      // 2-bit mask
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
// covers the ties of the neighbouring intervals.
__device__ __forceinline__ bool near_tie(float t, float bound) {
    const float tie = __uint_as_float((__float_as_uint(t) & 0xFFFF0000u) | 0x8000u);
    return (bool)((int)(fabsf(t - tie) <= bound) | (int)(bound > fabsf(t) * 0x1p-10f));
}

template <int ACT>
__device__ __forceinline__ BwdPair bwd_pair(uint32_t dw, uint32_t gw, uint32_t uw, float s, float L) {
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
    const uint32_t aw = pack_bf16(t[0], t[1]);
    const float av[2] = {lo_f(aw), hi_f(aw)};
    float vdg[2], vdu[2];
    out.risky = 0u;
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
        uint32_t r = (uint32_t)silu_risky(g[j], t[j]) | (uint32_t)product_risky(q, qs);
        r |= (uint32_t)!normal_or_zero(du_) | (uint32_t)!normal_or_zero(P) | (uint32_t)!normal_or_zero(tdg);
        r |= (uint32_t)(mg[j] != 0.0f) & (uint32_t)near_tie(tdg, dgate_err(tdg, P, g[j], sg[j], om[j]));
        out.risky |= r << j;
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
    *corr = (dhf * (float)u) * ((float)a - af);
    return dgb | (dub << 16);
}

// The backward splits a 32-row block over 8 waves of 4 rows (512 lanes): its
// per-element work is about twice the forward's, and 4 rows per wave keep it
// at ~100 VGPRs (4 waves per SIMD).
constexpr int BRPW = 4;
constexpr int BNWAVE = 8;
constexpr int BNWORDS = BRPW * CPT / 32;

constexpr int BNT = 64 * BNWAVE;  // backward threads per workgroup

// Slow path for lanes whose marked elements overflowed the queue (see the
// forward's); the queue column's .x holds indices / results, .y corrections.
template <int ACT>
__device__ __forceinline__ void bwd_fix_slow(const BwdArgs &a, int64_t rbase, int c0, const uint32_t *risk,
                                             uint32_t (&hg)[BRPW][CPT / 2], uint32_t (&hu)[BRPW][CPT / 2],
                                             uint2 *q, float (&dsum)[BRPW]) {
    int total = 0;
#pragma unroll
    for (int w = 0; w < BNWORDS; w++) total += __builtin_popcount(risk[w]);
    for (int base = 0; base < total; base += kFixQ) {
        const int nq = fix_gather<BNWORDS, BNT>(risk, base, q);
#pragma unroll 1
        for (int j = 0; j < nq; j++) {
            const int idx = (int)q[BNT * j].x;
            const int64_t r = rbase + idx / CPT, c = c0 + idx % CPT;
            const float d = bf16_at(a.grad + r * a.ld_grad + c);
            const float g = bf16_at(a.gate + r * a.ld_gate + c);
            const float u = bf16_at(a.up + r * a.ld_up + c);
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
// owns 8 columns j of gate/up/grad and produces dgate (columns j of
// [dgate | dup]) and dup (columns K + j).  dscale partials are reduced
// through LDS in a fixed order (deterministic) and written per (row, slab).
template <int ACT, int DIRS>
__global__ void __launch_bounds__(BNT) bwd_kernel(BwdArgs a, int64_t nslabs, int64_t nwork) {
    __shared__ uint2 fq[kQ + 1][BNT];   // slot kQ takes the writes of lanes whose queue is full
    __shared__ uint32_t cmx[2][BNWAVE][64][CPT / 2];
    __shared__ float red[TROWS][65];
    __shared__ float red2[TROWS][9];
    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    if (item >= nwork) return;  // grid padding (uniform over the workgroup)
    const int64_t t = item / nslabs;
    const int64_t slab = item - t * nslabs;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;  // wave index is uniform
    const int co = (int)(slab * SLAB) + lane * CPT;
    const bool active = co < a.K;
    const Tile T = tile_rows<TROWS>(t, a.M, a.groups, (DIRS & 2) && a.groups.G > 0);
    if (T.n == 0) return;
    const int nrow = min(max(T.n - wave * BRPW, 0), BRPW);
    const int64_t rbase = T.r0 + wave * BRPW;
    const float L = a.limit;
    const int K = (int)a.K;
    const bool dense = a.dgate != nullptr;
    const bool want_ds = a.dscale != nullptr;

    // pass 1: the fast path, PF rows of loads kept in flight
    constexpr int PF = 4;
    Vec<CPT> db[PF], gb[PF], ub[PF];
#pragma unroll
    for (int i = 0; i < PF; i++) {
        db[i] = gb[i] = ub[i] = zero_vec<CPT>();
        if (i < nrow && active) {
            const int64_t r = rbase + i;
            db[i] = load_vec<CPT>(a.grad + r * a.ld_grad + co);
            gb[i] = load_vec<CPT>(a.gate + r * a.ld_gate + co);
            ub[i] = load_vec<CPT>(a.up + r * a.ld_up + co);
        }
    }
    uint32_t hg[BRPW][CPT / 2], hu[BRPW][CPT / 2];
    uint32_t risk[BNWORDS];
    float dsum[BRPW];
    int nq = 0;  // this lane's marked elements (queued while nq <= kQ)
#pragma unroll
    for (int w = 0; w < BNWORDS; w++) risk[w] = 0u;
#pragma unroll
    for (int i = 0; i < BRPW; i++) {
        const Vec<CPT> dv = db[i % PF], gv = gb[i % PF], uv = ub[i % PF];
        if (i + PF < BRPW && i + PF < nrow && active) {
            const int64_t r = rbase + i + PF;
            db[i % PF] = load_vec<CPT>(a.grad + r * a.ld_grad + co);
            gb[i % PF] = load_vec<CPT>(a.gate + r * a.ld_gate + co);
            ub[i % PF] = load_vec<CPT>(a.up + r * a.ld_up + co);
        }
        const float s = (a.row_scale != nullptr && i < nrow) ? a.row_scale[rbase + i] : 1.0f;
        uint32_t bits = 0u;
        float ds = 0.0f;
#pragma unroll
        for (int k = 0; k < CPT / 2; k++) {
            const BwdPair p = bwd_pair<ACT>(dv.w[k], gv.w[k], uv.w[k], s, L);
            hg[i][k] = p.dg;
            hu[i][k] = p.du;
            ds += p.dsum;
            bits |= p.risky << (2 * k);
        }
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
            bwd_fix_slow<ACT>(a, rbase, co, rk, hg, hu, &fq[0][tid], dsum);
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
        if (dense && active && i < nrow) {
            store_bf16<CPT>(a.dgate + r * a.ld_dgate + co, hg[i]);
            store_bf16<CPT>(a.dup + r * a.ld_dup + co, hu[i]);
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
                mg = block_max<4>(max(mg & 0xFFFFu, mg >> 16));
                mu = block_max<4>(max(mu & 0xFFFFu, mu >> 16));
                const uint32_t Eg = e8m0_from_amax_bits(mg), Eu = e8m0_from_amax_bits(mu);
                uint32_t cg[CPT / 4], cu[CPT / 4];
#pragma unroll
                for (int q = 0; q < CPT / 4; q++) {
                    cg[q] = cvt4_same(hg[i][2 * q], hg[i][2 * q + 1], Eg);
                    cu[q] = cvt4_same(hu[i][2 * q], hu[i][2 * q + 1], Eu);
                }
                if (active) {
                    uint8_t *rowc = a.row.codes + r * a.row.ld_codes;
                    store_codes<CPT>(rowc + co, cg);
                    store_codes<CPT>(rowc + K + co, cu);
                    if ((lane & 3) == 0) {
                        uint8_t *rs = a.row.scales + r * a.row.ld_scales;
                        rs[co / 32] = (uint8_t)Eg;
                        rs[(K + co) / 32] = (uint8_t)Eu;
                    }
                }
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
            const ColScales sg = col_scales(cmg), su = col_scales(cmu);
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
                    store_codes<CPT>(colc + i * a.col.ld_codes + co, cg);
                    store_codes<CPT>(colc + i * a.col.ld_codes + K + co, cu);
                }
            }
            if (wave == 0) {
                uint8_t *cs = a.col.scales + T.srow * a.col.ld_scales;
                store_scale_bytes(cs + co, sg.E);
                store_scale_bytes(cs + K + co, su.E);
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

int64_t slabs_of(int64_t K) { return (K + SLAB - 1) / SLAB; }

int64_t tiles_of(int64_t M, const Groups &g, unsigned dirs) {
    const bool grouped = (dirs & 2) && g.G > 0;
    return grouped ? colwise_block_bound(M, g.G) : (M + TROWS - 1) / TROWS;
}

template <int ACT, int DIRS>
hipError_t fwd_launch(const FwdArgs &a, hipStream_t stream) {
    const int64_t ns = slabs_of(a.K);
    const int64_t nwork = tiles_of(a.M, a.groups, DIRS) * ns;
    if (nwork <= 0) return hipSuccess;
    hipLaunchKernelGGL((fwd_kernel<ACT, DIRS>), dim3((unsigned)xcd_grid(nwork)), dim3(FNT), 0, stream, a, ns, nwork);
    return hipGetLastError();
}

template <int ACT>
hipError_t fwd_dispatch(const FwdArgs &a, hipStream_t stream) {
    switch (a.dirs) {
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
    hipLaunchKernelGGL((bwd_kernel<ACT, DIRS>), dim3((unsigned)xcd_grid(nwork)), dim3(BNT), 0, stream, a, ns, nwork);
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
        default: return fwd_dispatch<ACT_IDENTITY>(a, stream);
    }
}

hipError_t launch_act_quant_bwd(const BwdArgs &a, hipStream_t stream) {
    if (a.act == ACT_CLAMPED) return bwd_dispatch<ACT_CLAMPED>(a, stream);
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

}  // namespace mxq
