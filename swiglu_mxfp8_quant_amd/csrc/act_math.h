// act_math.h -- the device arithmetic of the row-scaled activations and of the
// MXFP8 block quantizer, shared by the fused activation kernels
// (act_quant.hip) and the grouped GEMM's fused SwiGLU epilogue
// (grouped_gemm.hip), so that both produce the same bits: the fast fp32 path
// with its tie / range checks, the fp64 path for the elements those checks
// flag, the E8M0 scale from a block's |bf16| maximum (RCEIL) and the scaled
// E4M3 conversion.
//
// Pages: "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
// quantization kernel" (Summary: RCEIL scales; Numerics and tests: bitwise
// equality with the unfused definition); "Activation + GroupedLinear Fusion
// for MOE and other MOE optimizations" (Greptile Summary: the row-scaled
// SReLU, SwiGLU and ClampedSwiGLU); ByteDance-Seed/VeOmni pull 1340 ("What
// does this PR do?": SiLU rounded to the activation dtype before it
// multiplies up).
#pragma once

#include <math.h>

#include "mxq_internal.h"

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

// x rounded to bf16 (RNE), as an fp32: converting x into the high half of a
// packed pair whose low half is +0 gives exactly those bits, in one
// instruction.  (Written out: from the pair's plain form the compiler makes a
// convert into the low half and a shift or permute, two instructions per
// element, as it does when a packed pair is unpacked.)
__device__ __forceinline__ float bf16_round(float x) {
    uint32_t r;
    asm("v_cvt_pk_bf16_f32 %0, 0, %1" : "=v"(r) : "v"(x));
    return __uint_as_float(r);
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

// A comparison's lanes as a wave mask.  The checks below return such masks,
// combined with scalar ORs: a mask taken of a single comparison is that
// comparison's own result, whereas a flag made of several comparisons would
// be turned into a 0 / 1 vector value and compared again.
__device__ __forceinline__ uint64_t lanes(bool cmp) { return __builtin_amdgcn_ballot_w64(cmp); }

// Lanes where x is not normal-or-zero: the class test's own lane mask (written
// out, since the mask of the class intrinsic is not taken directly either),
// inverted within the active lanes.
__device__ __forceinline__ uint64_t odd_lanes(float x) {
    uint64_t m;
    asm("v_cmp_class_f32_e64 %0, %1, %2" : "=s"(m) : "v"(x), "s"(kNormalOrZero));
    return __builtin_amdgcn_read_exec() & ~m;
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
// (Returns the lanes where it may.)
__device__ __forceinline__ uint64_t silu_risky(float g, float t) {
    const float z = fabsf((float)(short)__float_as_uint(t));
    return lanes(g < -80.0f) | lanes((z + fabsf(g)) - g >= 32764.0f);
}

// May bf16(hs), hs = fl32(p * s) with p exact, differ from the bf16 rounding of
// the exact product?  Only if hs sits exactly on a bf16 tie, or p / hs are not
// normal-or-zero (underflow, overflow, NaN/Inf inputs).  (Returns the lanes.)
__device__ __forceinline__ uint64_t product_risky(float p, float hs) {
    return lanes((__float_as_uint(hs) & 0xFFFFu) == 0x8000u) | odd_lanes(p) | odd_lanes(hs);
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

// max(x, 0) with NaN passed through and -0 mapped to +0
__device__ __forceinline__ float relu_f(float x) { return x > 0.0f ? x : (x != x ? x : 0.0f); }

// Activations with a gate and an up input (the others read `gate` only).
template <int ACT>
constexpr bool gated() { return ACT == ACT_SWIGLU || ACT == ACT_CLAMPED; }

// 2 bits + this lane's bit of `mask`, in one instruction (an add with the
// mask as the carry in): shifting the flags of a row's elements in, last
// element first, leaves element k's flag in bit k.
__device__ __forceinline__ uint32_t shift_in(uint32_t bits, uint64_t mask) {
    uint32_t r;
    uint64_t carry_out;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(r), "=s"(carry_out) : "v"(bits), "s"(mask));
    return r;
}

// One element pair of the forward: packed gate / up words -> packed h word.
// m0 / m1: the lanes whose low / high element needs the exact path.
template <int ACT>
__device__ __forceinline__ void fwd_pair_r(uint32_t gw, uint32_t uw, float s, float L, uint32_t &hw, uint64_t &m0,
                                           uint64_t &m1) {
    if constexpr (ACT == ACT_IDENTITY) {
        hw = gw;
        m0 = m1 = 0ull;
    } else if constexpr (ACT == ACT_SRELU) {
        // a = bf16(v * v), v = max(x, 0): the square of a bf16 is exact in fp32
        // unless it leaves the normal range; h = bf16(a * s) as SwiGLU's product
        const float v0 = relu_f(lo_f(gw)), v1 = relu_f(hi_f(gw));
        const float t0 = v0 * v0, t1 = v1 * v1;
        const float a0 = bf16_round(t0), a1 = bf16_round(t1);
        const float h0 = a0 * s, h1 = a1 * s;
        hw = pack_bf16(h0, h1);
        (void)uw;
        (void)L;
        m0 = odd_lanes(t0) | product_risky(a0, h0);
        m1 = odd_lanes(t1) | product_risky(a1, h1);
    } else {
        float g0 = lo_f(gw), g1 = hi_f(gw), u0 = lo_f(uw), u1 = hi_f(uw);
        if constexpr (ACT == ACT_CLAMPED) {
            g0 = clamp_gate(g0, L); g1 = clamp_gate(g1, L);
            u0 = clamp_up(u0, L);   u1 = clamp_up(u1, L);
        }
        const Sig s0 = sig_fast(g0), s1 = sig_fast(g1);
        const float t0 = g0 * s0.sig, t1 = g1 * s1.sig;
        const float p0 = bf16_round(t0) * u0, p1 = bf16_round(t1) * u1;
        const float h0 = p0 * s, h1 = p1 * s;
        hw = pack_bf16(h0, h1);
        m0 = silu_risky(g0, t0) | product_risky(p0, h0);
        m1 = silu_risky(g1, t1) | product_risky(p1, h1);
    }
}

// The same, returning a 2-bit mask of the elements that need the exact path.
template <int ACT>
__device__ __forceinline__ uint32_t fwd_pair(uint32_t gw, uint32_t uw, float s, float L, uint32_t &hw) {
    uint64_t m0, m1;
    fwd_pair_r<ACT>(gw, uw, s, L, hw, m0, m1);
    return shift_in(shift_in(0u, m1), m0);
}

// h = bf16( bf16(silu(g)) * u * s ) in fp64 (the product is exact in fp64)
__device__ __forceinline__ uint32_t fwd_elem_f64(float g, float u, float s, float L, int act) {
    if (act == ACT_SRELU) {
        // h = bf16( bf16(max(x, 0)^2) * s ): the square and the product are exact in fp64
        const double v = (double)relu_f(g);
        const float a = __uint_as_float(bf16_from_f64(v * v) << 16);
        return bf16_from_f64((double)a * (double)s);
    }
    if (act == ACT_CLAMPED) {
        g = clamp_gate(g, L);
        u = clamp_up(u, L);
    }
    const double gd = (double)g;
    const float a = __uint_as_float(bf16_from_f64(gd * sigmoid_f64(gd)) << 16);
    return bf16_from_f64((double)a * (double)u * (double)s);
}

}  // namespace
}  // namespace mxq
