/*
 * mxq_oracle.c -- the plain, slow CPU oracle for the fused row-scaled SwiGLU +
 * MXFP8 path, the splits->offsets scan and the grouped GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header, table or constant generator
 * with the HIP library; the two meet only through the seeded input buffers.
 *
 * Every value is computed in IEEE double (fp64) with explicit rounding steps to
 * the destination formats, one element at a time, in the order the pages
 * describe: the activation first (with its bf16 roundings), then the standalone
 * block quantizer.  Build with -O2 -ffp-contract=off and no fast-math.
 *
 * Pages cited (the text of each page is the authority on what is computed):
 *   TAO4743 = "[mxfp8 training] Add a fused gated-activation (SwiGLU) + MXFP8
 *             quantization kernel" (pytorch/ao pull 4743)
 *   TE3238  = "Activation + GroupedLinear Fusion for MOE and other MOE
 *             optimizations" (NVIDIA/TransformerEngine pull 3238)
 *   TE3224  = NVIDIA/TransformerEngine pull 3224 (single grouped weight and the
 *             grouped GEMM backend)
 *   TE2600  = "[PyTorch] GroupedTensor integration" (NVIDIA/TransformerEngine
 *             pull 2600)
 *   VEO1340 = ByteDance-Seed/VeOmni pull 1340 (fused merged-FC1 SwiGLU forward)
 *
 * Readings the pages leave open are taken as follows (each one is also listed
 * with its reason in the design notes of the repository):
 *   - E4M3 is the OCP "fn" format (bias 7, no infinities, max 448, NaN = S.1111.111);
 *     E8M0 is the OCP scale byte 2^(E-127) with 0xFF = NaN.
 *   - RCEIL: the block scale exponent is the smallest integer e with
 *     amax <= 448 * 2^e, biased by 127 and clamped to [0, 254].
 *   - all-zero block: scale byte 0x00; a block holding NaN or Inf: scale byte 0xFF
 *     and every code 0x7F (parity of this case is not pinned by the pages).
 *   - no denormal flushing anywhere; the sign of zero is kept.
 *   - forward rounding: a = bf16(silu(g)), h = bf16(a * u * s) with one rounding.
 *   - clamped variant: g <- min(g, L), u <- clamp(u, -L, L), NaN passes through;
 *     gradients are masked strictly outside the range.
 *   - backward: dgate = bf16(dh*s*u*silu'(g)), dup = bf16(dh*s*a),
 *     dscale = fp32(sum_j dh*a*u); dact = quantize([dgate | dup]).
 *   - colwise blocks restart at each group's first row; a group's tail block is
 *     short; colwise scale rows are found through the block offsets.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>

#define EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------- */
/* O0: number formats                                                         */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> exact double.  bf16 is the top half of an IEEE binary32. */
EXPORT double oracle_bf16_to_double(uint16_t b)
{
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint16_t float_top_half(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/*
 * double -> bf16, round to nearest, ties to even.  bf16 keeps 8 significant
 * bits, binary exponents down to -126 for normals and a fixed quantum of
 * 2^-133 below that.  Values whose rounded magnitude reaches 2^128 become Inf.
 * NaN becomes the quiet NaN 0x7FC0 with its sign.
 */
EXPORT uint16_t oracle_double_to_bf16(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a)) return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);              /* a = f * 2^ex, f in [0.5, 1) => floor(log2 a) = ex - 1 */
    int e = ex - 1;
    if (e < -126) e = -126;     /* below the normal range the quantum is fixed */
    double q = ldexp(1.0, e - 7);
    double n = nearbyint(a / q); /* a/q is exact (power-of-two scaling); RNE */
    double r = n * q;
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80u);
    return (uint16_t)(sign | float_top_half((float)r)); /* r is exactly representable */
}

/* E4M3 ("fn") code -> exact double.  0x7F / 0xFF are NaN. */
EXPORT double oracle_e4m3_to_double(uint8_t c)
{
    int s = (c >> 7) & 1, e = (c >> 3) & 0xF, m = c & 7;
    double v;
    if (e == 0xF && m == 7) return s ? -NAN : NAN;
    if (e == 0) v = ldexp((double)m, -9);            /* subnormal: m * 2^-9 */
    else v = ldexp(1.0 + m / 8.0, e - 7);            /* normal: 1.m * 2^(e-7) */
    return s ? -v : v;
}

/*
 * double -> E4M3, round to nearest, ties to even, saturating at 448.
 * Normal exponents run from -6 to 8 with 3 mantissa bits; below 2^-6 the
 * quantum is fixed at 2^-9.  |y| >= 448 (Inf included) gives the max code.
 */
EXPORT uint8_t oracle_double_to_e4m3(double y)
{
    uint8_t sign = signbit(y) ? 0x80u : 0u;
    if (isnan(y)) return (uint8_t)(sign | 0x7Fu);
    double a = fabs(y);
    if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    if (e < -6) e = -6;
    double q = ldexp(1.0, e - 3);
    double n = nearbyint(a / q);
    double v = n * q;                                  /* rounded magnitude, <= 448 */
    if (v < ldexp(1.0, -6)) {
        /* subnormal (or zero): code = v / 2^-9, an integer 0..7 */
        return (uint8_t)(sign | (uint8_t)(v / ldexp(1.0, -9)));
    }
    frexp(v, &ex);
    e = ex - 1;                                         /* in [-6, 8] */
    int m = (int)((v / ldexp(1.0, e) - 1.0) * 8.0);     /* exact, 0..7 */
    return (uint8_t)(sign | (uint8_t)(((e + 7) << 3) | m));
}

/* E8M0 scale byte -> 2^(E-127) (NaN for 0xFF). */
EXPORT double oracle_e8m0_to_double(uint8_t e)
{
    if (e == 0xFF) return NAN;
    return ldexp(1.0, (int)e - 127);
}

/*
 * RCEIL scale byte of a block from its amax (TAO4743, Summary: "RCEIL MXFP8
 * cast"): the smallest integer e with amax <= 448 * 2^e, biased by 127 and
 * clamped to [0, 254].  NaN/Inf amax -> 0xFF; amax = 0 -> 0x00.
 */
EXPORT uint8_t oracle_e8m0_from_amax(double amax)
{
    if (isnan(amax) || isinf(amax)) return 0xFF;
    if (amax == 0.0) return 0x00;
    int e = (int)ceil(log2(amax / 448.0));
    /* settle the guess exactly; every comparison below is exact in fp64 */
    while (amax > ldexp(448.0, e)) e++;
    while (amax <= ldexp(448.0, e - 1)) e--;
    int E = e + 127;
    if (E < 0) E = 0;
    if (E > 254) E = 254;
    return (uint8_t)E;
}

/* ------------------------------------------------------------------------- */
/* O1: splits -> offsets (TE3238, Greptile Summary: offsets are computed once  */
/* up front from the split sizes instead of at every use site)               */
/* ------------------------------------------------------------------------- */

EXPORT void oracle_splits_to_offsets(const int64_t *splits, int64_t G,
                                     int64_t *row_off, int64_t *block_off)
{
    row_off[0] = 0;
    if (block_off) block_off[0] = 0;
    for (int64_t g = 0; g < G; g++) {
        row_off[g + 1] = row_off[g] + splits[g];
        if (block_off) block_off[g + 1] = block_off[g] + (splits[g] + 31) / 32;
    }
}

/* ------------------------------------------------------------------------- */
/* O3: the standalone MXFP8 block quantizer (TAO4743, Summary and Numerics and */
/* tests).  x is an (M x K) bf16 matrix with row stride ldx (elements).      */
/* Rowwise: one scale per 1x32 block of a row; codes (M x K), scales         */
/* (M x K/32).  Colwise: one scale per 32x1 block of a column inside a       */
/* group; codes (M x K) row-major, scales (sum_g ceil(m_g/32) x K).          */
/* row_off == NULL means one group of M rows.                                */
/* ------------------------------------------------------------------------- */

static uint8_t quantize_one(double x, uint8_t E)
{
    if (E == 0xFF) return 0x7F;
    /* y = x / 2^(E-127), exact in fp64 for every bf16 x and E in [0, 254] */
    return oracle_double_to_e4m3(x * ldexp(1.0, 127 - (int)E));
}

/* amax of a set of bf16 values: NaN if any is NaN (explicitly propagated). */
static double block_amax(const double *v, int n)
{
    double m = 0.0;
    for (int i = 0; i < n; i++) {
        if (isnan(v[i])) return NAN;
        double a = fabs(v[i]);
        if (a > m) m = a;
    }
    return m;
}

EXPORT void oracle_mx_quantize(int64_t M, int64_t K, const uint16_t *x, int64_t ldx,
                               int64_t G, const int64_t *row_off, uint32_t dirs,
                               uint8_t *row_codes, uint8_t *row_scales,
                               uint8_t *col_codes, uint8_t *col_scales)
{
    double v[32];
    if (dirs & 1u) {
        for (int64_t r = 0; r < M; r++) {
            for (int64_t b = 0; b < K / 32; b++) {
                for (int i = 0; i < 32; i++)
                    v[i] = oracle_bf16_to_double(x[r * ldx + b * 32 + i]);
                uint8_t E = oracle_e8m0_from_amax(block_amax(v, 32));
                row_scales[r * (K / 32) + b] = E;
                for (int i = 0; i < 32; i++)
                    row_codes[r * K + b * 32 + i] = quantize_one(v[i], E);
            }
        }
    }
    if (dirs & 2u) {
        int64_t one_group[2] = {0, M};
        const int64_t *ro = row_off ? row_off : one_group;
        int64_t ng = row_off ? G : 1;
        int64_t srow = 0; /* running colwise scale row = block offset */
        for (int64_t g = 0; g < ng; g++) {
            for (int64_t r0 = ro[g]; r0 < ro[g + 1]; r0 += 32, srow++) {
                int n = (int)((ro[g + 1] - r0) < 32 ? (ro[g + 1] - r0) : 32);
                for (int64_t c = 0; c < K; c++) {
                    for (int i = 0; i < n; i++)
                        v[i] = oracle_bf16_to_double(x[(r0 + i) * ldx + c]);
                    uint8_t E = oracle_e8m0_from_amax(block_amax(v, n));
                    col_scales[srow * K + c] = E;
                    for (int i = 0; i < n; i++)
                        col_codes[(r0 + i) * K + c] = quantize_one(v[i], E);
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Boundary closeness: is the exact value t within 2 binary32 ulps (of t) of a */
/* rounding tie of bf16?  Used to mark the elements where a correct fp32      */
/* evaluation may round the other way than the exact one.                     */
/* ------------------------------------------------------------------------- */

EXPORT int oracle_near_bf16_tie(double t)
{
    if (!isfinite(t) || t == 0.0) return 0;
    double a = fabs(t);
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    int eb = e < -126 ? -126 : e;
    double q = ldexp(1.0, eb - 7);          /* bf16 quantum at a */
    double lo = floor(a / q) * q;           /* bf16 neighbour below (exact) */
    double tie = lo + 0.5 * q;              /* the tie point between neighbours */
    int ef = e < -126 ? -126 : e;
    double ulp32 = ldexp(1.0, ef - 23);     /* binary32 ulp at a */
    return fabs(a - tie) <= 2.0 * ulp32;
}

/* ------------------------------------------------------------------------- */
/* O2: forward activation (TAO4743 Summary; VEO1340 "What does this PR do?":  */
/* SiLU is rounded to the activation dtype before the multiply; TE3238         */
/* Greptile Summary: per-row-scaled activation, SwiGLU and ClampedSwiGLU).     */
/* ------------------------------------------------------------------------- */

static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

/* kind 0 = SwiGLU, 1 = clamped SwiGLU with limit L. */
static void clamp_inputs(int kind, double L, double *g, double *u)
{
    if (kind != 1) return;
    if (*g > L) *g = L;                         /* NaN compares false: passes */
    if (*u > L) *u = L;
    else if (*u < -L) *u = -L;
}

/*
 * h = bf16( bf16(silu(g)) * u * s ) for every (r, j), j < K.  The product
 * a*u*s of an 8-, 8- and 24-bit significand is exact in fp64.
 * close (optional, M x K): bit0 = silu(g) is near a bf16 tie, bit1 = a*u*s is.
 */
EXPORT void oracle_swiglu_fwd(int kind, double limit, int64_t M, int64_t K,
                              const uint16_t *gate, int64_t ldg,
                              const uint16_t *up, int64_t ldu,
                              const float *scale, uint16_t *h, uint8_t *close)
{
    for (int64_t r = 0; r < M; r++) {
        double s = scale ? (double)scale[r] : 1.0;
        for (int64_t j = 0; j < K; j++) {
            double g = oracle_bf16_to_double(gate[r * ldg + j]);
            double u = oracle_bf16_to_double(up[r * ldu + j]);
            clamp_inputs(kind, limit, &g, &u);
            double t_silu = g * sigmoid(g);
            double a = oracle_bf16_to_double(oracle_double_to_bf16(t_silu));
            double t_h = a * u * s;
            h[r * K + j] = oracle_double_to_bf16(t_h);
            if (close)
                close[r * K + j] = (uint8_t)(oracle_near_bf16_tie(t_silu) | (oracle_near_bf16_tie(t_h) << 1));
        }
    }
}

/*
 * O4: backward (TAO4743 API: grad of the gated input is the packed
 * [dGate | dUp]; TE3238 Greptile Summary and Sequence Diagram: the scaled
 * activation backward also returns the gradient of the row scales).
 *
 *   silu'(g) = sigma(g) * (1 + g * (1 - sigma(g)))
 *   dgate    = bf16(dh * s * u * silu'(g) * m_g)
 *   dup      = bf16(dh * s * a * m_u),   a = bf16(silu(g))
 *   dscale_r = fp32( sum_j dh * a * u )  (summed in fp64)
 * With the clamped variant g, u are the clamped inputs, m_g = 0 where the
 * original g > L and m_u = 0 where |u| > L (both pass at equality).
 * dgate / dup are written with row strides lddg / lddu (may be NULL).
 * close (optional, M x 2K, laid out like [dgate | dup]): bit0 = the silu of g
 * is near a bf16 tie, bit1 = the pre-rounding value of that output is.
 * dscale_tol (optional, M): the tolerance for dscale (the pages give none):
 * 64 * 2^-24 * sum_j |dh*a*u| -- the error bound of an fp32 summation in which
 * no term passes through more than 63 additions, plus the final rounding --
 * + sum over the columns where silu(g) is near a bf16 tie of
 * |dh*u| * ulp_bf16(a) (a correct fp32 evaluation may round a the other way
 * there).
 */
EXPORT void oracle_swiglu_bwd(int kind, double limit, int64_t M, int64_t K,
                              const uint16_t *grad, int64_t ldgr,
                              const uint16_t *gate, int64_t ldg,
                              const uint16_t *up, int64_t ldu,
                              const float *scale,
                              uint16_t *dgate, int64_t lddg,
                              uint16_t *dup, int64_t lddu,
                              float *dscale, uint8_t *close, double *dscale_tol)
{
    for (int64_t r = 0; r < M; r++) {
        double s = scale ? (double)scale[r] : 1.0;
        double acc = 0.0, acc_abs = 0.0, flip = 0.0;
        for (int64_t j = 0; j < K; j++) {
            double dh = oracle_bf16_to_double(grad[r * ldgr + j]);
            double g0 = oracle_bf16_to_double(gate[r * ldg + j]);
            double u0 = oracle_bf16_to_double(up[r * ldu + j]);
            double g = g0, u = u0;
            clamp_inputs(kind, limit, &g, &u);
            double mg = 1.0, mu = 1.0;
            if (kind == 1) {
                if (g0 > limit) mg = 0.0;
                if (u0 > limit || u0 < -limit) mu = 0.0;
            }
            double sg = sigmoid(g);
            double t_silu = g * sg;
            double a = oracle_bf16_to_double(oracle_double_to_bf16(t_silu));
            double dsilu = sg * (1.0 + g * (1.0 - sg));
            double t_dg = dh * s * u * dsilu * mg;
            double t_du = dh * s * a * mu;
            if (dgate) dgate[r * lddg + j] = oracle_double_to_bf16(t_dg);
            if (dup) dup[r * lddu + j] = oracle_double_to_bf16(t_du);
            double term = dh * a * u;
            acc += term;
            acc_abs += fabs(term);
            int ca = oracle_near_bf16_tie(t_silu);
            if (ca) {
                int ex;
                frexp(fabs(a) > 0 ? fabs(a) : 1e-300, &ex);
                int eb = (ex - 1) < -126 ? -126 : (ex - 1);
                flip += fabs(dh * u) * ldexp(1.0, eb - 7);
            }
            if (close) {
                close[r * 2 * K + j] = (uint8_t)(ca | (oracle_near_bf16_tie(t_dg) << 1));
                close[r * 2 * K + K + j] = (uint8_t)(ca | (oracle_near_bf16_tie(t_du) << 1));
            }
        }
        if (dscale) dscale[r] = (float)acc;
        /* an fp32 summation in which no term passes through more than 63
           additions is within 63 * 2^-24 * sum|t| of the exact sum, and the
           exact sum's own rounding to fp32 adds at most 2^-24 * sum|t| */
        if (dscale_tol) dscale_tol[r] = ldexp(64.0, -24) * acc_abs + flip;
    }
}

/* ------------------------------------------------------------------------- */
/* O2' / O4': the row-scaled SReLU (TE3238, Greptile Summary: the per-row-    */
/* scaled activations are SReLU, SwiGLU and ClampedSwiGLU; SReLU is unary).   */
/* The pages print no formula.  Reading: SReLU is the squared ReLU, and its   */
/* value is rounded to bf16 before the row scale multiplies it, as SwiGLU's   */
/* activation is (VEO1340: the activation is rounded to its dtype first).     */
/*   forward:  a = bf16(max(x, 0)^2),  h = bf16(a * s)                        */
/*   backward: dx = bf16(dh * s * 2 * max(x, 0)),  dscale = fp32(sum_j dh*a)  */
/* max(x, 0) passes NaN and maps -0 and negative values (-Inf included) to   */
/* +0; every product below is exact in fp64 (at most 8+8+24+1 significant    */
/* bits), so each output is one rounding of the exact value.                  */
/* ------------------------------------------------------------------------- */

static double relu(double x) { return isnan(x) ? x : (x > 0.0 ? x : 0.0); }

/* close (optional, M x K): bit0 = max(x,0)^2 is near a bf16 tie, bit1 = a*s is. */
EXPORT void oracle_srelu_fwd(int64_t M, int64_t K, const uint16_t *x, int64_t ldx,
                             const float *scale, uint16_t *h, uint8_t *close)
{
    for (int64_t r = 0; r < M; r++) {
        double s = scale ? (double)scale[r] : 1.0;
        for (int64_t j = 0; j < K; j++) {
            double v = relu(oracle_bf16_to_double(x[r * ldx + j]));
            double t_a = v * v;
            double a = oracle_bf16_to_double(oracle_double_to_bf16(t_a));
            double t_h = a * s;
            h[r * K + j] = oracle_double_to_bf16(t_h);
            if (close)
                close[r * K + j] = (uint8_t)(oracle_near_bf16_tie(t_a) | (oracle_near_bf16_tie(t_h) << 1));
        }
    }
}

/* dx written with row stride lddx; close (optional, M x K): bit1 = the exact
 * dx is near a bf16 tie; dscale_tol (optional, M): 64 * 2^-24 * sum|dh*a| (a
 * is computed exactly on every path, so no term for a rounding the other way). */
EXPORT void oracle_srelu_bwd(int64_t M, int64_t K, const uint16_t *grad, int64_t ldgr,
                             const uint16_t *x, int64_t ldx, const float *scale,
                             uint16_t *dx, int64_t lddx, float *dscale, uint8_t *close,
                             double *dscale_tol)
{
    for (int64_t r = 0; r < M; r++) {
        double s = scale ? (double)scale[r] : 1.0;
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t j = 0; j < K; j++) {
            double dh = oracle_bf16_to_double(grad[r * ldgr + j]);
            double v = relu(oracle_bf16_to_double(x[r * ldx + j]));
            double a = oracle_bf16_to_double(oracle_double_to_bf16(v * v));
            double t_dx = dh * s * 2.0 * v;
            if (dx) dx[r * lddx + j] = oracle_double_to_bf16(t_dx);
            double term = dh * a;
            acc += term;
            acc_abs += fabs(term);
            if (close) close[r * K + j] = (uint8_t)(oracle_near_bf16_tie(t_dx) << 1);
        }
        if (dscale) dscale[r] = (float)acc;
        if (dscale_tol) dscale_tol[r] = ldexp(64.0, -24) * acc_abs;
    }
}

/* ------------------------------------------------------------------------- */
/* O5: grouped GEMM (TE3224 and TE2600: one grouped GEMM over per-expert      */
/* groups of rows; TE3238 Sequence Diagram: FC1 forward, dgrad and wgrad).     */
/* Operands are dequantized exactly (code * 2^(E-127), or the bf16 value);     */
/* products are exact in fp32 and are accumulated in fp32 in natural order.    */
/* ------------------------------------------------------------------------- */

/*
 * One operand.  dtype 0 = bf16 (data is uint16), 1 = MXFP8 E4M3 (data is
 * uint8 codes + uint8 E8M0 scales).  Element (i, k) of group g lives at
 *   data[g * gstride + i * ld_i + k * ld_k]
 * and its scale (MXFP8 only) at
 *   scales[g * sgstride + sblock(k) * sld_k + i * sld_i]
 * where sblock(k) is the scale block of the contraction index:
 *   k / 32 for operands blocked along k from index 0, or
 *   block_off[g] + (k - row_off[g]) / 32 for the K-grouped operands, whose
 *   contraction index is a global row r inside group g.
 */
typedef struct {
    int dtype;
    const void *data;
    int64_t gstride, ld_i, ld_k;
    const uint8_t *scales;
    int64_t sgstride, sld_i, sld_k;
} oracle_operand;

static double operand_value(const oracle_operand *op, int64_t g, int64_t i, int64_t k,
                            int64_t sblock)
{
    int64_t idx = g * op->gstride + i * op->ld_i + k * op->ld_k;
    if (op->dtype == 0) return oracle_bf16_to_double(((const uint16_t *)op->data)[idx]);
    uint8_t c = ((const uint8_t *)op->data)[idx];
    uint8_t E = op->scales[g * op->sgstride + sblock * op->sld_k + i * op->sld_i];
    return oracle_e4m3_to_double(c) * oracle_e8m0_to_double(E);
}

static void store_out(void *out, int out_dtype, int64_t idx, float v, int accumulate)
{
    if (out_dtype == 1) {
        float *o = (float *)out;
        o[idx] = accumulate ? (float)((double)o[idx] + (double)v) : v;
    } else {
        uint16_t *o = (uint16_t *)out;
        double base = accumulate ? oracle_bf16_to_double(o[idx]) : 0.0;
        o[idx] = oracle_double_to_bf16(base + (double)v);
    }
}

/*
 * mode 0 (M-grouped): for each group g and row r in [row_off[g], row_off[g+1]):
 *     C[r, n] = sum_{k<Kdim} A(0, r, k) * B(g, n, k)       (n < N)
 *   A's element (i=r, k); B's element (i=n, k) of group g.  out row stride ldc.
 * mode 1 (K-grouped): for each group g:
 *     C_g[m, n] = sum_{r in group g} A(0, m, r) * B(0, n, r)  (m < Mdim, n < N)
 *   written at out[g * out_gstride + m * ldc + n]; an empty group writes zeros
 *   (or leaves the output untouched with accumulate).
 * out_dtype 0 = bf16 (RNE), 1 = fp32.  accumulate adds into the output.
 */
EXPORT void oracle_grouped_gemm(int mode, int64_t G, const int64_t *row_off,
                                int64_t Mdim, int64_t N, int64_t Kdim,
                                const oracle_operand *A, const oracle_operand *B,
                                void *out, int out_dtype, int64_t ldc, int64_t out_gstride,
                                int accumulate)
{
    if (mode == 0) {
        for (int64_t g = 0; g < G; g++) {
            for (int64_t r = row_off[g]; r < row_off[g + 1]; r++) {
                for (int64_t n = 0; n < N; n++) {
                    float acc = 0.0f;
                    for (int64_t k = 0; k < Kdim; k++) {
                        double a = operand_value(A, 0, r, k, k / 32);
                        double b = operand_value(B, g, n, k, k / 32);
                        acc = (float)((double)acc + (double)(float)(a * b));
                    }
                    store_out(out, out_dtype, r * ldc + n, acc, accumulate);
                }
            }
        }
    } else {
        int64_t boff = 0;
        for (int64_t g = 0; g < G; g++) {
            int64_t r0 = row_off[g], r1 = row_off[g + 1];
            for (int64_t m = 0; m < Mdim; m++) {
                for (int64_t n = 0; n < N; n++) {
                    float acc = 0.0f;
                    for (int64_t r = r0; r < r1; r++) {
                        int64_t sb = boff + (r - r0) / 32;
                        double a = operand_value(A, 0, m, r, sb);
                        double b = operand_value(B, 0, n, r, sb);
                        acc = (float)((double)acc + (double)(float)(a * b));
                    }
                    int64_t idx = g * out_gstride + m * ldc + n;
                    if (r1 > r0) store_out(out, out_dtype, idx, acc, accumulate);
                    else if (!accumulate) store_out(out, out_dtype, idx, 0.0f, 0);
                }
            }
            boff += (r1 - r0 + 31) / 32;
        }
    }
}
