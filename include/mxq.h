/*
 * mxq.h -- C ABI of libmxq, the MI355X (gfx950) library for the MoE expert-MLP
 * activation path: per-row-scaled SwiGLU fused with MXFP8 block quantization
 * (forward and backward), the splits->offsets scan, a plain MXFP8 quantizer
 * and the grouped GEMM over experts that consumes the quantized tensors.
 *
 * Pages cited (their text defines what each call computes):
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
 * Conventions shared by every entry point
 *   - Every data pointer is DEVICE memory owned by the caller.  The library
 *     never allocates or frees memory; scratch space is a caller-provided
 *     workspace whose size a *_workspace query returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     null stream).  No call synchronizes or reads device memory on the host,
 *     so every call can be captured into a HIP graph.
 *   - Sizes and leading dimensions are int64 and counted in ELEMENTS.
 *   - bf16 values are passed as uint16_t bit patterns; E4M3 codes and E8M0
 *     scale bytes as uint8_t.
 *   - Errors are returned as an mxq_status; nothing is launched when a call
 *     fails validation.  mxq_last_error_message() returns a thread-local text
 *     describing the last failure on the calling thread.
 *   - Inputs are never written (VEO1340, Design & Code Changes: no input
 *     mutation); an output range that overlaps an input range is rejected.
 *   - Thread-safe: the library holds no mutable global state except the
 *     thread-local error text, and the per-GPU scratch of the one
 *     allocation-free entry point (mxq_swiglu_quantize_bwd_noalloc), whose
 *     calls on one GPU the caller must not overlap.
 *
 * Number formats (TAO4743, Summary and Numerics and tests)
 *   - E4M3 is the OCP FP8 "fn" format: bias 7, max finite 448, no infinities,
 *     NaN = 0x7F / 0xFF.  Codes are round-to-nearest-even and saturate at 448.
 *   - E8M0 scale byte E stands for 2^(E-127); 0xFF is NaN.
 *   - RCEIL: a block's scale byte is the smallest e with amax <= 448 * 2^e,
 *     biased by 127 and clamped to [0, 254]; amax = 0 gives 0x00; a block
 *     holding a NaN or an Inf gets scale 0xFF and every code in it 0x7F.
 *     Codes are e4m3(x * 2^(127-E)).  Denormals are never flushed and the sign
 *     of zero is kept.
 *   - Rowwise blocks are 1x32 (32 consecutive columns of a row); colwise
 *     blocks are 32x1 (up to 32 consecutive rows of a column inside one group,
 *     restarting at each group's first row; a group's last block may be
 *     short).  In both directions the codes are stored (rows x cols)
 *     row-major.  Rowwise scales are (rows x cols/32) row-major; colwise scales
 *     are (sum_g ceil(m_g/32) x cols) row-major, the scale row of block b of
 *     group g being block_off[g] + b.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ----------------------------------------------------------------- status */

typedef enum {
    MXQ_OK = 0,
    MXQ_ERR_NULL = 1,        /* a required pointer is NULL, or an enabled output is missing */
    MXQ_ERR_SHAPE = 2,       /* negative size, K % 32 != 0, ld too small, bad dirs/mode/G ... */
    MXQ_ERR_ALIGN = 3,       /* a bf16/code pointer or row pitch is not 16-byte aligned, ... */
    MXQ_ERR_OVERFLOW = 4,    /* an extent exceeds the library's 62-bit / 31-bit index bounds */
    MXQ_ERR_ALIAS = 5,       /* an output overlaps an input */
    MXQ_ERR_UNSUPPORTED = 6, /* a dtype / layout / mode combination that is not built */
    MXQ_ERR_HIP = 7,         /* the HIP runtime reported an error at launch */
    MXQ_ERR_WORKSPACE = 8    /* the workspace is NULL or smaller than the query returned */
} mxq_status;

/* Directions of an MXFP8 output. */
#define MXQ_ROWWISE 1u /* 1x32 blocks */
#define MXQ_COLWISE 2u /* 32x1 blocks */

/* ------------------------------------------------------------ descriptors */

/* Row-scaled activation (TE3238, Greptile Summary: the scaled activations are
 * SReLU, SwiGLU and ClampedSwiGLU).
 * MXQ_ACT_SWIGLU:          a = bf16(silu(g)),  h = bf16(a * u * s)
 * MXQ_ACT_CLAMPED_SWIGLU:  the same on g' = min(g, limit), u' = clamp(u, -limit,
 *                          limit) (NaN passes through); limit is typically 7.
 * MXQ_ACT_SRELU:           unary: a = bf16(max(x, 0)^2),  h = bf16(a * s); the
 *                          pages give no formula, this is the squared ReLU
 *                          with the activation rounded before the row scale
 *                          as for SwiGLU.  x is passed as `gate`; `up` (and
 *                          in the backward `dup`) must be NULL.
 * glu_interleave (SwiGLU kinds only): 0 for gate and up as given; B > 0 (a
 * multiple of 32 dividing K) when the gated input holds gate and up
 * interleaved in blocks of B columns (TE3238, Important Files Changed: the GLU
 * interleave is handled inside the scaled SwiGLU kernels): logical column j
 * of gate sits at column 2B*(j/B) + j%B of the `gate` view, and likewise for
 * `up`, so a packed interleaved buffer p of ld 2K is passed as gate = p,
 * up = p + B.  The backward then writes [dgate | dup] in the same layout (dup
 * = dgate + B) and its MXFP8 form too (dup's columns B on from dgate's).  B =
 * K is the plain packed [gate | up]. */
typedef enum { MXQ_ACT_SWIGLU = 0, MXQ_ACT_CLAMPED_SWIGLU = 1, MXQ_ACT_SRELU = 2 } mxq_act_kind;

typedef struct {
    int32_t kind;            /* mxq_act_kind */
    float limit;             /* clamp limit for MXQ_ACT_CLAMPED_SWIGLU, > 0 */
    int32_t glu_interleave;  /* 0, or the interleave block B (see above) */
} mxq_act;

/* Row groups (experts).  Both arrays are DEVICE int64[G+1], as written by
 * mxq_splits_to_offsets: row_off[g] is the first row of group g and
 * row_off[G] must equal the number of rows M; block_off[g] is the first
 * colwise scale row of group g (the prefix sum of ceil(split/32)).
 * Rows outside [0, M) are never touched, whatever the arrays hold. */
typedef struct {
    int64_t G;
    const int64_t *row_off;
    const int64_t *block_off;
} mxq_groups;

/* One direction of an MXFP8 output: codes (rows x cols, row pitch ld_codes
 * bytes) and scales (row pitch ld_scales bytes).  Rowwise codes may instead
 * be K-blocked by 64 for the grouped GEMM (kblock_plane = P > 0: code (r, c)
 * at byte (c / 64) * P + r * 64 + c % 64; ld_codes must be 64, cols a
 * multiple of 64, P a multiple of 16 and at least 64 * rows, and the codes
 * must span less than 2^31 bytes, else MXQ_ERR_SHAPE / _ALIGN / _OVERFLOW);
 * colwise codes are always row-major (MXQ_ERR_UNSUPPORTED otherwise), and the
 * fused FC1 epilogue writes row-major codes only. */
typedef struct {
    uint8_t *codes;
    int64_t ld_codes;
    uint8_t *scales;
    int64_t ld_scales;
    int64_t kblock_plane;   /* 0: row-major codes; P > 0: K-blocked (rowwise only) */
} mxq_mx_out;

/* ------------------------------------------------------------ entry points */

/*
 * Splits -> offsets (TE3238, Greptile Summary and Sequence Diagram: every
 * per-group offset array is computed once, up front, from the split sizes).
 *   splits    device int64[G], the row count of each group (expert)
 *   row_off   device int64[G+1] out: row_off[0] = 0, row_off[g+1] = row_off[g] + splits[g]
 *   block_off device int64[G+1] out or NULL: the same prefix sum of ceil(splits[g]/32),
 *             i.e. the first colwise scale row of each group
 *   err_flag  device int32 or NULL: set to 1 if any split is negative (the
 *             prefix sums are still written); never cleared by the call
 * G >= 1, G <= 2^20.  One workgroup; exact integer arithmetic.
 */
mxq_status mxq_splits_to_offsets(const int64_t *splits, int64_t G, int64_t *row_off,
                                 int64_t *block_off, int32_t *err_flag, void *stream);

/*
 * Fused row-scaled SwiGLU + MXFP8 forward (TAO4743, Summary and API; TE3238,
 * Greptile Summary; VEO1340, "What does this PR do?").
 * For every row r < M and column j < K:
 *     a = bf16(silu(g[r,j])),  h = bf16(a * u[r,j] * s[r])
 * and h is block-quantized rowwise and/or colwise without ever being stored.
 *   gate, up    device bf16 (M x K) with row pitches ld_gate, ld_up (elements);
 *               the packed [gate | up] (M x 2K) layout is gate = p, up = p + K,
 *               ld = 2K
 *   row_scale   device fp32[M], or NULL for s = 1
 *   groups      NULL for one group of M rows; otherwise colwise blocks
 *               restart at every group (rowwise output ignores groups)
 *   dirs        MXQ_ROWWISE, MXQ_COLWISE or both
 *   row_out     required iff dirs has MXQ_ROWWISE: codes (M x K), scales (M x K/32)
 *   col_out     required iff dirs has MXQ_COLWISE: codes (M x K), scales
 *               (n_blocks x K) with n_blocks = ceil(M/32) for one group, else
 *               sum_g ceil(m_g/32)
 * K % 32 == 0; M == 0 is a successful no-op.  Pointers to bf16 data and codes
 * and the row pitches in bytes must be multiples of 16.
 */
mxq_status mxq_swiglu_quantize_fwd(const mxq_act *act, int64_t M, int64_t K,
                                   const uint16_t *gate, int64_t ld_gate,
                                   const uint16_t *up, int64_t ld_up,
                                   const float *row_scale, const mxq_groups *groups,
                                   uint32_t dirs, const mxq_mx_out *row_out,
                                   const mxq_mx_out *col_out, void *stream);

/*
 * The activation as dense bf16, with or without its MXFP8 forms from the same
 * pass (TAO4743, Performance: the BF16-wgrad recipe recomputes the activation
 * in bf16 at the autograd boundary for the two wgrad GEMMs, while the kernel
 * emits rowwise-only casts).  The same computation, arguments, rules and
 * MXFP8 outputs as mxq_swiglu_quantize_fwd (every activation kind and the
 * GLU interleave included), plus:
 *   h      device bf16 (M x K) output, row pitch ld_h (elements; pointer and
 *          pitch in bytes multiples of 16), in logical column order (not
 *          interleaved); required unless M or K is 0
 *   dirs   0 for the dense activation alone (row_out and col_out unused), or
 *          ROWWISE, COLWISE or both as for mxq_swiglu_quantize_fwd
 * h holds exactly the values the MXFP8 outputs quantize.  h may not overlap
 * an input or another output (MXQ_ERR_ALIAS).
 */
mxq_status mxq_swiglu_fwd_bf16(const mxq_act *act, int64_t M, int64_t K,
                               const uint16_t *gate, int64_t ld_gate,
                               const uint16_t *up, int64_t ld_up,
                               const float *row_scale, const mxq_groups *groups,
                               uint32_t dirs, const mxq_mx_out *row_out,
                               const mxq_mx_out *col_out, uint16_t *h, int64_t ld_h,
                               void *stream);

/*
 * Workspace bytes for mxq_swiglu_quantize_bwd at (M, K): the per-row partial
 * sums of dscale (0 if dscale is not requested, but the query always reports
 * the size needed with dscale).
 */
mxq_status mxq_swiglu_quantize_bwd_workspace(int64_t M, int64_t K, uint32_t dirs,
                                             size_t *bytes);

/*
 * Fused backward of the row-scaled SwiGLU with MXFP8 quantization of the
 * gradient of the gated input (TAO4743, API: the backward returns the packed
 * [dGate | dUp]; TE3238, Greptile Summary and Sequence Diagram: the scaled
 * activation backward returns the quantized dy, the dense dy and the gradient
 * of the scales, which may be requested on its own).
 * With dh = grad[r,j], sigma = sigmoid(g), a = bf16(silu(g)):
 *     dgate = bf16(dh * s * u * sigma * (1 + g * (1 - sigma)))
 *     dup   = bf16(dh * s * a)
 *     dscale[r] = sum_j dh * a * u            (fp32, deterministic order)
 * (clamped variant: g, u clamped as in the forward; dgate is 0 where g > limit,
 * dup is 0 where |u| > limit).  The MXFP8 outputs quantize the (M x 2K)
 * matrix [dgate | dup]: row_out codes (M x 2K) + scales (M x 2K/32); col_out
 * codes (M x 2K) + scales (n_blocks x 2K).  With act->glu_interleave = B the
 * dense and MXFP8 gradients are interleaved like the input (dup = dgate + B).
 * MXQ_ACT_SRELU (unary, x passed as gate, up = dup = NULL):
 *     dx = bf16(dh * s * 2 * max(x, 0)) written through dgate,
 *     dscale[r] = sum_j dh * bf16(max(x, 0)^2),
 * and the MXFP8 outputs quantize the (M x K) matrix dx.
 *   dgate, dup  device bf16 (M x K) outputs with pitches ld_dgate, ld_dup, or
 *               both NULL to skip the dense gradients
 *   dscale      device fp32[M] output, or NULL; needs row_scale semantics only
 *               through a and u, so it is valid with row_scale == NULL too
 *   dirs        0 (only if a dense output or dscale is requested), ROWWISE,
 *               COLWISE or both
 *   ws          device workspace of at least mxq_swiglu_quantize_bwd_workspace
 *               bytes when dscale != NULL (NULL otherwise)
 */
mxq_status mxq_swiglu_quantize_bwd(const mxq_act *act, int64_t M, int64_t K,
                                   const uint16_t *grad, int64_t ld_grad,
                                   const uint16_t *gate, int64_t ld_gate,
                                   const uint16_t *up, int64_t ld_up,
                                   const float *row_scale, const mxq_groups *groups,
                                   uint16_t *dgate, int64_t ld_dgate,
                                   uint16_t *dup, int64_t ld_dup, float *dscale,
                                   uint32_t dirs, const mxq_mx_out *row_out,
                                   const mxq_mx_out *col_out, void *ws, size_t ws_bytes,
                                   void *stream);

/*
 * mxq_swiglu_quantize_bwd for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation, arguments and results, with no workspace argument.  The
 * dscale partial sums go to a scratch array built into the library, 16 MiB
 * per GPU (held until the process ends), which covers every call whose
 * mxq_swiglu_quantize_bwd_workspace is at most 16 MiB (one fp32 per row and
 * column slab of 512, or of 256 when K mod 512 is in (0, 256]; e.g. M = 131072
 * at K = 8192, M = 1,398,101 at K = 768); a larger call with dscale != NULL
 * returns MXQ_ERR_WORKSPACE before touching the device.  Every call on one
 * GPU shares that GPU's scratch: calls that overlap on one GPU (two streams,
 * two threads) race on it and must be ordered by the caller.  The stream must
 * belong to the calling thread's current device.  Nothing is allocated or
 * freed.
 */
mxq_status mxq_swiglu_quantize_bwd_noalloc(const mxq_act *act, int64_t M, int64_t K,
                                           const uint16_t *grad, int64_t ld_grad,
                                           const uint16_t *gate, int64_t ld_gate,
                                           const uint16_t *up, int64_t ld_up,
                                           const float *row_scale, const mxq_groups *groups,
                                           uint16_t *dgate, int64_t ld_dgate,
                                           uint16_t *dup, int64_t ld_dup, float *dscale,
                                           uint32_t dirs, const mxq_mx_out *row_out,
                                           const mxq_mx_out *col_out, void *stream);

/*
 * Plain MXFP8 block quantization of a bf16 (M x K) matrix (TAO4743, Summary:
 * the standalone quantizers the fused kernel is bit-compatible with;
 * TE3224, Greptile Summary: grouped quantization of the expert weights).
 * Same output layouts and rules as mxq_swiglu_quantize_fwd, with h = x.
 */
mxq_status mxq_quantize(int64_t M, int64_t K, const uint16_t *x, int64_t ld_x,
                        const mxq_groups *groups, uint32_t dirs,
                        const mxq_mx_out *row_out, const mxq_mx_out *col_out,
                        void *stream);

/*
 * Graph-safe quantization into reused outputs (TE3224, Greptile Summary: the
 * grouped quantization of the expert weights fills a cached output in place
 * and takes a no-op flag, so that a captured weight quantization can be
 * replayed with unchanged pointers; TE2600, review discussion: an optional
 * no-op tensor for graph capture).  The same computation and layouts as
 * mxq_quantize, into the caller-owned outputs given, except that when
 * noop_flag is non-NULL and the device int32 it points to is non-zero when the
 * kernel runs, the call writes nothing and leaves every output as it was (the
 * flag is read on the device, so the host never synchronizes and a graph that
 * holds the call replays correctly whatever the flag holds at replay time).
 *   noop_flag  device int32, 4-byte aligned, or NULL (then as mxq_quantize);
 *              an input: no output may overlap it
 */
mxq_status mxq_quantize_noop(int64_t M, int64_t K, const uint16_t *x, int64_t ld_x,
                             const mxq_groups *groups, uint32_t dirs,
                             const mxq_mx_out *row_out, const mxq_mx_out *col_out,
                             const int32_t *noop_flag, void *stream);

/* ------------------------------------------------------------ grouped GEMM */

typedef enum { MXQ_DTYPE_BF16 = 0, MXQ_DTYPE_MXFP8_E4M3 = 1, MXQ_DTYPE_F32 = 2 } mxq_dtype;

/* Grouped GEMM modes (TE3224 and TE2600: one grouped GEMM over the experts'
 * row groups; TE3238, Sequence Diagram: forward, dgrad and wgrad).
 *
 * MXQ_GEMM_NT  (M-grouped, B contiguous along the contraction; FC1 / FC2 forward)
 *     for each group g, row r in group g, n < N:  C[r,n] = sum_{k<K} A[r,k] * B_g[n,k]
 *     A (M x K) row-major, ld_a; B per group (N x K) row-major, ld_b, group
 *     stride b_gstride.  MXFP8: A rowwise scales (M x K/32), B rowwise scales
 *     (N x K/32) per group.
 * MXQ_GEMM_NN  (M-grouped, B strided along the contraction; dgrad)
 *     C[r,n] = sum_k A[r,k] * B_g[k,n]
 *     B per group (K x N) row-major.  MXFP8: B colwise scales (K/32 x N) per
 *     group (its 32x1 blocks run along k).
 * MXQ_GEMM_TN  (K-grouped, contraction over each group's rows; wgrad)
 *     C_g[m,n] = sum_{r in group g} A[r,m] * B[r,n]   (m < M, n < N)
 *     A (rows x M), B (rows x N) row-major.  MXFP8: both colwise-quantized with
 *     per-group 32-row blocks (scales (n_blocks x M) and (n_blocks x N),
 *     rows located through block_off).  An empty group writes zeros (or, with
 *     accumulate, leaves C_g untouched).
 * For NT/NN, "M" is the total row count (= row_off[G]); for TN it is the
 * output row count, and the total row count is rows.
 * Every mode takes bf16 or MXFP8 operands (both the same); bf16 TN is the
 * wgrad of the BF16-wgrad recipe (TAO4743, Performance: the recipe with the
 * activation recomputed in bf16 for the two wgrad GEMMs) and needs no
 * block_off.
 * Every product is accumulated in fp32 and rounded once to the output dtype.
 *
 * K-blocked operands (an operand read along the contraction: A of NT and
 * NN, B of NT; MXFP8 codes or bf16).  With kblock_plane = P > 0 the operand
 * is stored in planes of 64 contraction bytes (e = 64 codes or 32 bf16 per
 * plane row): element (r, k) of row r lies at byte
 * (k / e) * P + r * 64 + (k % e) * element size of data (for B of NT,
 * r = g * gstride / e + n: gstride, in elements, is the distance of group
 * g's rows within a plane).  ld must then be e, K a multiple of e, P a
 * multiple of 16 and at least the rows' extent within a plane (else
 * MXQ_ERR_SHAPE / _ALIGN; MXQ_ERR_UNSUPPORTED for B of NN and for TN).  The
 * values and results are those of the row-major layout; what changes is that
 * a 64-byte stage of 16 rows is one contiguous kilobyte, so every load of the
 * GEMM covers whole cache lines.  The fused activation kernels and the
 * quantizer write their rowwise codes in this layout when their mxq_mx_out
 * asks for it (mxq_mx_out.kblock_plane).  Scales keep their row-major layout.
 */
typedef enum { MXQ_GEMM_NT = 0, MXQ_GEMM_NN = 1, MXQ_GEMM_TN = 2 } mxq_gemm_mode;

typedef struct {
    int32_t dtype;          /* MXQ_DTYPE_BF16 or MXQ_DTYPE_MXFP8_E4M3 */
    const void *data;       /* bf16 bits or E4M3 codes */
    int64_t ld;             /* row pitch, elements */
    int64_t gstride;        /* group stride, elements (B of NT/NN only) */
    const uint8_t *scales;  /* E8M0 bytes (MXFP8 only) */
    int64_t ld_scales;      /* scale row pitch, bytes */
    int64_t scale_gstride;  /* scale group stride, bytes (B of NT/NN only) */
    int64_t kblock_plane;   /* 0: row-major; P > 0: K-blocked, plane stride P
                               bytes (see above) */
} mxq_operand;

typedef struct {
    int32_t mode;           /* mxq_gemm_mode */
    int64_t G;              /* groups, >= 1 */
    const int64_t *row_off; /* device int64[G+1] */
    const int64_t *block_off; /* device int64[G+1]; required for MXFP8 TN */
    int64_t M, N, K;        /* see the modes; K unused for TN */
    int64_t rows;           /* total rows (TN only; must equal row_off[G]) */
    mxq_operand A, B;
    int32_t out_dtype;      /* MXQ_DTYPE_BF16 or MXQ_DTYPE_F32 */
    void *out;              /* device output */
    int64_t ld_out;         /* output row pitch, elements */
    int64_t out_gstride;    /* output group stride, elements (TN only) */
    int32_t accumulate;     /* 1: C += result (TN with F32 output only) */
    int32_t max_workgroups; /* 0: one workgroup per CU; n > 0: at most n (rounded
                               down to a multiple of 8, at least 8), e.g. to leave
                               CUs to work overlapping on another stream */
} mxq_gemm_args;

/* Workspace bytes for mxq_grouped_gemm with these arguments (pointers unused):
 * 256 for MXQ_GEMM_TN, 0 otherwise. */
mxq_status mxq_grouped_gemm_workspace(const mxq_gemm_args *args, size_t *bytes);

/* Run the grouped GEMM.  Group sizes are read on the device only; the grid is
 * sized from M (NT/NN) or from G and the output size (TN), never from a
 * host copy of the offsets.
 *   ws  device workspace of at least mxq_grouped_gemm_workspace bytes, 4-byte
 *       aligned (NULL allowed when that is 0), owned by the caller; its
 *       contents need no initialisation and are overwritten.  MXQ_GEMM_TN
 *       keeps a counter there: with skewed group sizes the tiles are handed
 *       out largest group first to whichever workgroup finishes first, which
 *       balances the work (the result does not depend on the order).  Two
 *       calls in flight at once must not share a workspace.
 * Errors: MXQ_ERR_WORKSPACE if ws is NULL or smaller than needed,
 * MXQ_ERR_ALIGN if it is not 4-byte aligned. */
mxq_status mxq_grouped_gemm(const mxq_gemm_args *args, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * FC1 grouped GEMM with the row-scaled SwiGLU and its MXFP8 quantization in
 * the epilogue (TE3238, discussion: the activation plus its grouped
 * quantization fused with the grouped linear, the FC1 - activation - FC2
 * module; TAO4743, Summary: the bf16 activation is never stored).  A bf16 NT
 * grouped GEMM as mxq_grouped_gemm (args->mode = MXQ_GEMM_NT, bf16 operands
 * and output, N a multiple of 256, no workspace), whose B rows hold gate and
 * up interleaved in blocks of 128 (act->glu_interleave must be 128): rows
 * 256 t .. 256 t + 127 of each B_g are gate rows 128 t .. 128 t + 127 and the
 * next 128 the matching up rows.  It writes the bf16 product to args->out as
 * usual (the interleaved [gate | up], kept for the backward) and, from the
 * same registers, the MXFP8 activation of (M x N/2) with
 *     a = bf16(silu(gate)), h = bf16(a * up * row_scale[r])
 * (act->kind SwiGLU or clamped SwiGLU), rowwise and / or colwise with the
 * colwise 32-row blocks restarting at every group (scale rows through
 * args->block_off, required for MXQ_COLWISE).  The codes and scales equal
 * those of mxq_swiglu_quantize_fwd applied to args->out with the same act.
 *   row_scale  device fp32[M] or NULL (s = 1)
 *   row_out, col_out as for mxq_swiglu_quantize_fwd with K = N/2
 */
mxq_status mxq_grouped_gemm_swiglu(const mxq_gemm_args *args, const mxq_act *act,
                                   const float *row_scale, uint32_t dirs,
                                   const mxq_mx_out *row_out, const mxq_mx_out *col_out,
                                   void *stream);

/* ------------------------------------------------------------------- misc */

const char *mxq_status_string(mxq_status s);
const char *mxq_last_error_message(void);
const char *mxq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXQ_H */
