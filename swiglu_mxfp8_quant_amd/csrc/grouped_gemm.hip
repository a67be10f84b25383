// grouped_gemm.hip -- the grouped GEMM over experts on gfx950 MFMA: bf16 and
// MXFP8 (E4M3 codes with E8M0 block scales), M-grouped (forward, dgrad) and
// K-grouped (wgrad), with device-side group offsets.
//
// Pages: NVIDIA/TransformerEngine pull 3224 (Greptile Summary, Sequence
// Diagram: one grouped GEMM over the experts' row groups, with a single
// stacked grouped weight); "[PyTorch] GroupedTensor integration" (Changes: a
// contiguous grouped buffer plus offsets consumed directly by the grouped
// GEMM); "Activation + GroupedLinear Fusion for MOE and other MOE
// optimizations" (Sequence Diagram: grouped forward, then dgrad and wgrad
// of the grouped linear from the quantized gradient).
//
// Design (the pages' cuBLASLt / CuTe GEMMs for NVIDIA parts are prior art only):
//   * A workgroup of 4 waves computes a 128 x 128 output tile; each wave a
//     64 x 64 quadrant as 4 x 4 MFMA tiles of 16 x 16.  Every K step stages a
//     128-row x 128-byte tile of each operand in LDS (128 fp8 or 64 bf16
//     contraction elements), while the next step's global loads are already
//     in flight in registers.
//   * MXFP8 uses v_mfma_scale_f32_16x16x128_f8f6f4: lane 16g+i carries row i's
//     contraction bytes [16g, 16g+16) and [64+16g, 80+16g) and the E8M0 scale of
//     row i's 32-element block g, so the block scales are applied inside the
//     matrix core.  bf16 uses v_mfma_f32_16x16x32_bf16.
//   * Operands whose contraction index is strided in memory (the dgrad weight
//     and both wgrad operands) are staged as they lie and read with
//     ds_read_b64_tr_b8, which transposes 16 lanes' 8-byte rows in flight.
//   * The output tile is computed transposed (the MFMA's first operand is the
//     N side), so every lane owns 4 consecutive output columns of one row and
//     stores them with one vector store.
//   * Group boundaries come from the device offsets only: an M-grouped launch
//     has ceil(M/128) + G tiles per column of tiles and each workgroup finds
//     its group by walking the offsets; surplus workgroups exit.
#include "gemm_internal.h"

#include <string>

namespace mxq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int TM = 128;        // output tile rows (m)
constexpr int TN = 128;        // output tile cols (n)
constexpr int KBYTES = 128;    // contraction bytes per stage and row
constexpr int LROW = KBYTES + 16;  // LDS row pitch (bytes) of a row-major stage tile
constexpr int NTHR = 256;

enum { MODE_NT = 0, MODE_NN = 1, MODE_TN = 2 };

typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

// ------------------------------------------------------------------ staging

// One operand's stage tile: 128 rows x 128 bytes, loaded by 256 lanes as
// 4 x 16 bytes each (lane t: rows t/8 + 32c, byte offset 16 * (t % 8)).
struct Stage {
    u32x4_t v[4];
};

__device__ __forceinline__ void stage_load(Stage &s, const uint8_t *base, int64_t pitch, int rows_valid,
                                           int bytes_valid, int tid) {
    const int col = (tid & 7) * 16;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const int row = (tid >> 3) + 32 * c;
        s.v[c] = u32x4_t{0u, 0u, 0u, 0u};
        if (row < rows_valid && col < bytes_valid)
            s.v[c] = *reinterpret_cast<const u32x4_t *>(base + row * pitch + col);
    }
}

__device__ __forceinline__ void stage_store(const Stage &s, uint8_t *lds, int tid) {
    const int col = (tid & 7) * 16;
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const int row = (tid >> 3) + 32 * c;
        *reinterpret_cast<u32x4_t *>(lds + row * LROW + col) = s.v[c];
    }
}

// Scale tile of one operand for one stage: 4 blocks x 128 rows of E8M0 bytes,
// stored [block][row].  Lanes 0..127 load one row's 4 bytes each.
struct ScaleStage {
    uint32_t w;   // 4 bytes: blocks 0..3 of this lane's row
};

// ------------------------------------------------------------------ operand fetch

// 32 contraction bytes of row `row` of a row-major stage tile, in the
// split-16 order the scaled MFMA expects for lane group g.
__device__ __forceinline__ i32x8_t frag_rowmajor_f8(const uint8_t *lds, int row, int g) {
    const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(lds + row * LROW + 16 * g);
    const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(lds + row * LROW + 64 + 16 * g);
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// The same 32 bytes for column `col0 + i` of a tile stored [k][col] (rows =
// contraction), via transposed LDS reads: lane m of the 16-lane group points
// at row k0 + m/2, column col0 + 8*(m%2), and receives 8 consecutive k of
// column col0 + m.
__device__ __forceinline__ i32x2_t tr8(const uint8_t *lds, int k0, int col0, int m) {
    const uint8_t *p = lds + (k0 + (m >> 1)) * LROW + col0 + 8 * (m & 1);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)p);
}

__device__ __forceinline__ i32x8_t frag_colmajor_f8(const uint8_t *lds, int col0, int g, int m) {
    const i32x2_t a = tr8(lds, 16 * g, col0, m);
    const i32x2_t b = tr8(lds, 16 * g + 8, col0, m);
    const i32x2_t c = tr8(lds, 64 + 16 * g, col0, m);
    const i32x2_t d = tr8(lds, 64 + 16 * g + 8, col0, m);
    return i32x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// bf16: lane 16g+i carries row i's elements 8g..8g+7 of a 32-element k step
__device__ __forceinline__ bf16x8_t frag_rowmajor_bf16(const uint8_t *lds, int row, int g, int kk) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(lds + row * LROW + 64 * kk + 16 * g);
    return __builtin_bit_cast(bf16x8_t, v);
}

// ------------------------------------------------------------------ tile mapping

struct TileInfo {
    int64_t g;       // group
    int64_t r0;      // first output row (NT/NN) or first contraction row (TN)
    int64_t rend;    // end of the group's rows
    int64_t m0;      // first output row of the tile (TN: output m)
    int64_t n0;      // first output col
    bool valid;
};

// M-grouped: linear tile -> (group, m tile, n tile), walking the offsets.
__device__ __forceinline__ TileInfo map_m_grouped(const GemmArgs &a, int64_t t, int64_t ntn) {
    TileInfo T;
    T.valid = false;
    const int64_t nt = t % ntn, mt = t / ntn;
    int64_t cum = 0;
    for (int64_t g = 0; g < a.G; g++) {
        const int64_t r0 = a.row_off[g], r1 = a.row_off[g + 1];
        const int64_t m = r1 > r0 ? r1 - r0 : 0;
        const int64_t c = (m + TM - 1) / TM;
        if (mt < cum + c) {
            T.g = g;
            T.r0 = r0 + (mt - cum) * TM;
            T.rend = r1 < a.M ? r1 : a.M;
            T.m0 = T.r0;
            T.n0 = nt * TN;
            T.valid = T.r0 >= 0 && T.r0 < T.rend;
            return T;
        }
        cum += c;
    }
    return T;
}

// ------------------------------------------------------------------ kernel

template <int MODE, int DT, int OUT>
__global__ void __launch_bounds__(NTHR) gemm_kernel(GemmArgs a, int64_t ntn, int64_t ntm) {
    __shared__ uint8_t ldsX[TN * LROW];   // N side (MFMA first operand)
    __shared__ uint8_t ldsY[TM * LROW];   // M side (MFMA second operand)
    __shared__ uint8_t scX[4][TN];
    __shared__ uint8_t scY[4][TM];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = (wave & 1) * 64, wn = (wave >> 1) * 64;   // this wave's quadrant
    const int gq = lane >> 4, li = lane & 15;
    constexpr bool F8 = (DT == MXQ_DTYPE_MXFP8_E4M3);
    constexpr int ESZ = F8 ? 1 : 2;

    // ---- which tile
    TileInfo T;
    int64_t ksteps;
    if constexpr (MODE == MODE_TN) {
        const int64_t t = blockIdx.x;
        const int64_t per_g = ntm * ntn;
        T.g = t / per_g;
        const int64_t rem = t - T.g * per_g;
        T.m0 = (rem / ntn) * TM;
        T.n0 = (rem % ntn) * TN;
        int64_t r0 = a.row_off[T.g], r1 = a.row_off[T.g + 1];
        if (r1 > a.rows) r1 = a.rows;
        if (r0 < 0) r0 = 0;
        T.r0 = r0;
        T.rend = r1;
        T.valid = true;
        ksteps = r1 > r0 ? (r1 - r0 + 127) / 128 : 0;
    } else {
        T = map_m_grouped(a, blockIdx.x, ntn);
        if (!T.valid) return;
        ksteps = (a.K * ESZ + KBYTES - 1) / KBYTES;
    }
    const int m_valid = (int)((MODE == MODE_TN ? a.M : T.rend) - T.m0 < TM ? (MODE == MODE_TN ? a.M : T.rend) - T.m0 : TM);
    const int n_valid = (int)(a.N - T.n0 < TN ? a.N - T.n0 : TN);

    // ---- operand bases
    const uint8_t *A = static_cast<const uint8_t *>(a.A.data);
    const uint8_t *B = static_cast<const uint8_t *>(a.B.data);
    const int64_t lda = a.A.ld * ESZ, ldb = a.B.ld * ESZ;   // row pitches in bytes
    const uint8_t *Bg = B + (MODE == MODE_TN ? 0 : T.g * a.B.gstride * ESZ);
    const uint8_t *Bsg = F8 ? a.B.scales + (MODE == MODE_TN ? 0 : T.g * a.B.scale_gstride) : nullptr;
    int64_t blk0 = 0;   // TN: first colwise scale row of the group
    if constexpr (MODE == MODE_TN) {
        if (F8) blk0 = a.block_off[T.g];
    }

    f32x4_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // global stage loads for step s into registers
    Stage sx, sy;
    uint32_t sxs = 0x7F7F7F7Fu, sys = 0x7F7F7F7Fu;   // this lane's scale words (lanes < 128)
    auto load_step = [&](int64_t s) {
        if constexpr (MODE == MODE_NT) {
            // X: B_g rows n0.., bytes of step s; Y: A rows r0.., same bytes
            const int64_t kb = s * KBYTES;
            const int kbytes = (int)(a.K * ESZ - kb < KBYTES ? a.K * ESZ - kb : KBYTES);
            stage_load(sx, Bg + T.n0 * ldb + kb, ldb, n_valid, kbytes, tid);
            stage_load(sy, A + T.r0 * lda + kb, lda, m_valid, kbytes, tid);
            if (F8 && tid < 128) {
                const int64_t nb = (a.K + 31) / 32;
                uint32_t wx = 0x7F7F7F7Fu, wy = 0x7F7F7F7Fu;
                if (tid < n_valid) {
                    const uint8_t *p = Bsg + (T.n0 + tid) * a.B.ld_scales + 4 * s;
                    wx = 0;
                    for (int b = 0; b < 4; b++) wx |= (uint32_t)(4 * s + b < nb ? p[b] : 127) << (8 * b);
                }
                if (tid < m_valid) {
                    const uint8_t *p = a.A.scales + (T.r0 + tid) * a.A.ld_scales + 4 * s;
                    wy = 0;
                    for (int b = 0; b < 4; b++) wy |= (uint32_t)(4 * s + b < nb ? p[b] : 127) << (8 * b);
                }
                sxs = wx;
                sys = wy;
            }
        } else if constexpr (MODE == MODE_NN) {
            // X: B_g rows k (128 of them), bytes n0..; Y: A rows r0.., bytes of step s
            const int64_t k0 = s * 128;
            const int krows = (int)(a.K - k0 < 128 ? a.K - k0 : 128);
            stage_load(sx, Bg + k0 * ldb + T.n0, ldb, krows, n_valid, tid);
            stage_load(sy, A + T.r0 * lda + k0, lda, m_valid, krows, tid);
            if (tid < 128) {
                const int64_t nb = (a.K + 31) / 32;
                uint32_t wx = 0x7F7F7F7Fu, wy = 0x7F7F7F7Fu;
                if (tid < n_valid) {
                    wx = 0;
                    for (int b = 0; b < 4; b++)
                        wx |= (uint32_t)(4 * s + b < nb ? Bsg[(4 * s + b) * a.B.ld_scales + T.n0 + tid] : 127) << (8 * b);
                }
                if (tid < m_valid) {
                    const uint8_t *p = a.A.scales + (T.r0 + tid) * a.A.ld_scales + 4 * s;
                    wy = 0;
                    for (int b = 0; b < 4; b++) wy |= (uint32_t)(4 * s + b < nb ? p[b] : 127) << (8 * b);
                }
                sxs = wx;
                sys = wy;
            }
        } else {
            // TN: X: B rows r (group rows), bytes n0..; Y: A rows r, bytes m0..
            const int64_t r = T.r0 + s * 128;
            const int rrows = (int)(T.rend - r < 128 ? T.rend - r : 128);
            stage_load(sx, B + r * ldb + T.n0, ldb, rrows, n_valid, tid);
            stage_load(sy, A + r * lda + T.m0, lda, rrows, m_valid, tid);
            if (tid < 128) {
                const int64_t gblocks = (T.rend - T.r0 + 31) / 32;
                uint32_t wx = 0x7F7F7F7Fu, wy = 0x7F7F7F7Fu;
                if (tid < n_valid) {
                    wx = 0;
                    for (int b = 0; b < 4; b++) {
                        const int64_t bi = 4 * s + b;
                        wx |= (uint32_t)(bi < gblocks ? a.B.scales[(blk0 + bi) * a.B.ld_scales + T.n0 + tid] : 127) << (8 * b);
                    }
                }
                if (tid < m_valid) {
                    wy = 0;
                    for (int b = 0; b < 4; b++) {
                        const int64_t bi = 4 * s + b;
                        wy |= (uint32_t)(bi < gblocks ? a.A.scales[(blk0 + bi) * a.A.ld_scales + T.m0 + tid] : 127) << (8 * b);
                    }
                }
                sxs = wx;
                sys = wy;
            }
        }
    };

    if (ksteps > 0) load_step(0);
    for (int64_t s = 0; s < ksteps; s++) {
        __syncthreads();   // the previous step's reads of LDS are done
        stage_store(sx, ldsX, tid);
        stage_store(sy, ldsY, tid);
        if (F8 && tid < 128) {
#pragma unroll
            for (int b = 0; b < 4; b++) {
                scX[b][tid] = (uint8_t)(sxs >> (8 * b));
                scY[b][tid] = (uint8_t)(sys >> (8 * b));
            }
        }
        __syncthreads();
        if (s + 1 < ksteps) load_step(s + 1);   // next step's loads in flight during the MFMAs

        if constexpr (F8) {
            i32x8_t fx[4], fy[4];
            int sa[4], sb[4];
#pragma unroll
            for (int x = 0; x < 4; x++) {
                const int n = wn + 16 * x;
                if constexpr (MODE == MODE_NT) fx[x] = frag_rowmajor_f8(ldsX, n + li, gq);
                else fx[x] = frag_colmajor_f8(ldsX, n, gq, li);
                sa[x] = scX[gq][n + li];
            }
#pragma unroll
            for (int y = 0; y < 4; y++) {
                const int m = wm + 16 * y;
                if constexpr (MODE == MODE_TN) fy[y] = frag_colmajor_f8(ldsY, m, gq, li);
                else fy[y] = frag_rowmajor_f8(ldsY, m + li, gq);
                sb[y] = scY[gq][m + li];
            }
#pragma unroll
            for (int x = 0; x < 4; x++)
#pragma unroll
                for (int y = 0; y < 4; y++)
                    acc[x][y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fx[x], fy[y], acc[x][y], 0, 0, 0,
                                                                                  sa[x], 0, sb[y]);
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                bf16x8_t fx[4], fy[4];
#pragma unroll
                for (int x = 0; x < 4; x++) fx[x] = frag_rowmajor_bf16(ldsX, wn + 16 * x + li, gq, kk);
#pragma unroll
                for (int y = 0; y < 4; y++) fy[y] = frag_rowmajor_bf16(ldsY, wm + 16 * y + li, gq, kk);
#pragma unroll
                for (int x = 0; x < 4; x++)
#pragma unroll
                    for (int y = 0; y < 4; y++)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx[x], fy[y], acc[x][y], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: lane holds C[m][n .. n+3] for m = wm + 16y + li, n = wn + 16x + 4gq
    uint8_t *out = static_cast<uint8_t *>(a.out);
    const int64_t obase = (MODE == MODE_TN) ? T.g * a.out_gstride : 0;
#pragma unroll
    for (int y = 0; y < 4; y++) {
        const int ml = wm + 16 * y + li;
        if (ml >= m_valid) continue;
        const int64_t mrow = T.m0 + ml;
#pragma unroll
        for (int x = 0; x < 4; x++) {
            const int nl = wn + 16 * x + 4 * gq;
            if (nl >= n_valid) continue;
            const int64_t idx = obase + mrow * a.ld_out + T.n0 + nl;
            const f32x4_t v = acc[x][y];
            if constexpr (OUT == MXQ_DTYPE_F32) {
                float *o = reinterpret_cast<float *>(out) + idx;
                if (a.accumulate) {
                    const f32x4_t old = *reinterpret_cast<const f32x4_t *>(o);
                    *reinterpret_cast<f32x4_t *>(o) = old + v;
                } else {
                    *reinterpret_cast<f32x4_t *>(o) = v;
                }
            } else {
                uint16_t *o = reinterpret_cast<uint16_t *>(out) + idx;
                typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
                bf16x4_t b;
                b.x = (__bf16)v.x; b.y = (__bf16)v.y; b.z = (__bf16)v.z; b.w = (__bf16)v.w;
                *reinterpret_cast<bf16x4_t *>(o) = b;
            }
        }
    }
}

template <int MODE, int DT, int OUT>
hipError_t launch_mode(const GemmArgs &g, hipStream_t stream) {
    const int64_t ntn = (g.N + TN - 1) / TN;
    int64_t ntm, nblocks;
    if (MODE == MODE_TN) {
        ntm = (g.M + TM - 1) / TM;
        nblocks = g.G * ntm * ntn;
    } else {
        ntm = (g.M + TM - 1) / TM + g.G;   // upper bound of m tiles over all groups
        nblocks = ntm * ntn;
    }
    if (nblocks <= 0) return hipSuccess;
    hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT>), dim3((unsigned)nblocks), dim3(NTHR), 0, stream, g, ntn, ntm);
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

int gemm_prepare(const mxq_gemm_args &in, GemmArgs &g, std::string &err) {
    g = GemmArgs{};
    g.mode = in.mode;
    g.G = in.G;
    g.row_off = in.row_off;
    g.block_off = in.block_off;
    g.M = in.M;
    g.N = in.N;
    g.K = in.K;
    g.rows = in.rows;
    g.A = GemmOperand{in.A.dtype, in.A.data, in.A.ld, in.A.gstride, in.A.scales, in.A.ld_scales, in.A.scale_gstride};
    g.B = GemmOperand{in.B.dtype, in.B.data, in.B.ld, in.B.gstride, in.B.scales, in.B.ld_scales, in.B.scale_gstride};
    g.out_dtype = in.out_dtype;
    g.out = in.out;
    g.ld_out = in.ld_out;
    g.out_gstride = in.out_gstride;
    g.accumulate = in.accumulate;
    g.noop = false;
    if (in.mode < MXQ_GEMM_NT || in.mode > MXQ_GEMM_TN) { err = "unknown GEMM mode"; return MXQ_ERR_SHAPE; }
    if (in.G < 1 || in.G > (int64_t(1) << 24)) { err = "G must be in [1, 2^24]"; return MXQ_ERR_SHAPE; }
    if (in.row_off == nullptr) { err = "row_off is required"; return MXQ_ERR_NULL; }
    if (in.M < 0 || in.N < 0 || in.K < 0 || in.rows < 0) { err = "negative size"; return MXQ_ERR_SHAPE; }
    if (in.A.dtype != in.B.dtype) { err = "A and B must have the same dtype"; return MXQ_ERR_UNSUPPORTED; }
    const bool f8 = in.A.dtype == MXQ_DTYPE_MXFP8_E4M3;
    if (!f8 && in.A.dtype != MXQ_DTYPE_BF16) { err = "operand dtype must be BF16 or MXFP8_E4M3"; return MXQ_ERR_UNSUPPORTED; }
    if (!f8 && in.mode != MXQ_GEMM_NT) { err = "bf16 operands are built for the NT mode only"; return MXQ_ERR_UNSUPPORTED; }
    if (in.out_dtype != MXQ_DTYPE_BF16 && in.out_dtype != MXQ_DTYPE_F32) { err = "out_dtype must be BF16 or F32"; return MXQ_ERR_UNSUPPORTED; }
    if (in.accumulate && !(in.mode == MXQ_GEMM_TN && in.out_dtype == MXQ_DTYPE_F32)) {
        err = "accumulate is supported for TN with an F32 output";
        return MXQ_ERR_UNSUPPORTED;
    }
    if (in.A.data == nullptr || in.B.data == nullptr || in.out == nullptr) { err = "A, B and out are required"; return MXQ_ERR_NULL; }
    if (f8 && (in.A.scales == nullptr || in.B.scales == nullptr)) { err = "MXFP8 operands need scales"; return MXQ_ERR_NULL; }
    if (f8 && in.mode == MXQ_GEMM_TN && in.block_off == nullptr) { err = "MXFP8 TN needs block_off"; return MXQ_ERR_NULL; }
    const int64_t esz = f8 ? 1 : 2;
    // every dimension that is read with 16-byte vectors must keep 16-byte alignment
    if (in.N % 16 != 0) { err = "N must be a multiple of 16"; return MXQ_ERR_SHAPE; }
    if (in.mode != MXQ_GEMM_TN && in.K % 32 != 0) { err = "K must be a multiple of 32"; return MXQ_ERR_SHAPE; }
    if (in.mode == MXQ_GEMM_TN && in.M % 16 != 0) { err = "M must be a multiple of 16 for TN"; return MXQ_ERR_SHAPE; }
    if (!aligned16(in.A.data) || !aligned16(in.B.data) || (in.A.ld * esz) % 16 != 0 || (in.B.ld * esz) % 16 != 0 ||
        (in.B.gstride * esz) % 16 != 0) {
        err = "operand pointers, row pitches and group strides must be multiples of 16 bytes";
        return MXQ_ERR_ALIGN;
    }
    if (!aligned16(in.out) || (in.ld_out % 8) != 0 || (in.out_gstride % 8) != 0) {
        err = "out pointer and pitches must be 16-byte aligned";
        return MXQ_ERR_ALIGN;
    }
    // operand extents
    if (in.mode == MXQ_GEMM_NT) {
        if (in.A.ld < in.K || in.B.ld < in.K || in.ld_out < in.N) { err = "ld too small"; return MXQ_ERR_SHAPE; }
        if (in.B.gstride < (in.N - 1) * in.B.ld + in.K && in.G > 1) { err = "B group stride too small"; return MXQ_ERR_SHAPE; }
        if (f8 && (in.A.ld_scales < (in.K + 31) / 32 || in.B.ld_scales < (in.K + 31) / 32)) { err = "ld_scales too small"; return MXQ_ERR_SHAPE; }
    } else if (in.mode == MXQ_GEMM_NN) {
        if (in.A.ld < in.K || in.B.ld < in.N || in.ld_out < in.N) { err = "ld too small"; return MXQ_ERR_SHAPE; }
        if (in.B.gstride < (in.K - 1) * in.B.ld + in.N && in.G > 1) { err = "B group stride too small"; return MXQ_ERR_SHAPE; }
        if (f8 && (in.A.ld_scales < (in.K + 31) / 32 || in.B.ld_scales < in.N)) { err = "ld_scales too small"; return MXQ_ERR_SHAPE; }
    } else {
        if (in.A.ld < in.M || in.B.ld < in.N || in.ld_out < in.N) { err = "ld too small"; return MXQ_ERR_SHAPE; }
        if (in.G > 1 && in.out_gstride < (in.M - 1) * in.ld_out + in.N) { err = "out group stride too small"; return MXQ_ERR_SHAPE; }
        if (f8 && (in.A.ld_scales < in.M || in.B.ld_scales < in.N)) { err = "ld_scales too small"; return MXQ_ERR_SHAPE; }
    }
    const int64_t tiles = in.mode == MXQ_GEMM_TN ? in.G * ((in.M + 127) / 128) * ((in.N + 127) / 128)
                                                 : ((in.M + 127) / 128 + in.G) * ((in.N + 127) / 128);
    if (tiles >= (int64_t(1) << 31)) { err = "launch grid beyond 2^31 workgroups"; return MXQ_ERR_OVERFLOW; }
    g.noop = (in.M == 0 || in.N == 0);
    return MXQ_OK;
}

hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream) {
    const bool f8 = g.A.dtype == MXQ_DTYPE_MXFP8_E4M3;
    const bool o32 = g.out_dtype == MXQ_DTYPE_F32;
    switch (g.mode) {
        case MXQ_GEMM_NT:
            if (f8) return o32 ? launch_mode<MODE_NT, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_F32>(g, stream)
                               : launch_mode<MODE_NT, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_BF16>(g, stream);
            return o32 ? launch_mode<MODE_NT, MXQ_DTYPE_BF16, MXQ_DTYPE_F32>(g, stream)
                       : launch_mode<MODE_NT, MXQ_DTYPE_BF16, MXQ_DTYPE_BF16>(g, stream);
        case MXQ_GEMM_NN:
            return o32 ? launch_mode<MODE_NN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_F32>(g, stream)
                       : launch_mode<MODE_NN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_BF16>(g, stream);
        default:
            return o32 ? launch_mode<MODE_TN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_F32>(g, stream)
                       : launch_mode<MODE_TN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_BF16>(g, stream);
    }
}

}  // namespace mxq
