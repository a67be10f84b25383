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
//   * A workgroup of 4 waves computes a 256 x 256 output tile, each wave a
//     128 x 128 quadrant as 8 x 8 MFMA tiles of 16 x 16 (256 fp32 accumulators
//     per lane).  Per 128-byte contraction step a wave reads 16 fragments of
//     2 KB from LDS for 64 MFMAs, which keeps LDS reads at half of its
//     bandwidth while the matrix cores run.
//   * Operand tiles go from HBM straight into LDS (buffer_load ... lds, 16 bytes
//     per lane), double-buffered: one barrier per step, the next step's loads in
//     flight during the current step's MFMAs.  Buffer loads are range-checked by
//     the hardware, so rows, columns and contraction tails outside the operand
//     arrive as zeros without a branch.
//   * LDS tiles are XOR-swizzled at 16-byte granularity (chunk c of row r at
//     c ^ (r mod 8) for 128-byte rows, c ^ (r mod 16) for 256-byte rows), which
//     makes both the fragment reads and the transposed reads conflict-free.
//   * MXFP8 uses v_mfma_scale_f32_16x16x128_f8f6f4: lane 16g+i carries row i's
//     contraction bytes [16g, 16g+16) and [64+16g, 80+16g) and the E8M0 scale of
//     row i's 32-element block g, so the block scales are applied inside the
//     matrix core.  bf16 uses v_mfma_f32_16x16x32_bf16.
//   * Operands whose contraction index is strided in memory (the dgrad weight
//     and both wgrad operands) are staged as they lie ([k][column] tiles) and
//     read with ds_read_b64_tr_b8, which transposes 16 lanes' 8-byte rows.
//   * The output tile is computed transposed (the MFMA's first operand is the
//     N side), so every lane owns 4 consecutive output columns of one row.
//   * Group boundaries come from the device offsets only: an M-grouped launch
//     has ceil(M/256) + G tiles per column of tiles and each workgroup finds
//     its group by walking the offsets; surplus workgroups exit.  Work items are
//     spread so that each XCD takes a contiguous range (one expert's tiles
//     share that XCD's L2).
#include "gemm_internal.h"

#include <string>

namespace mxq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

constexpr int BT = 256;            // tile rows on each side (X = output n, Y = output m)
constexpr int BK = 128;            // contraction bytes per step
constexpr int NTHR = 256;
constexpr int OPB = BT * BK;       // bytes of one operand's stage tile (either layout)
constexpr int SCB = 1024;          // bytes of one operand's stage scales
constexpr int STAGE = 2 * OPB + 2 * SCB;
constexpr uint32_t kOOB = 0x80000000u;   // a buffer offset past every range: loads zeros
constexpr int kXCD = 8;

enum { MODE_NT = 0, MODE_NN = 1, MODE_TN = 2 };

__device__ __forceinline__ int64_t xcd_item(int64_t bid, int64_t grid) {
    return (bid % kXCD) * (grid / kXCD) + bid / kXCD;
}

// ------------------------------------------------------------------ staging

// A wave-uniform value the compiler cannot prove uniform, moved to SGPRs.
__device__ __forceinline__ int64_t uni64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Buffer resource over [base, base + bytes) (raw, 32-bit offsets); the
// arguments are wave-uniform, and are moved to SGPRs so that the resource is.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint8_t *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0 : (int)bytes);
    uint8_t *b = reinterpret_cast<uint8_t *>(uni64(reinterpret_cast<int64_t>(base)));
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, __builtin_amdgcn_readfirstlane(n), 0x00020000);
}

// Workgroup barrier that waits only for this wave's LDS operations and for
// all but the last `keep` vector-memory operations (the usual __syncthreads
// fence would also wait for the warm-up loads still in flight).  The empty
// asm statements keep the compiler from moving memory accesses across it.
template <int KEEP>
__device__ __forceinline__ void step_barrier() {
    static_assert(KEEP >= 0 && KEEP < 16, "vmcnt field");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0070 | KEEP);   // vmcnt(KEEP) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void to_lds(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, off, 0, 0, 0);
}

// One operand's view for staging.  K-contiguous: tile rows are output rows,
// 128 contraction bytes each per step.  K-strided: tile rows are contraction
// rows, 256 output columns (bytes) each.
struct Src {
    const uint8_t *base;   // tile origin (row 0 / contraction row 0, first column)
    int64_t pitch;         // bytes between rows in memory
    int64_t kext;          // K-contiguous: contraction bytes per row; K-strided: contraction rows
    int valid;             // K-contiguous: valid tile rows; K-strided: valid column bytes
};

// K-contiguous stage s -> LDS [256 rows][128 B], chunk c of row r at c ^ (r & 7).
// Wave w fills 1 KB blocks 8w..8w+7 (8 rows each).
__device__ __forceinline__ void stage_kc(const Src &o, int64_t s, uint8_t *dst, int wave, int lane) {
    const int64_t k0 = s * BK;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + k0, (int64_t)o.valid * o.pitch - k0);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int b = wave * 8 + j;
        const int row = 8 * b + (lane >> 3);
        const int c = (lane & 7) ^ (row & 7);
        const bool ok = (row < o.valid) & (k0 + 16 * c < o.kext);
        to_lds(r, dst + 1024 * b, ok ? (uint32_t)(row * o.pitch + 16 * c) : kOOB);
    }
}

// K-strided stage s -> LDS [128 contraction rows][256 B], chunk c of row k at c ^ (k & 15).
// Wave w fills 1 KB blocks 8w..8w+7 (4 contraction rows each).
__device__ __forceinline__ void stage_ks(const Src &o, int64_t s, uint8_t *dst, int wave, int lane) {
    const int64_t kr0 = s * 128;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + kr0 * o.pitch, (o.kext - kr0) * o.pitch);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int b = wave * 8 + j;
        const int kr = 4 * b + (lane >> 4);
        const int c = (lane & 15) ^ (kr & 15);
        const bool ok = (kr0 + kr < o.kext) & (16 * c < o.valid);
        to_lds(r, dst + 1024 * b, ok ? (uint32_t)(kr * o.pitch + 16 * c) : kOOB);
    }
}

// L2 warm-up two steps ahead: one 4-byte load per 128-byte line of the
// stage's tile (thread t: K-contiguous row t; K-strided contraction row t / 2,
// half t % 2), delivered into a scratch LDS area that nothing reads, so no
// register waits on them: they only bring the lines into L2.
__device__ __forceinline__ void touch_kc(const Src &o, int64_t s, int t, uint8_t *junk) {
    const int64_t k0 = s * BK;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + k0, (int64_t)o.valid * o.pitch - k0);
    const bool ok = (t < o.valid) & (k0 < o.kext);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)junk, 4, ok ? (uint32_t)(t * o.pitch) : kOOB, 0, 0, 0);
}

__device__ __forceinline__ void touch_ks(const Src &o, int64_t s, int t, uint8_t *junk) {
    const int64_t kr0 = s * 128;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + kr0 * o.pitch, (o.kext - kr0) * o.pitch);
    const int kr = t >> 1, c = 128 * (t & 1);
    const bool ok = (kr0 + kr < o.kext) & (c < o.valid);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)junk, 4, ok ? (uint32_t)(kr * o.pitch + c) : kOOB, 0, 0, 0);
}

// Rowwise E8M0 scales of a K-contiguous operand: thread t packs row t's 4 block
// bytes of step s (blocks past the contraction read 0, i.e. 2^-127 times zeros).
struct RowScales {
    const uint8_t *base;   // scales of tile row 0
    int64_t ld;            // bytes between rows
    int64_t nblk;          // blocks per row
    int valid;             // valid tile rows
};

struct RowScaleBytes {
    uint32_t b[4];
};

// Issued with the stage's loads (range-checked byte loads, no branch), packed
// into a word only when the stage is written to LDS.
__device__ __forceinline__ RowScaleBytes rowscale_load(const RowScales &sc, int64_t s, int t) {
    const __amdgpu_buffer_rsrc_t r = rsrc(sc.base, (int64_t)sc.valid * sc.ld);
    RowScaleBytes v;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const bool ok = (t < sc.valid) & (4 * s + b < sc.nblk);
        v.b[b] = __builtin_amdgcn_raw_buffer_load_b8(r, ok ? (uint32_t)(t * sc.ld + 4 * s + b) : kOOB, 0, 0);
    }
    return v;
}

__device__ __forceinline__ uint32_t rowscale_word(const RowScaleBytes &v) {
    return v.b[0] | (v.b[1] << 8) | (v.b[2] << 16) | (v.b[3] << 24);
}

// When the step's 4 block bytes of every row are one aligned word inside the
// row (the common case: ld % 4 == 0 and a full step of blocks), they go
// straight to LDS [row][4] with one 4-byte load per thread; returns false
// when the byte path above has to be used instead.
__device__ __forceinline__ bool rowscale_dma(const RowScales &sc, int64_t s, int t, uint8_t *dst) {
    if (!((sc.ld % 4 == 0) & (4 * s + 4 <= sc.nblk))) return false;
    const __amdgpu_buffer_rsrc_t r = rsrc(sc.base, (int64_t)sc.valid * sc.ld);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(dst + 4 * (t & ~63)), 4,
                                             t < sc.valid ? (uint32_t)(t * sc.ld + 4 * s) : kOOB, 0, 0, 0);
    return true;
}

// Colwise E8M0 scales of a K-strided operand, step s: block rows 4s..4s+3 x
// 256 columns -> LDS [4][256], loaded by wave 0 (16 bytes per lane).
struct ColScales {
    const uint8_t *base;   // block row 0, tile column 0
    int64_t ld;            // bytes between block rows
    int64_t nblk;          // block rows of the contraction
    int valid;             // valid column bytes
};

__device__ __forceinline__ void stage_colscales(const ColScales &sc, int64_t s, uint8_t *dst, int lane) {
    const int64_t b0 = 4 * s;
    const __amdgpu_buffer_rsrc_t r = rsrc(sc.base + b0 * sc.ld, (sc.nblk - b0) * sc.ld);
    const int b = lane >> 4, c = lane & 15;
    const bool ok = (b0 + b < sc.nblk) & (16 * c < sc.valid);
    to_lds(r, dst, ok ? (uint32_t)(b * sc.ld + 16 * c) : kOOB);
}

// ------------------------------------------------------------------ fragments

// fp8, K-contiguous tile: lane (g, i) gets row `row`'s chunks g and 4 + g.
__device__ __forceinline__ i32x8_t frag_kc_f8(const uint8_t *t, int row, int g) {
    const int sw = row & 7;
    const u32x4_t lo = *reinterpret_cast<const u32x4_t *>(t + row * BK + 16 * (g ^ sw));
    const u32x4_t hi = *reinterpret_cast<const u32x4_t *>(t + row * BK + 16 * ((4 + g) ^ sw));
    return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// fp8, K-strided tile: the same 32 bytes for column col0 + m via transposed
// reads: lane m of the 16-lane group points at contraction row k0 + m/2, bytes
// col0 + 8 (m % 2) .. + 8, and receives 8 consecutive contraction bytes of
// column col0 + m.
__device__ __forceinline__ i32x2_t tr8(const uint8_t *t, int k0, int col0, int m) {
    const int kr = k0 + (m >> 1);
    const uint8_t *p = t + kr * 256 + 16 * ((col0 >> 4) ^ (kr & 15)) + 8 * (m & 1);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)p);
}

__device__ __forceinline__ i32x8_t frag_ks_f8(const uint8_t *t, int col0, int g, int m) {
    const i32x2_t a = tr8(t, 16 * g, col0, m);
    const i32x2_t b = tr8(t, 16 * g + 8, col0, m);
    const i32x2_t c = tr8(t, 64 + 16 * g, col0, m);
    const i32x2_t d = tr8(t, 64 + 16 * g + 8, col0, m);
    return i32x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// bf16, K-contiguous: lane (g, i) carries row i's elements 8g..8g+7 of the
// 32-element half kk of the 64-element step (chunk 4 kk + g).
__device__ __forceinline__ bf16x8_t frag_kc_bf16(const uint8_t *t, int row, int g, int kk) {
    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(t + row * BK + 16 * ((4 * kk + g) ^ (row & 7)));
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

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

// M-grouped: m tile `mt` (counted over all groups in order) -> its group and
// rows.  Each wave scans the groups' tile counts 64 groups at a time (one
// vector load of the offsets per lane and a wave prefix sum), so the search
// costs a few memory round trips whatever G is.
__device__ __forceinline__ TileInfo map_m_grouped(const GemmArgs &a, int64_t mt, int64_t nt, int lane) {
    TileInfo T;
    T.valid = false;
    int64_t cum = 0;
    for (int64_t base = 0; base < a.G; base += 64) {
        const int64_t g = base + lane;
        int c = 0;
        if (g < a.G) {
            const int64_t r0 = a.row_off[g], r1 = a.row_off[g + 1];
            c = r1 > r0 ? (int)((r1 - r0 + BT - 1) / BT) : 0;
        }
        const int incl = wave_scan(c, lane);
        const int total = __shfl(incl, 63, 64);
        if (mt < cum + total) {
            const uint64_t hit = __builtin_amdgcn_ballot_w64(cum + incl > mt);
            const int lg = __builtin_ctzll(hit);
            const int64_t gg = base + lg;
            const int64_t before = cum + __shfl(incl - c, lg, 64);
            const int64_t r0 = a.row_off[gg], r1 = a.row_off[gg + 1];
            T.g = gg;
            T.r0 = r0 + (mt - before) * BT;
            T.rend = r1 < a.M ? r1 : a.M;
            T.m0 = T.r0;
            T.n0 = nt * BT;
            T.valid = T.r0 >= 0 && T.r0 < T.rend;
            return T;
        }
        cum += total;
    }
    return T;
}

// Tile order: within each XCD's contiguous range of items, blocks of RGM m
// tiles x all n tiles are walked m-fastest, so the ~32 tiles an XCD runs at
// once share RGM row panels of A and a few column panels of B in its L2.
constexpr int RGM = 4;

__device__ __forceinline__ void raster(int64_t item, int64_t ntm, int64_t ntn, int64_t &mt, int64_t &nt) {
    const int64_t per = RGM * ntn;
    const int64_t blk = item / per, r = item - blk * per;
    const int64_t m_first = blk * RGM;
    const int64_t gm = ntm - m_first < RGM ? ntm - m_first : RGM;
    mt = m_first + r % gm;
    nt = r / gm;
}

// ------------------------------------------------------------------ kernel

template <int MODE, int DT, int OUT>
__global__ void __launch_bounds__(NTHR) gemm_kernel(GemmArgs a, int64_t ntn, int64_t ntm, int64_t nwork) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t junk[4][256];   // warm-up load sink, one row per wave
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wy = (wave & 1) * 128, wx = (wave >> 1) * 128;   // this wave's quadrant (m, n)
    const int gq = lane >> 4, li = lane & 15;
    constexpr bool F8 = (DT == MXQ_DTYPE_MXFP8_E4M3);
    constexpr int ESZ = F8 ? 1 : 2;
    constexpr bool XKS = (MODE != MODE_NT);   // X (N side) K-strided
    constexpr bool YKS = (MODE == MODE_TN);   // Y (M side) K-strided

    const int64_t item = xcd_item(blockIdx.x, gridDim.x);
    if (item >= nwork) return;

    // ---- which tile
    TileInfo T;
    int64_t ksteps;
    if constexpr (MODE == MODE_TN) {
        const int64_t per_g = ntm * ntn;
        T.g = item / per_g;
        const int64_t rem = item - T.g * per_g;
        T.m0 = (rem / ntn) * BT;
        T.n0 = (rem % ntn) * BT;
        int64_t r0 = a.row_off[T.g], r1 = a.row_off[T.g + 1];
        if (r1 > a.rows) r1 = a.rows;
        if (r0 < 0) r0 = 0;
        T.r0 = r0;
        T.rend = r1 > r0 ? r1 : r0;
        T.valid = true;
        ksteps = (T.rend - T.r0 + 127) / 128;
    } else {
        int64_t mt, nt;
        raster(item, ntm, ntn, mt, nt);
        T = map_m_grouped(a, mt, nt, lane);
        if (!__builtin_amdgcn_readfirstlane((int)T.valid)) return;
        T.g = uni64(T.g);
        T.r0 = uni64(T.r0);
        T.rend = uni64(T.rend);
        T.m0 = uni64(T.m0);
        T.n0 = uni64(T.n0);
        ksteps = (a.K * ESZ + BK - 1) / BK;
    }
    const int64_t mlim = MODE == MODE_TN ? a.M : T.rend;
    const int m_valid = (int)(mlim - T.m0 < BT ? mlim - T.m0 : BT);
    const int n_valid = (int)(a.N - T.n0 < BT ? a.N - T.n0 : BT);

    // ---- operand views
    const uint8_t *A = static_cast<const uint8_t *>(a.A.data);
    const uint8_t *B = static_cast<const uint8_t *>(a.B.data);
    const int64_t lda = a.A.ld * ESZ, ldb = a.B.ld * ESZ;
    Src X, Y;
    if constexpr (MODE == MODE_NT) {
        X = Src{B + T.g * a.B.gstride * ESZ + T.n0 * ldb, ldb, a.K * ESZ, n_valid};
        Y = Src{A + T.r0 * lda, lda, a.K * ESZ, m_valid};
    } else if constexpr (MODE == MODE_NN) {
        X = Src{B + T.g * a.B.gstride + T.n0, ldb, a.K, n_valid};
        Y = Src{A + T.r0 * lda, lda, a.K, m_valid};
    } else {
        X = Src{B + T.r0 * ldb + T.n0, ldb, T.rend - T.r0, n_valid};
        Y = Src{A + T.r0 * lda + T.m0, lda, T.rend - T.r0, m_valid};
    }
    RowScales xr{}, yr{};
    ColScales xc{}, yc{};
    if constexpr (F8) {
        const int64_t nblk = (a.K + 31) / 32;
        if constexpr (MODE == MODE_NT) {
            xr = RowScales{a.B.scales + T.g * a.B.scale_gstride + T.n0 * a.B.ld_scales, a.B.ld_scales, nblk, n_valid};
            yr = RowScales{a.A.scales + T.r0 * a.A.ld_scales, a.A.ld_scales, nblk, m_valid};
        } else if constexpr (MODE == MODE_NN) {
            xc = ColScales{a.B.scales + T.g * a.B.scale_gstride + T.n0, a.B.ld_scales, nblk, n_valid};
            yr = RowScales{a.A.scales + T.r0 * a.A.ld_scales, a.A.ld_scales, nblk, m_valid};
        } else {
            const int64_t blk0 = a.block_off[T.g];
            const int64_t gblk = (T.rend - T.r0 + 31) / 32;
            xc = ColScales{a.B.scales + blk0 * a.B.ld_scales + T.n0, a.B.ld_scales, gblk, n_valid};
            yc = ColScales{a.A.scales + blk0 * a.A.ld_scales + T.m0, a.A.ld_scales, gblk, m_valid};
        }
    }

    f32x4_t acc[8][8];
#pragma unroll
    for (int x = 0; x < 8; x++)
#pragma unroll
        for (int y = 0; y < 8; y++) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // stage s -> buffer s & 1: data tiles straight to LDS, row scales via registers

    auto issue = [&](int64_t s) {
        uint8_t *st = smem + (s & 1) * STAGE;
        if constexpr (XKS) stage_ks(X, s, st, wave, lane);
        else stage_kc(X, s, st, wave, lane);
        if constexpr (YKS) stage_ks(Y, s, st + OPB, wave, lane);
        else stage_kc(Y, s, st + OPB, wave, lane);
        if constexpr (F8) {
            if constexpr (MODE == MODE_NT) {
                if (!rowscale_dma(xr, s, tid, st + 2 * OPB))   // rare: byte path, written at once
                    *reinterpret_cast<uint32_t *>(st + 2 * OPB + 4 * tid) = rowscale_word(rowscale_load(xr, s, tid));
            } else if (wave == 0) {
                stage_colscales(xc, s, st + 2 * OPB, lane);
            }
            if constexpr (MODE == MODE_TN) {
                if (wave == 1) stage_colscales(yc, s, st + 2 * OPB + SCB, lane);
            } else {
                if (!rowscale_dma(yr, s, tid, st + 2 * OPB + SCB))
                    *reinterpret_cast<uint32_t *>(st + 2 * OPB + SCB + 4 * tid) = rowscale_word(rowscale_load(yr, s, tid));
            }
        }
    };
    auto touch = [&](int64_t s) {
        if (s < ksteps) {
            if constexpr (XKS) touch_ks(X, s, tid, junk[wave]);
            else touch_kc(X, s, tid, junk[wave]);
            if constexpr (YKS) touch_ks(Y, s, tid, junk[wave]);
            else touch_kc(Y, s, tid, junk[wave]);
        }
    };

    if (ksteps > 0) issue(0);
    touch(1);
    for (int64_t s = 0; s < ksteps; s++) {
        // this wave's loads of step s have landed (only the 2 warm-up loads of
        // step s + 1 may still be in flight behind them)
        __builtin_amdgcn_s_waitcnt(0x0F72);
        step_barrier<2>();               // everyone's loads have landed, and step s - 1's reads are done
        if (s + 1 < ksteps) issue(s + 1);
        touch(s + 2);                    // after the step's loads: the last vector loads in flight
        const uint8_t *st = smem + (s & 1) * STAGE;
        const uint8_t *tx = st, *ty = st + OPB, *scx = st + 2 * OPB, *scy = st + 2 * OPB + SCB;

        if constexpr (F8) {
            i32x8_t fy[8];
            int sy[8];
#pragma unroll
            for (int y = 0; y < 8; y++) {
                const int m = wy + 16 * y;
                if constexpr (YKS) {
                    fy[y] = frag_ks_f8(ty, m, gq, li);
                    sy[y] = scy[gq * 256 + m + li];
                } else {
                    fy[y] = frag_kc_f8(ty, m + li, gq);
                    sy[y] = scy[(m + li) * 4 + gq];
                }
            }
#pragma unroll
            for (int x = 0; x < 8; x++) {
                const int n = wx + 16 * x;
                i32x8_t fx;
                int sx;
                if constexpr (XKS) {
                    fx = frag_ks_f8(tx, n, gq, li);
                    sx = scx[gq * 256 + n + li];
                } else {
                    fx = frag_kc_f8(tx, n + li, gq);
                    sx = scx[(n + li) * 4 + gq];
                }
#pragma unroll
                for (int y = 0; y < 8; y++)
                    acc[x][y] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(fx, fy[y], acc[x][y], 0, 0, 0, sx, 0,
                                                                                  sy[y]);
            }
            // Issue order: a wave's instructions issue in order and an MFMA holds
            // the issue for its whole pipeline slot, so LDS reads bunched between
            // MFMA runs would leave the LDS idle.  Interleave one read after each
            // MFMA (after the first few reads that the first MFMAs need).
#pragma unroll
            for (int i = 0; i < 8; i++) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
            for (int i = 0; i < 40; i++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
        } else {
#pragma unroll
            for (int kk = 0; kk < 2; kk++) {
                bf16x8_t fy[8];
#pragma unroll
                for (int y = 0; y < 8; y++) fy[y] = frag_kc_bf16(ty, wy + 16 * y + li, gq, kk);
#pragma unroll
                for (int x = 0; x < 8; x++) {
                    const bf16x8_t fx = frag_kc_bf16(tx, wx + 16 * x + li, gq, kk);
#pragma unroll
                    for (int y = 0; y < 8; y++)
                        acc[x][y] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fx, fy[y], acc[x][y], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue: lane holds C[m][n .. n+3] for m = wy + 16y + li, n = wx + 16x + 4gq
    uint8_t *out = static_cast<uint8_t *>(a.out);
    const int64_t obase = (MODE == MODE_TN) ? T.g * a.out_gstride : 0;
    if constexpr (OUT == MXQ_DTYPE_BF16) {
        // through LDS, so that each row leaves as 512 contiguous bytes: tile
        // [256 m][256 n] bf16, 16-byte chunk c of row m at c ^ (m & 31)
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        __syncthreads();   // every wave is done with the stage buffers
#pragma unroll
        for (int y = 0; y < 8; y++) {
            const int m = wy + 16 * y + li;
#pragma unroll
            for (int x = 0; x < 8; x++) {
                const int n = wx + 16 * x + 4 * gq;
                const f32x4_t v = acc[x][y];
                bf16x4_t b;
                b.x = (__bf16)v.x; b.y = (__bf16)v.y; b.z = (__bf16)v.z; b.w = (__bf16)v.w;
                *reinterpret_cast<bf16x4_t *>(smem + m * 512 + 16 * ((n >> 3) ^ (m & 31)) + 8 * ((n >> 2) & 1)) = b;
            }
        }
        __syncthreads();
        uint16_t *o16 = reinterpret_cast<uint16_t *>(out) + obase;
#pragma unroll 4
        for (int j = 0; j < 32; j++) {
            const int row = 2 * (4 * j + wave) + (lane >> 5), c = lane & 31;
            if (row < m_valid && 8 * c < n_valid) {
                const u32x4_t v = *reinterpret_cast<const u32x4_t *>(smem + row * 512 + 16 * (c ^ (row & 31)));
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(o16 + (T.m0 + row) * a.ld_out + T.n0 + 8 * c));
            }
        }
        return;
    }
#pragma unroll
    for (int y = 0; y < 8; y++) {
        const int ml = wy + 16 * y + li;
        if (ml >= m_valid) continue;
        const int64_t mrow = T.m0 + ml;
#pragma unroll
        for (int x = 0; x < 8; x++) {
            const int nl = wx + 16 * x + 4 * gq;
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
    const int64_t ntn = (g.N + BT - 1) / BT;
    int64_t ntm, nwork;
    if (MODE == MODE_TN) {
        ntm = (g.M + BT - 1) / BT;
        nwork = g.G * ntm * ntn;
    } else {
        ntm = (g.M + BT - 1) / BT + g.G;   // upper bound of m tiles over all groups
        nwork = ntm * ntn;
    }
    if (nwork <= 0) return hipSuccess;
    const int64_t grid = (nwork + kXCD - 1) / kXCD * kXCD;
    hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT>), dim3((unsigned)grid), dim3(NTHR), 0, stream, g, ntn, ntm, nwork);
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
    // operand tiles are addressed with 32-bit buffer offsets: up to 256 rows of a pitch
    if (in.A.ld * esz >= (int64_t(1) << 23) || in.B.ld * esz >= (int64_t(1) << 23) ||
        (f8 && (in.A.ld_scales >= (int64_t(1) << 23) || in.B.ld_scales >= (int64_t(1) << 23)))) {
        err = "row pitches must stay below 2^23 bytes";
        return MXQ_ERR_OVERFLOW;
    }
    const int64_t tiles = in.mode == MXQ_GEMM_TN ? in.G * ((in.M + 255) / 256) * ((in.N + 255) / 256)
                                                 : ((in.M + 255) / 256 + in.G) * ((in.N + 255) / 256);
    if (tiles + 8 >= (int64_t(1) << 24)) { err = "launch beyond 2^32 work-items"; return MXQ_ERR_OVERFLOW; }
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
