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
//   * Group boundaries come from the device offsets only.  Each workgroup of
//     an M-grouped launch first builds the groups' m-tile prefix sums in LDS
//     (for up to 4096 groups; beyond that every lookup scans the offsets), so
//     the exact tile count is known on the device and a tile's group is two
//     wave-wide LDS probes away.
//   * The grid is persistent: one workgroup per CU, each looping over its
//     share of the tiles.  Each XCD takes a contiguous range of tiles (one
//     expert's tiles share that XCD's L2).  The next tile's first stage is
//     loaded during the current tile's last step, and the epilogue stores
//     straight from the accumulators, so consecutive tiles overlap.
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
    static_assert(KEEP >= 0 && KEEP < 64, "vmcnt field");
    asm volatile("" ::: "memory");
    // vmcnt(KEEP) (low 4 bits in [3:0], high 2 bits in [15:14]) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt(0x0070 | (KEEP & 15) | ((KEEP >> 4) << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A uniform value the compiler must treat as unknown at each use, so that
// per-lane products of it are recomputed where they are needed instead of
// being hoisted out of the tile loop into long-lived registers.
__device__ __forceinline__ int opaque(int v) {
    asm volatile("" : "+s"(v));
    return v;
}

__device__ __forceinline__ void to_lds(__amdgpu_buffer_rsrc_t r, uint8_t *dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)dst, 16, off, 0, 0, 0);
}

// One operand's view for staging.  K-contiguous: tile rows are output rows,
// 128 contraction bytes each per step.  K-strided: tile rows are contraction
// rows, 256 output columns (bytes) each.
struct Src {
    const uint8_t *base;   // tile origin (row 0 / contraction row 0, first column)
    int pitch;             // bytes between rows in memory (< 2^23)
    int kext;              // K-contiguous: contraction bytes per row; K-strided: contraction rows
    int valid;             // K-contiguous: valid tile rows; K-strided: valid column bytes
};

// K-contiguous stage s -> LDS [256 rows][128 B], chunk c of row r at c ^ (r & 7).
// Wave w fills 1 KB blocks 8w..8w+7 (8 rows each).
__device__ __forceinline__ void stage_kc(const Src &o, int s, uint8_t *dst, int wave, int lane) {
    const int k0 = s * BK;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + k0, (int64_t)o.valid * o.pitch - k0);
    const int pitch = opaque(o.pitch);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int b = wave * 8 + j;
        const int row = 8 * b + (lane >> 3);
        const int c = (lane & 7) ^ (row & 7);
        const bool ok = (row < o.valid) & (k0 + 16 * c < o.kext);
        to_lds(r, dst + 1024 * b, ok ? (uint32_t)(row * pitch + 16 * c) : kOOB);
    }
}

// K-strided stage s -> LDS [128 contraction rows][256 B], chunk c of row k at c ^ (k & 15).
// Wave w fills 1 KB blocks 8w..8w+7 (4 contraction rows each).
__device__ __forceinline__ void stage_ks(const Src &o, int s, uint8_t *dst, int wave, int lane) {
    const int kr0 = s * 128;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + (int64_t)kr0 * o.pitch, (int64_t)(o.kext - kr0) * o.pitch);
    const int pitch = opaque(o.pitch);
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const int b = wave * 8 + j;
        const int kr = 4 * b + (lane >> 4);
        const int c = (lane & 15) ^ (kr & 15);
        const bool ok = (kr0 + kr < o.kext) & (16 * c < o.valid);
        to_lds(r, dst + 1024 * b, ok ? (uint32_t)(kr * pitch + 16 * c) : kOOB);
    }
}

// L2 warm-up two steps ahead: one 4-byte load per 128-byte line of the
// stage's tile (thread t: K-contiguous row t; K-strided contraction row t / 2,
// half t % 2), delivered into a scratch LDS area that nothing reads, so no
// register waits on them: they only bring the lines into L2.  When `live` is
// false the load is still issued, out of range (no memory access).
__device__ __forceinline__ void touch_kc(const Src &o, int s, int t, uint8_t *junk, bool live) {
    const int k0 = s * BK;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + k0, (int64_t)o.valid * o.pitch - k0);
    const bool ok = live & (t < o.valid) & (k0 < o.kext);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)junk, 4, ok ? (uint32_t)(t * o.pitch) : kOOB, 0, 0, 0);
}

__device__ __forceinline__ void touch_ks(const Src &o, int s, int t, uint8_t *junk, bool live) {
    const int kr0 = s * 128;
    const __amdgpu_buffer_rsrc_t r = rsrc(o.base + (int64_t)kr0 * o.pitch, (int64_t)(o.kext - kr0) * o.pitch);
    const int kr = t >> 1, c = 128 * (t & 1);
    const bool ok = live & (kr0 + kr < o.kext) & (c < o.valid);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)junk, 4, ok ? (uint32_t)(kr * o.pitch + c) : kOOB, 0, 0, 0);
}

// Rowwise E8M0 scales of a K-contiguous operand: thread t packs row t's 4 block
// bytes of step s (blocks past the contraction read 0, i.e. 2^-127 times zeros).
struct RowScales {
    const uint8_t *base;   // scales of tile row 0
    int ld;                // bytes between rows (< 2^23)
    int nblk;              // blocks per row
    int valid;             // valid tile rows
};

struct RowScaleBytes {
    uint32_t b[4];
};

// Issued with the stage's loads (range-checked byte loads, no branch), packed
// into a word only when the stage is written to LDS.
__device__ __forceinline__ RowScaleBytes rowscale_load(const RowScales &sc, int s, int t) {
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
__device__ __forceinline__ bool rowscale_dma(const RowScales &sc, int s, int t, uint8_t *dst) {
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
    int ld;                // bytes between block rows (< 2^23)
    int nblk;              // block rows of the contraction
    int valid;             // valid column bytes
};

__device__ __forceinline__ void stage_colscales(const ColScales &sc, int s, uint8_t *dst, int lane) {
    const int b0 = 4 * s;
    const __amdgpu_buffer_rsrc_t r = rsrc(sc.base + (int64_t)b0 * sc.ld, (int64_t)(sc.nblk - b0) * sc.ld);
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
    int64_t item;    // work item
    int64_t g;       // group
    int64_t r0;      // first output row (NT/NN) or first contraction row (TN)
    int64_t rend;    // end of the group's rows
    int64_t m0;      // first output row of the tile (TN: output m)
    int64_t n0;      // first output col
    int64_t ksteps;  // contraction steps
    bool valid;
};

// Inclusive prefix sum over the 64 lanes of a wave, saturating at cap (every
// input in [0, cap], cap < 2^30, so no partial sum overflows).
__device__ __forceinline__ int wave_scan(int v, int lane, int cap) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v = min(v + u, cap);
    }
    return v;
}

// Rows of M-grouped group g, clipped to [0, M).
__device__ __forceinline__ void group_rows(const GemmArgs &a, int64_t g, int64_t &r0, int64_t &r1) {
    r0 = a.row_off[g];
    r1 = a.row_off[g + 1];
    r0 = r0 < 0 ? 0 : r0;
    r1 = r1 > a.M ? a.M : r1;
    r1 = r1 < r0 ? r0 : r1;
}

__device__ __forceinline__ int group_mtiles(const GemmArgs &a, int64_t g, int cap) {
    int64_t r0, r1;
    group_rows(a, g, r0, r1);
    const int64_t c = (r1 - r0 + BT - 1) / BT;
    return (int)(c < cap ? c : cap);
}

// Groups up to this count keep their offsets and m-tile prefix in LDS.
constexpr int kTab = 2048;

// LDS group tables, so that the tile loop reads no global memory:
//   rs[g]  (g <= G) = row_off[g] clipped to [0, M] (TN: [0, rows]), so group
//          g's rows are [rs[g], max(rs[g + 1], rs[g]));
//   tab[g] (M-grouped) = m tiles of the groups before g, saturating at cap,
//          tab[G] = all of them; (TN) = block_off[g].
template <int MODE>
__device__ void build_group_tables(const GemmArgs &a, int *rs, int *tab, int *wsum, int cap, int tid, int lane,
                                   int wave) {
    const int64_t lim = MODE == MODE_TN ? a.rows : a.M;
    for (int64_t g = tid; g <= a.G; g += NTHR) {
        const int64_t r = a.row_off[g];
        rs[g] = (int)(r < 0 ? 0 : (r > lim ? lim : r));
    }
    if constexpr (MODE == MODE_TN) {
        for (int64_t g = tid; g < a.G; g += NTHR) tab[g] = a.block_off != nullptr ? (int)a.block_off[g] : 0;
        __syncthreads();
        return;
    }
    __syncthreads();
    int carry = 0;
    for (int64_t base = 0; base < a.G; base += NTHR) {
        const int64_t g = base + tid;
        int c = 0;
        if (g < a.G) {
            const int n = rs[g + 1] - rs[g];
            c = n > 0 ? min(n / BT + (n % BT != 0), cap) : 0;
        }
        const int incl = wave_scan(c, lane, cap);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        int before = carry;
        for (int w = 0; w < wave; w++) before = min(before + wsum[w], cap);
        if (g < a.G) tab[g + 1] = min(before + incl, cap);
        carry = min(carry + min(wsum[0] + wsum[1], cap) + min(wsum[2] + wsum[3], cap), cap);
        __syncthreads();   // wsum is rewritten by the next round
    }
    if (tid == 0) tab[0] = 0;
    __syncthreads();
}

// Group of m tile mt (< tab[G]) from the table: the last g with tab[g] <= mt,
// found with two wave-wide probes (every S-th entry, then S entries).
__device__ __forceinline__ int64_t table_group(const int *tab, int G, int mt, int lane) {
    const int S = (G + 63) / 64;   // <= 64
    const int i1 = lane * S;
    const uint64_t b1 = __builtin_amdgcn_ballot_w64(i1 <= G && tab[i1 <= G ? i1 : G] <= mt);
    const int L = 63 - __builtin_clzll(b1);   // tab[0] = 0 <= mt: lane 0 is always set
    const int i2 = L * S + lane;
    const uint64_t b2 = __builtin_amdgcn_ballot_w64(lane < S && i2 <= G && tab[i2 <= G ? i2 : G] <= mt);
    return (int64_t)L * S + (63 - __builtin_clzll(b2));
}

// Without the table: each wave scans the groups' tile counts 64 groups at a
// time (one vector load of the offsets per lane and a wave prefix sum).
__device__ __forceinline__ int64_t scan_group(const GemmArgs &a, int64_t mt, int cap, int lane, int64_t &before) {
    int64_t cum = 0;
    for (int64_t base = 0; base < a.G; base += 64) {
        const int64_t g = base + lane;
        const int c = g < a.G ? group_mtiles(a, g, cap) : 0;
        const int incl = wave_scan(c, lane, cap);
        const int total = __shfl(incl, 63, 64);
        if (mt < cum + total) {
            const int lg = __builtin_ctzll(__builtin_amdgcn_ballot_w64(cum + incl > mt));
            before = cum + __shfl(incl - c, lg, 64);
            return base + lg;
        }
        cum += total;
    }
    return -1;
}

// Tile order: within each XCD's contiguous range of items, blocks of RGM m
// tiles x all n tiles are walked m-fastest, so the ~32 tiles an XCD runs at
// once share RGM row panels of A and a few column panels of B in its L2.
constexpr int RGM = 4;

__device__ __forceinline__ void raster(int item, int ntm, int ntn, int &mt, int &nt) {
    const int per = RGM * ntn;
    const int blk = item / per, r = item - blk * per;
    const int m_first = blk * RGM;
    const int gm = ntm - m_first < RGM ? ntm - m_first : RGM;
    mt = m_first + r % gm;
    nt = r / gm;
}

// ------------------------------------------------------------------ kernel

// What the steps and the epilogue of one tile need (32-bit counts, origins
// precomputed), so that two of them fit in scalar registers beside the loop.
struct Tile {
    const uint8_t *x, *y;     // operand tile origins (contraction position 0)
    const uint8_t *xs, *ys;   // E8M0 scale origins
    uint8_t *o;               // output tile origin
    int xv, yv;               // valid output columns (n) and rows (m)
    int kext;                 // contraction extent: bytes (NT/NN) or the group's rows (TN)
    int nblk;                 // E8M0 blocks along the contraction
    int ksteps;
    int item;
    int valid;
};

// A persistent grid (one workgroup per CU at most): workgroup j of XCD x runs
// items x * per + j, + nj, ... of that XCD's contiguous range.  While a tile's
// last step computes, the next tile's first stage is already loading into the
// free buffer, and the epilogue stores straight from registers, so the stores
// drain under the next tile's loads and MFMAs.  TAB: the groups' m-tile
// prefix is kept in LDS (G <= kTab), else every lookup scans the offsets.
template <int MODE, int DT, int OUT, bool TAB>
__global__ void __launch_bounds__(NTHR) gemm_kernel(GemmArgs a, int ntn, int ntm_ub) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t junk[4][256];   // warm-up load sink, one row per wave
    __shared__ int tab[TAB ? kTab + 1 : 1];
    __shared__ int rs[TAB ? kTab + 1 : 1];
    __shared__ int wsum[4];
    // the arguments that only the per-tile lookup reads live in LDS, so that
    // they do not hold scalar registers through the loop
    __shared__ GemmArgs sa;
    // the next tile's descriptor, one copy per wave: read back only at the
    // tile's last steps, so it holds no scalar registers through the loop
    __shared__ Tile tnext[4];
    // Per-lane indices are refreshed through an opaque copy at every tile, so
    // that values derived from them are recomputed per tile instead of being
    // hoisted out of the tile loop, where they would hold registers for good.
    int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wy = (wave & 1) * 128, wx = (wave >> 1) * 128;   // this wave's quadrant (m, n)
    int gq = lane >> 4, li = lane & 15;
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        gq = lane >> 4;
        li = lane & 15;
    };
    constexpr bool F8 = (DT == MXQ_DTYPE_MXFP8_E4M3);
    constexpr int ESZ = F8 ? 1 : 2;
    constexpr int OSZ = OUT == MXQ_DTYPE_F32 ? 4 : 2;
    constexpr bool XKS = (MODE != MODE_NT);   // X (N side) K-strided
    constexpr bool YKS = (MODE == MODE_TN);   // Y (M side) K-strided

    if (tid == 0) sa = a;
    // row pitches in bytes (each below 2^23)
    const int lda = (int)(a.A.ld * ESZ), ldb = (int)(a.B.ld * ESZ);
    const int ldsa = (int)a.A.ld_scales, ldsb = (int)a.B.ld_scales;

    // ---- this workgroup's items
    int ntm = ntm_ub;
    if constexpr (TAB) {
        build_group_tables<MODE>(a, rs, tab, wsum, ntm_ub, tid, lane, wave);   // ends with a barrier
        if constexpr (MODE != MODE_TN) ntm = tab[a.G];
    } else {
        __syncthreads();
    }
    const int nitems = (MODE == MODE_TN ? (int)a.G : 1) * ntm * ntn;
    const int nj = gridDim.x / kXCD;
    const int per = (nitems + kXCD - 1) / kXCD;
    const int xcd = blockIdx.x % kXCD;
    const int lo = xcd * per + blockIdx.x / kXCD;
    const int hi = (xcd + 1) * per < nitems ? (xcd + 1) * per : nitems;

    // tile of work item `item` (false: an m tile past its group's rows)
    auto describe = [&](int item, Tile &T) -> bool {
        const uint8_t *A = static_cast<const uint8_t *>(sa.A.data);
        const uint8_t *B = static_cast<const uint8_t *>(sa.B.data);
        int64_t m0, n0, r0, r1, g;
        if constexpr (MODE == MODE_TN) {
            const int per_g = ntm * ntn;
            g = item / per_g;
            const int rem = item - (int)g * per_g;
            m0 = (int64_t)(rem / ntn) * BT;
            n0 = (int64_t)(rem % ntn) * BT;
            int64_t blk0;
            if constexpr (TAB) {
                r0 = rs[g];
                r1 = rs[g + 1];
                blk0 = tab[g];
            } else {
                r0 = sa.row_off[g];
                r1 = sa.row_off[g + 1];
                r1 = r1 > sa.rows ? sa.rows : r1;
                r0 = r0 < 0 ? 0 : r0;
                blk0 = sa.block_off != nullptr ? sa.block_off[g] : 0;
            }
            r1 = r1 > r0 ? r1 : r0;
            T.x = B + r0 * ldb + n0;
            T.y = A + r0 * lda + m0;
            T.xs = sa.B.scales + blk0 * ldsb + n0;
            T.ys = sa.A.scales + blk0 * ldsa + m0;
            T.o = static_cast<uint8_t *>(sa.out) + (g * sa.out_gstride + m0 * sa.ld_out + n0) * OSZ;
            T.yv = (int)(sa.M - m0 < BT ? sa.M - m0 : BT);
            T.kext = (int)(r1 - r0);
            T.nblk = (T.kext + 31) / 32;
            T.ksteps = (T.kext + 127) / 128;
        } else {
            int mt, nt;
            raster(item, ntm, ntn, mt, nt);
            int64_t before;
            if constexpr (TAB) {
                g = table_group(tab, (int)sa.G, mt, lane);
                before = tab[g];
                r0 = rs[g];
                r1 = rs[g + 1];
                r1 = r1 > r0 ? r1 : r0;
            } else {
                g = scan_group(sa, mt, ntm_ub, lane, before);
                if (__builtin_amdgcn_readfirstlane((int)(g < 0))) return false;
                group_rows(sa, g, r0, r1);
            }
            m0 = r0 + (mt - before) * BT;
            if (__builtin_amdgcn_readfirstlane((int)!(m0 < r1))) return false;
            n0 = (int64_t)nt * BT;
            if constexpr (MODE == MODE_NT) {
                T.x = B + g * sa.B.gstride * ESZ + n0 * ldb;
                T.xs = sa.B.scales + g * sa.B.scale_gstride + n0 * ldsb;
            } else {
                T.x = B + g * sa.B.gstride + n0;
                T.xs = sa.B.scales + g * sa.B.scale_gstride + n0;
            }
            T.y = A + m0 * lda;
            T.ys = sa.A.scales + m0 * ldsa;
            T.o = static_cast<uint8_t *>(sa.out) + (m0 * sa.ld_out + n0) * OSZ;
            T.yv = (int)(r1 - m0 < BT ? r1 - m0 : BT);
            T.kext = (int)(sa.K * ESZ);
            T.nblk = (int)((sa.K + 31) / 32);
            T.ksteps = (T.kext + BK - 1) / BK;
        }
        T.xv = (int)(sa.N - n0 < BT ? sa.N - n0 : BT);
        T.item = item;
        T.x = reinterpret_cast<const uint8_t *>(uni64(reinterpret_cast<int64_t>(T.x)));
        T.y = reinterpret_cast<const uint8_t *>(uni64(reinterpret_cast<int64_t>(T.y)));
        T.xs = reinterpret_cast<const uint8_t *>(uni64(reinterpret_cast<int64_t>(T.xs)));
        T.ys = reinterpret_cast<const uint8_t *>(uni64(reinterpret_cast<int64_t>(T.ys)));
        T.o = reinterpret_cast<uint8_t *>(uni64(reinterpret_cast<int64_t>(T.o)));
        T.xv = __builtin_amdgcn_readfirstlane(T.xv);
        T.yv = __builtin_amdgcn_readfirstlane(T.yv);
        T.kext = __builtin_amdgcn_readfirstlane(T.kext);
        T.nblk = __builtin_amdgcn_readfirstlane(T.nblk);
        T.ksteps = __builtin_amdgcn_readfirstlane(T.ksteps);
        T.valid = 1;
        return true;
    };
    auto next_tile = [&](int from) {
        Tile T{};
        for (int item = from; item < hi; item += nj)
            if (describe(item, T)) return T;
        T.valid = 0;
        T.ksteps = 0;
        return T;
    };

    auto src_x = [&](const Tile &T) {
        return XKS ? Src{T.x, ldb, T.kext, T.xv} : Src{T.x, ldb, T.kext, T.xv};
    };
    auto src_y = [&](const Tile &T) { return Src{T.y, lda, T.kext, T.yv}; };

    // stage s of tile T -> stage buffer st: data tiles straight to LDS, scales
    // by 4-byte LDS loads (or, rarely, bytes through registers)
    auto issue = [&](const Tile &T, int s, uint8_t *st) {
        if constexpr (XKS) stage_ks(src_x(T), s, st, wave, lane);
        else stage_kc(src_x(T), s, st, wave, lane);
        if constexpr (YKS) stage_ks(src_y(T), s, st + OPB, wave, lane);
        else stage_kc(src_y(T), s, st + OPB, wave, lane);
        if constexpr (F8) {
            if constexpr (MODE == MODE_NT) {
                const RowScales xr{T.xs, ldsb, T.nblk, T.xv};
                if (!rowscale_dma(xr, s, tid, st + 2 * OPB))
                    *reinterpret_cast<uint32_t *>(st + 2 * OPB + 4 * tid) = rowscale_word(rowscale_load(xr, s, tid));
            } else if (wave == 0) {
                stage_colscales(ColScales{T.xs, ldsb, T.nblk, T.xv}, s, st + 2 * OPB, lane);
            }
            if constexpr (MODE == MODE_TN) {
                if (wave == 1) stage_colscales(ColScales{T.ys, ldsa, T.nblk, T.yv}, s, st + 2 * OPB + SCB, lane);
            } else {
                const RowScales yr{T.ys, ldsa, T.nblk, T.yv};
                if (!rowscale_dma(yr, s, tid, st + 2 * OPB + SCB))
                    *reinterpret_cast<uint32_t *>(st + 2 * OPB + SCB + 4 * tid) = rowscale_word(rowscale_load(yr, s, tid));
            }
        }
    };
    // always exactly two loads per thread (out of range past the tile's steps),
    // so that a step's wait can keep exactly two loads in flight
    auto touch = [&](const Tile &T, int s) {
        const bool live = T.valid && s < T.ksteps;
        if constexpr (XKS) touch_ks(src_x(T), s, tid, junk[wave], live);
        else touch_kc(src_x(T), s, tid, junk[wave], live);
        if constexpr (YKS) touch_ks(src_y(T), s, tid, junk[wave], live);
        else touch_kc(src_y(T), s, tid, junk[wave], live);
    };

    f32x4_t acc[8][8];
#pragma unroll
    for (int x = 0; x < 8; x++)
#pragma unroll
        for (int y = 0; y < 8; y++) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](const uint8_t *st) {
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
    };

    // ---- epilogue: lane holds C[m][n .. n+3] for m = wy + 16y + li, n = wx + 16x + 4gq;
    // stored straight from registers with buffer stores (one 32-bit row offset
    // per y, the column as the immediate offset; elements outside the tile go
    // out of range and are dropped).  A row's 256 bytes of one wave leave in
    // eight 32-byte pieces, which meet again in L2.
    const int ldo = (int)(a.ld_out * OSZ);   // output row pitch in bytes (< 2^23)
    const bool accumulate = a.accumulate != 0;
    auto epilogue = [&](const Tile &T, uint8_t *stg) {
        const __amdgpu_buffer_rsrc_t ro = rsrc(T.o, 0x7FFFFFF0);
        if constexpr (OUT == MXQ_DTYPE_BF16) {
            // Through LDS, so that each output row leaves as 512 contiguous
            // bytes (16-byte nontemporal stores, 32 lanes per row): the stage
            // buffer the last step read from holds half the tile, 128 rows x
            // 512 B with 16-byte chunk c of row m at c ^ (m & 31); the two
            // waves holding rows [128h, 128h + 128) (waves h and h + 2) write
            // half h, then all four store it.
            typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int h = 0; h < 2; h++) {
                step_barrier<63>();   // everyone is done reading stg (last step's fragments, or half h - 1)
                if ((wave & 1) == h) {
#pragma unroll
                    for (int y = 0; y < 8; y++) {
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int x = 0; x < 8; x++) asm volatile("" : "+a"(acc[x][y]));
                        const int m = 16 * y + li;
#pragma unroll
                        for (int x = 0; x < 8; x++) {
                            const int n = wx + 16 * x + 4 * gq;
                            const f32x4_t v = acc[x][y];
                            bf16x4_t b;
                            b.x = (__bf16)v.x; b.y = (__bf16)v.y; b.z = (__bf16)v.z; b.w = (__bf16)v.w;
                            *reinterpret_cast<bf16x4_t *>(stg + m * 512 + 16 * ((n >> 3) ^ (m & 31)) + 8 * ((n >> 2) & 1)) = b;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                step_barrier<63>();   // half h is in LDS
#pragma unroll
                for (int j = 0; j < 16; j++) {
                    const int q = j * NTHR + tid;
                    const int m = q >> 5, c = q & 31;
                    const int row = 128 * h + m;
                    const u32x4_t v = *reinterpret_cast<const u32x4_t *>(stg + m * 512 + 16 * (c ^ (m & 31)));
                    const uint32_t off = (row < T.yv) & (8 * c < T.xv) ? (uint32_t)(row * opaque(ldo) + 16 * c) : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(v, ro, off, 0, 2);   // nt
                }
            }
        } else {
            // fp32: straight from the accumulators (a row's 256 bytes of one
            // wave in eight 64-byte pieces)
#pragma unroll
            for (int y = 0; y < 8; y++) {
                // one row of fragments at a time, so that only its accumulators
                // are copied out of the matrix registers at once
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int x = 0; x < 8; x++) asm volatile("" : "+a"(acc[x][y]));
                const int ml = wy + 16 * y + li;
                const uint32_t row = ml < T.yv ? (uint32_t)(ml * opaque(ldo) + (wx + 4 * gq) * OSZ) : kOOB;
#pragma unroll
                for (int x = 0; x < 8; x++) {
                    // columns past N (last n tile only) go out of range too
                    const uint32_t off = wx + 16 * x + 4 * gq < T.xv ? row + 16 * x * OSZ : kOOB;
                    f32x4_t w = acc[x][y];
                    if (accumulate) w += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), ro, off, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // vector memory operations each wave's epilogue issues (loads it waits
    // for itself aside): 2 x 16 row stores (bf16), 64 stores (fp32)
    constexpr int kEpiOps = OUT == MXQ_DTYPE_BF16 ? 32 : 64;
    constexpr int kFirstWait = 2 + kEpiOps < 63 ? 2 + kEpiOps : 63;

    Tile cur = next_tile(lo);
    if (!cur.valid) return;
    int gs = 0;   // steps this workgroup has run: step gs computes from stage buffer gs & 1
    if (cur.ksteps > 0) issue(cur, 0, smem);
    touch(cur, 1);
    // Vector memory operations of a wave complete in issue order on this
    // target, loads and stores alike (the compiler's wait counts rely on the
    // same), so a step's wait may leave every later operation in flight: the
    // 2 warm-up loads, and after a tile whose last step prefetched this one,
    // also the previous tile's kEpiOps epilogue stores (vmcnt saturates at 63,
    // which still covers the stage when more operations follow it).
    bool after_epilogue = false;
    for (;;) {
        refresh_lane();
        tnext[wave] = next_tile(cur.item + nj);
        for (int s = 0; s < cur.ksteps; s++, gs++) {
            // (the condition is opaque so that the compiler does not peel the
            // first step into a second copy of the loop body)
            if (opaque(__builtin_amdgcn_readfirstlane((int)((s == 0) & after_epilogue))))
                // vmcnt(kFirstWait) expcnt(7) lgkmcnt(15)
                __builtin_amdgcn_s_waitcnt((kFirstWait & 15) | ((kFirstWait >> 4) << 14) | 0x0F70);   // vmcnt(63) expcnt(7) lgkmcnt(15)
            else __builtin_amdgcn_s_waitcnt(0x0F72);                                    // vmcnt(2) expcnt(7) lgkmcnt(15)
            step_barrier<63>();   // everyone's loads have landed, and step gs - 1's reads are done
            uint8_t *nb = smem + ((gs + 1) & 1) * STAGE;
            if (s + 2 < cur.ksteps) {
                issue(cur, s + 1, nb);
                touch(cur, s + 2);
            } else {
                const Tile nxt = tnext[wave];
                if (s + 1 < cur.ksteps) issue(cur, s + 1, nb);
                else if (nxt.ksteps > 0) issue(nxt, 0, nb);
                touch(nxt, s + 2 - cur.ksteps);
            }
            compute(smem + (gs & 1) * STAGE);
        }
        // the stage buffer the last step read from (or, after a tile without
        // steps, the one no load is headed for)
        epilogue(cur, smem + ((gs + 1) & 1) * STAGE);
        const Tile nxt = tnext[wave];
        if (!nxt.valid) break;
        after_epilogue = cur.ksteps > 0;
        if (cur.ksteps == 0 && nxt.ksteps > 0) {
            // nothing prefetched the next tile; buffer gs & 1 was last read by
            // step gs - 2, which every wave finished before step gs - 1's barrier
            issue(nxt, 0, smem + (gs & 1) * STAGE);
            touch(nxt, 1);
        }
#pragma unroll
        for (int x = 0; x < 8; x++)
#pragma unroll
            for (int y = 0; y < 8; y++) acc[x][y] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        cur = nxt;
    }
}

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
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
    // one workgroup per CU (the LDS of a stage pair fills a CU), a multiple of
    // the XCD count, never more than the work
    int64_t grid = cu_count();
    if (g.max_workgroups > 0 && g.max_workgroups < grid) grid = g.max_workgroups;
    grid = grid / kXCD * kXCD;
    if (grid < kXCD) grid = kXCD;
    const int64_t need = (nwork + kXCD - 1) / kXCD * kXCD;
    if (need < grid) grid = need;
    if (g.G <= kTab)
        hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true>), dim3((unsigned)grid), dim3(NTHR), 0, stream, g,
                           (int)ntn, (int)ntm);
    else
        hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false>), dim3((unsigned)grid), dim3(NTHR), 0, stream, g,
                           (int)ntn, (int)ntm);
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
    g.max_workgroups = in.max_workgroups;
    g.noop = false;
    if (in.mode < MXQ_GEMM_NT || in.mode > MXQ_GEMM_TN) { err = "unknown GEMM mode"; return MXQ_ERR_SHAPE; }
    if (in.G < 1 || in.G > (int64_t(1) << 24)) { err = "G must be in [1, 2^24]"; return MXQ_ERR_SHAPE; }
    if (in.row_off == nullptr) { err = "row_off is required"; return MXQ_ERR_NULL; }
    if (in.M < 0 || in.N < 0 || in.K < 0 || in.rows < 0) { err = "negative size"; return MXQ_ERR_SHAPE; }
    if (in.max_workgroups < 0) { err = "max_workgroups must be >= 0"; return MXQ_ERR_SHAPE; }
    if (in.M >= (int64_t(1) << 31) || in.rows >= (int64_t(1) << 31)) { err = "M and rows must stay below 2^31"; return MXQ_ERR_OVERFLOW; }
    if (in.ld_out * (in.out_dtype == MXQ_DTYPE_F32 ? 4 : 2) >= (int64_t(1) << 23)) { err = "the output row pitch must stay below 2^23 bytes"; return MXQ_ERR_OVERFLOW; }
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
