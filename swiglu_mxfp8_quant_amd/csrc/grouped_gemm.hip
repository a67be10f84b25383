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
//     128 x 128 quadrant as 4 x 4 MFMA tiles of 32 x 32 (256 fp32 accumulators
//     per lane, in the matrix registers).  MXFP8 uses
//     v_mfma_scale_f32_32x32x64_f8f6f4: lane 32g + i carries row i's
//     contraction bytes [16g, 16g + 16) and [32 + 16g, 48 + 16g) and the E8M0
//     scale of row i's 32-element block g, so the block scales are applied
//     inside the matrix core.  bf16 uses v_mfma_f32_32x32x16_bf16.
//   * A stage is 64 contraction bytes of the tile's 256 rows per operand
//     (16 KB).  Operand tiles go from memory straight into LDS (buffer_load
//     ... lds, 16 bytes per lane).  Each lane's offsets are worked out once
//     per tile; lanes whose rows, columns or contraction tail lie outside the
//     operand take an offset past the resource's range, which the hardware
//     turns into zeros without a branch, so a stage's data load is three
//     instructions.
//   * Four stage buffers.  Stage c is computed from registers while stage
//     c + 1 sits in LDS and stages c + 2 .. c + 4 load: after two of stage c's
//     MFMAs a wave waits for stage c + 1, passes the step's barrier, then
//     alternates the remaining MFMAs with the reads of stage c + 1's fragments
//     (into a second register set) and with the loads of stage c + 4 (into
//     stage c's buffer).
//   * LDS tiles are XOR-swizzled at 16-byte granularity (chunk c of row r at
//     c ^ ((r >> 2) & 3) for 64-byte rows, c ^ (k & 15) for the 256-byte
//     contraction rows of K-strided operands), which keeps the fragment reads
//     and the transposed reads conflict-free.
//   * Operands whose contraction index is strided in memory (the dgrad weight
//     and both wgrad operands) are staged as they lie ([k][column] tiles) and
//     read with ds_read_b64_tr_b8, which transposes 16 lanes' 8-byte rows.
//   * The row scales of K-contiguous MXFP8 operands come through a two-slot
//     ring, 16 bytes per row per 8 stages, instead of a load per stage.
//   * The output tile is computed transposed (the MFMA's first operand is the
//     N side), so every lane owns 4 consecutive output columns of one row; a
//     bf16 tile is staged through LDS so that each output row leaves as 512
//     contiguous bytes, fp32 goes straight from the accumulators.
//   * A bf16 NT launch can carry the row-scaled SwiGLU in its epilogue (FC1
//     with the gate / up rows of its weight interleaved in blocks of 128): the
//     staged quarter tiles that leave as the bf16 output are also turned into
//     the MXFP8 activation, rowwise and / or colwise (page "Activation +
//     GroupedLinear Fusion for MOE and other MOE optimizations", discussion:
//     the activation and its quantization fused with the grouped GEMM).
//   * Group boundaries come from the device offsets only.  Each workgroup of
//     an M-grouped launch first builds the groups' m-tile prefix sums in LDS
//     (for up to 1024 groups; beyond that every lookup scans the offsets), so
//     the exact tile count is known on the device and a tile's group is two
//     wave-wide LDS probes away.
//   * The grid is persistent: one workgroup per CU, each looping over its
//     share of the tiles.  Each XCD takes a contiguous range of tiles (one
//     expert's tiles share that XCD's L2).  The load side walks the same tile
//     sequence as the compute side, a few stages ahead, so consecutive tiles
//     overlap.  K-grouped launches whose static ranges would be unbalanced
//     (skewed group sizes) take their tiles largest group first from a
//     counter in the caller's workspace instead.
#include "gemm_internal.h"
#include "act_math.h"

#include <string>
#include <type_traits>

namespace mxq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2;

constexpr int BT = 256;            // tile rows on each side (X = output n, Y = output m)
constexpr int BK = 64;             // contraction bytes per step (one stage)
constexpr int NBUF = 4;            // stage buffers: one computing, three loading
constexpr int NTHR = 256;
constexpr int OPB = BT * BK;       // bytes of one operand's stage tile (either layout)
constexpr int SCB = 1024;          // bytes of one operand's per-stage scales
constexpr int RGS = 8;             // stages per scale-ring group (16 E8M0 bytes per row)
constexpr int RSLOT = BT * 16;     // bytes of one operand's ring slot
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

// Buffer loads straight into LDS (lane l's bytes land at M0 + size * l).
// They are written out here rather than through the compiler's builtin: the
// compiler would otherwise wait for every such load in flight before any LDS
// access it cannot tell apart from their destinations (which would serialize
// the stage pipeline), while the kernel orders them itself with its explicit
// vmcnt waits and barriers.  They have no register results.  They read M0
// (the LDS address), an input the compiler writes before each, and the
// resource from SGPRs.  The compiler cannot see that these statements hold a
// vector-memory instruction, so it does not keep its distance from them
// either: a vector instruction that writes an SGPR (a readfirstlane, an SGPR
// spill reload) needs five wait states before a vector-memory instruction
// reads that SGPR, and each statement pads itself to five.
__device__ __forceinline__ i32x4_t rsrc4(const uint8_t *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7FFFFFF0ll ? 0x7FFFFFF0 : (int)bytes);
    const uint64_t b = (uint64_t)uni64(reinterpret_cast<int64_t>(base));
    return i32x4_t{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), (int)__builtin_amdgcn_readfirstlane(n), 0x00020000};
}

// A resource from `base` on whose range checks nothing relies: every load
// through it either carries an offset its own bounds checks have admitted or
// kOOB.
__device__ __forceinline__ i32x4_t rsrc_open(const uint8_t *base) {
    const uint64_t b = (uint64_t)uni64(reinterpret_cast<int64_t>(base));
    return i32x4_t{(int)(uint32_t)b, (int)(uint32_t)(b >> 32), 0x7FFFFFF0, 0x00020000};
}

// LDS byte address of a generic pointer into LDS: the shared aperture is
// 4 GB aligned, so it is the pointer's low word.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)p);
}

__device__ __forceinline__ void to_lds(const i32x4_t &r, uint8_t *dst, uint32_t off) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr(dst))
                 : "memory");
}

__device__ __forceinline__ void to_lds4(const i32x4_t &r, uint8_t *dst, uint32_t off) {
    asm volatile("s_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_addr(dst))
                 : "memory");
}

// 16 bytes per lane to LDS address `dst`, from offset `off` in the lanes of
// `mask` and from kOOB in the others.
__device__ __forceinline__ void to_lds_sel(const i32x4_t &r, uint32_t dst, uint32_t off, uint64_t mask, uint32_t oob) {
    uint32_t t;
    asm volatile("v_cndmask_b32_e64 %0, %1, %2, %3\n\ts_nop 3\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
                 : "=&v"(t)
                 : "v"(oob), "v"(off), "s"(mask), "s"(r), "{m0}"(dst)
                 : "memory");
}

// One operand's view for staging.  K-contiguous: tile rows are output rows,
// 64 contraction bytes each per step.  K-strided: tile rows are contraction
// rows, 256 output columns (bytes) each.
struct Src {
    const uint8_t *base;   // tile origin (row 0 / contraction row 0, first column)
    int pitch;             // bytes between rows in memory (< 2^23)
    int kext;              // K-contiguous: contraction bytes per row; K-strided: contraction rows
    int valid;             // K-contiguous: valid tile rows; K-strided: valid column bytes
};

// Every stage issue below is a fixed number of load instructions per wave
// (4 + 4 data, 2 scale for MXFP8), whether or not it carries data: loads
// with `live` false or outside the operand go out of range (no memory
// access; zeros land in LDS).  The step waits count on that.
//
// The data loads of a wave, load j of 4 per operand, fill the 1 KB blocks
// 4w + j of the operand's stage tile.  Their per-lane offsets from the tile
// origin do not depend on the stage; they are worked out once per tile (kOOB
// for rows or columns outside the tile, and for every lane of a tile that
// carries nothing), and each stage adds its contraction offset to the
// resource's base and masks out what lies past the contraction.
struct Feed {
    uint32_t v[4];
};

// K-contiguous stage s -> LDS [256 rows][64 B], chunk c of row r at c ^ ((r >> 2) & 3).
// Lane l of load j covers row 16 (4w + j) + l / 4, whose swizzle is (l >> 4) & 3.
__device__ __forceinline__ int kc_chunk(int lane) { return (lane & 3) ^ ((lane >> 4) & 3); }

__device__ __forceinline__ Feed feed_kc(const Src &o, bool live, int wave, int lane) {
    Feed f;
    const int c = kc_chunk(lane);
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const int row = 16 * (4 * wave + j) + (lane >> 2);
        f.v[j] = (live & (row < o.valid)) ? (uint32_t)(row * o.pitch + 16 * c) : kOOB;
    }
    return f;
}

// `sb`: the operand's origin advanced to stage s (o.base + s * BK)
template <int J>
__device__ __forceinline__ void stage_kc(const Src &o, const uint8_t *sb, const Feed &f, int s, uint32_t dst, int lane,
                                         uint32_t oob) {
    const int k0 = s * BK;
    const uint64_t in_k = __builtin_amdgcn_ballot_w64(16 * kc_chunk(lane) < o.kext - k0);
    to_lds_sel(rsrc_open(sb), dst + 1024 * J, f.v[J], in_k, oob);
}

// K-strided stage s -> LDS, 256 output columns by 64 contraction bytes' worth
// of rows: fp8 [64 contraction rows][256 B], chunk c of row k at c ^ (k & 15);
// bf16 [32 contraction rows][512 B], chunk c of row k at c ^ 4 (k & 3).
// Lane l of load j covers contraction row 4 (4w + j) + l / 16 (fp8) or
// 2 (4w + j) + l / 32 (bf16).
template <int ESZ>
__device__ __forceinline__ Feed feed_ks(const Src &o, bool live, int wave, int lane) {
    Feed f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        int kr, c;
        if constexpr (ESZ == 1) {
            kr = 4 * (4 * wave + j) + (lane >> 4);
            c = (lane & 15) ^ (kr & 15);
        } else {
            kr = 2 * (4 * wave + j) + (lane >> 5);
            c = (lane & 31) ^ (4 * (kr & 3));
        }
        f.v[j] = (live & (16 * c < o.valid)) ? (uint32_t)(kr * o.pitch + 16 * c) : kOOB;
    }
    return f;
}

// `sb`: the operand's origin advanced to stage s (o.base + s * (BK / ESZ) * o.pitch)
template <int J, int ESZ>
__device__ __forceinline__ void stage_ks(const Src &o, const uint8_t *sb, const Feed &f, int s, uint32_t dst, int wave,
                                         int lane, uint32_t oob) {
    const int kr0 = s * (BK / ESZ);
    const bool in = ESZ == 1 ? (lane >> 4) < o.kext - kr0 - 4 * (4 * wave + J)
                             : (lane >> 5) < o.kext - kr0 - 2 * (4 * wave + J);
    const uint64_t in_k = __builtin_amdgcn_ballot_w64(in);
    to_lds_sel(rsrc_open(sb), dst + 1024 * J, f.v[J], in_k, oob);
}

// Rowwise E8M0 scales of a K-contiguous operand.  Stage s uses blocks 2s and
// 2s + 1, which sit in the aligned 4-byte word s / 2 of the row; thread t
// puts row t's word into LDS [row][4] (one 4-byte LDS load per thread).
struct RowScales {
    const uint8_t *base;   // scales of tile row 0
    int ld;                // bytes between rows (< 2^23)
    int nblk;              // blocks per row
    int valid;             // valid tile rows
};

// One load instruction per wave.  The word goes straight to LDS when it lies
// inside the row (ld % 4 == 0 and 4 blocks left); otherwise (a ragged last
// word) its bytes are read one by one through registers and stored, and an
// out-of-range load into `junk` keeps the instruction count.
// WORDS: every row's words lie inside it (ld % 4 == 0, blocks per row a
// multiple of 4), decided per launch so that the common path has no branch.
// (Touching one cache line per row for two stages' scales costs the address
// unit as much as a whole 1 KB data load; the scale ring in the kernel loads
// 16 bytes per row once per 8 stages instead, where the shape allows.)
template <bool WORDS>
__device__ __forceinline__ void stage_rowscales(const RowScales &sc, int s, int t, uint8_t *dst, uint8_t *junk,
                                                bool live) {
    const int w = s >> 1;
    const i32x4_t r4 = rsrc4(sc.base, (int64_t)sc.valid * sc.ld);
    if (WORDS || !live || ((sc.ld % 4 == 0) & (4 * w + 4 <= sc.nblk))) {
        to_lds4(r4, dst + 4 * (t & ~63), (live & (t < sc.valid)) ? (uint32_t)(t * sc.ld + 4 * w) : kOOB);
        return;
    }
    const __amdgpu_buffer_rsrc_t r = rsrc(sc.base, (int64_t)sc.valid * sc.ld);
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const bool ok = (t < sc.valid) & (4 * w + b < sc.nblk);
        word |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, ok ? (uint32_t)(t * sc.ld + 4 * w + b) : kOOB, 0, 0)
                << (8 * b);
    }
    *reinterpret_cast<uint32_t *>(dst + 4 * t) = word;
    to_lds4(r4, junk, kOOB);
}

// Colwise E8M0 scales of a K-strided operand, stage s: block rows 2s, 2s + 1
// x 256 columns -> LDS [2][256] (lanes 32-63 fill the next 512 bytes with
// zeros).  One load instruction per wave; only wave `owner` carries data,
// the others load out of range into `junk`.
struct ColScales {
    const uint8_t *base;   // block row 0, tile column 0
    int ld;                // bytes between block rows (< 2^23)
    int nblk;              // block rows of the contraction
    int valid;             // valid column bytes
};

// `sb`: sc.base advanced to stage s (block row 2s)
__device__ __forceinline__ void stage_colscales(const ColScales &sc, const uint8_t *sb, int s, uint8_t *dst, uint8_t *junk,
                                                int wave, int owner, int lane, bool live) {
    const int b0 = 2 * s;
    const i32x4_t r = rsrc_open(sb);
    const int b = lane >> 4, c = lane & 15;
    const bool mine = wave == owner;
    const bool ok = live & mine & (lane < 32) & (b0 + b < sc.nblk) & (16 * c < sc.valid);
    to_lds(r, mine ? dst : junk, ok ? (uint32_t)(b * sc.ld + 16 * c) : kOOB);
}

// ------------------------------------------------------------------ fragments
//
// The scaled fp8 32x32x64 MFMA: lane 32g + i carries row i's contraction
// bytes [16g, 16g + 16) (E8M0 block 0) and [32 + 16g, 48 + 16g) (block 1),
// and the scale of row i's block g.  Any assignment of bytes to contraction
// positions works as long as both operands use the same one and every byte
// sits in its own block.  bf16 32x32x16: lane 32g + i carries row i's
// elements [8g, 8g + 8) of the 16.  The 32x32 fp32 result: lane 32g + j holds
// C[8q + 4g + r][j] in its register 4q + r.

// fp8, K-strided tile: the same 32 bytes for column col0 + m (col0 a multiple
// of 16) via transposed reads: lane m of the 16-lane group points at
// contraction row k0 + m/2, bytes col0 + 8 (m % 2) .. + 8, and receives 8
// consecutive contraction bytes of column col0 + m.
__device__ __forceinline__ i32x2_t tr8(const uint8_t *t, int k0, int col0, int m) {
    const int kr = k0 + (m >> 1);
    const uint8_t *p = t + kr * 256 + 16 * ((col0 >> 4) ^ (kr & 15)) + 8 * (m & 1);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)p);
}

__device__ __forceinline__ i32x8_t frag_ks_f8(const uint8_t *t, int col0, int g, int m) {
    const i32x2_t a = tr8(t, 16 * g, col0, m);
    const i32x2_t b = tr8(t, 16 * g + 8, col0, m);
    const i32x2_t c = tr8(t, 32 + 16 * g, col0, m);
    const i32x2_t d = tr8(t, 40 + 16 * g, col0, m);
    return i32x8_t{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// bf16, K-strided tile ([32 contraction rows][256 columns], 512-byte rows):
// ds_read_b64_tr_b16 moves a 4-row x 16-column block of 16-bit elements
// between the 16 lanes of a group: lane m points at row k0 + m/4, bytes
// 8 (m % 4) .. + 8 of the block's 32, and receives the 4 elements of column
// col0 + m in rows k0 .. k0 + 3 (checked on the device with a probe of
// known values).  The swizzle 4 (k & 3) puts the 4 rows' 32-byte pieces of
// one group, and those of the group 16 columns on, in 8 different 32-byte
// bank slots.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
__device__ __forceinline__ i32x2_t tr16(const uint8_t *t, int k0, int col0, int m) {
    const int kr = k0 + (m >> 2);
    const int chunk = (col0 >> 3) + ((m & 3) >> 1);
    const uint8_t *p = t + kr * 512 + 16 * (chunk ^ (4 * (kr & 3))) + 8 * (m & 1);
    return __builtin_bit_cast(i32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}

// The bf16 32x32x16 operand of column col0 + m (col0 a multiple of 16):
// contraction elements 16 kk + 8 g .. + 8 of the stage.
__device__ __forceinline__ bf16x8_t frag_ks_bf16(const uint8_t *t, int col0, int kk, int g, int m) {
    const i32x2_t a = tr16(t, 16 * kk + 8 * g, col0, m);
    const i32x2_t b = tr16(t, 16 * kk + 8 * g + 4, col0, m);
    return __builtin_bit_cast(bf16x8_t, i32x4_t{a.x, a.y, b.x, b.y});
}

// One stage's fragments of a wave's 128 x 128 quadrant: MXFP8, 4 + 4 operand
// fragments with their E8M0 scale bytes; bf16, the same for each of the two
// 16-element halves of the stage.
struct FragsF8 {
    i32x8_t fx[4], fy[4];
    int sx[4], sy[4];
    int in_k;   // ring scales: this lane's block lies inside the contraction (else the unit scale applies)
};
struct FragsBF16 {
    bf16x8_t fx[2][4], fy[2][4];
};

template <int I>
using IC = std::integral_constant<int, I>;

// f(IC<I>{}) for I = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
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
constexpr int kTab = 1024;

// K-grouped launches with up to kDynG groups can take their tiles in a
// dynamic largest-first order (see the kernel); an epilogue counts as this
// many contraction steps when the schedules are compared.
constexpr int kDynG = 256;
constexpr int kEpiCost = 2;
constexpr int kQueue = 16;   // entries of a workgroup's queue of taken tiles
constexpr int kTake0 = 7;    // tiles a workgroup is dealt before it takes any

// Sets the dynamic tile counter of a K-grouped launch to zero (a kernel, not
// a memset, so that the pair can be captured in a graph).
__global__ void sched_reset(int *counter) {
    if (threadIdx.x == 0) counter[0] = 0;
}

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
// precomputed).
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
    // fused epilogue only: the tile's first output row and column, and the
    // colwise scale row of its first 32-row block (tiles start at a group's
    // first row plus a multiple of 256, so their 32-row blocks are the group's)
    int64_t m0, n0, srow;
};

// A persistent grid (one workgroup per CU at most): workgroup j of XCD x runs
// items x * per + j, + nj, ... of that XCD's contiguous range.  Four stage
// buffers: while one stage computes from registers, the next one is read from
// LDS and the three after it load; the load side runs ahead across tile
// boundaries (it walks the same tile sequence, skipping tiles without steps),
// so a tile's first stages are in LDS when its first step starts.  TAB: the
// groups' offsets and m-tile prefix are kept in LDS (G <= kTab), else every
// lookup reads the offsets.
// SC, the row scales' path (MXFP8 NT/NN): 0 bytes per stage through
// registers, 1 a 4-byte word per row per stage, 2 the scale ring: 16 bytes per
// row per 8-stage group into one of two LDS slots (used when every group
// spans at least 3 stages: a group's slot is refilled when the load side
// issues the first stage of the group after next, which happens after the
// barrier that follows the last read of that slot's earlier group; blocks
// past the contraction take the unit scale in registers, so bytes read past a
// row's end are harmless).
// EPI (bf16 NT with a bf16 output only): 0, or the fused SwiGLU epilogue
// (1 plain, 2 clamped; see fused_act below).
template <int MODE, int DT, int OUT, bool TAB, int SC, int EPI = 0>
__global__ void __launch_bounds__(NTHR) gemm_kernel(GemmArgs a, int ntn, int ntm_ub) {
    static_assert(EPI == 0 || (MODE == MODE_NT && DT == MXQ_DTYPE_BF16 && OUT == MXQ_DTYPE_BF16),
                  "the fused epilogue is built for bf16 NT launches with a bf16 output");
    constexpr bool F8_ = (DT == MXQ_DTYPE_MXFP8_E4M3);
    constexpr bool XKS_ = (MODE != MODE_NT), YKS_ = (MODE == MODE_TN);
    constexpr bool XRING = F8_ && !XKS_ && SC == 2, YRING = F8_ && !YKS_ && SC == 2;
    constexpr int XSB = F8_ && !XRING ? SCB : 0, YSB = F8_ && !YRING ? SCB : 0;   // per-stage scale bytes
    constexpr int STAGE = 2 * OPB + XSB + YSB;
    constexpr int NRING = (XRING ? 1 : 0) + (YRING ? 1 : 0);
    static_assert(STAGE >= 64 * 512, "the epilogue stages a quarter tile in one stage buffer");
    __shared__ __attribute__((aligned(16))) uint8_t smem[NBUF * STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t ring[NRING ? NRING * 2 * RSLOT : 16];
    __shared__ __attribute__((aligned(16))) uint8_t junk[1024];   // sink of the loads that carry nothing
    __shared__ int tab[TAB ? kTab + 1 : 1];
    __shared__ int rs[TAB ? kTab + 1 : 1];
    __shared__ int wsum[4];
    constexpr bool DYN = MODE == MODE_TN && TAB;   // the dynamic order is available
    __shared__ int gsteps[DYN ? kDynG : 1];   // contraction steps per group
    __shared__ int gord[DYN ? kDynG : 1];     // groups by steps, largest first
    __shared__ int dq[DYN ? kQueue : 1];      // taken tiles, in order
    __shared__ int64_t red[8];
    // the arguments that only the per-tile lookup reads live in LDS, so that
    // they do not hold scalar registers through the loop
    __shared__ GemmArgs sa;
    // the computing tile's descriptor, one copy per wave: read back only by
    // the epilogue, so it holds no scalar registers through the steps
    __shared__ Tile tcur[4];
    // Per-lane indices are refreshed through an opaque copy at every tile, so
    // that values derived from them are recomputed per tile instead of being
    // hoisted out of the tile loop, where they would hold registers for good.
    int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wy = (wave & 1) * 128, wx = (wave >> 1) * 128;   // this wave's quadrant (m, n)
    int g32 = lane >> 5, l32 = lane & 31, l16 = lane & 15;
    auto refresh_lane = [&]() {
        asm volatile("" : "+v"(tid));
        lane = tid & 63;
        g32 = lane >> 5;
        l32 = lane & 31;
        l16 = lane & 15;
    };
    constexpr bool F8 = (DT == MXQ_DTYPE_MXFP8_E4M3);
    constexpr int ESZ = F8 ? 1 : 2;
    constexpr int KSR = BK / ESZ;   // contraction elements (rows of a K-strided operand) per stage
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
    int lo = xcd * per + blockIdx.x / kXCD;
    int hi = (xcd + 1) * per < nitems ? (xcd + 1) * per : nitems;
    int istep = nj;   // from one item of this workgroup to its next

    // ---- K-grouped: static or dynamic tile order.  The static order gives
    // each XCD a contiguous range of tiles (a group's tiles share an L2), which
    // balances when the groups are alike.  When the heaviest workgroup of that
    // order would carry more than 9/8 of the mean (skewed routing: a few large
    // groups), the tiles of non-empty groups are taken instead from one
    // counter in the workspace, largest group first, each workgroup taking its
    // next tile as it finishes one (list scheduling, largest first); the tiles
    // of empty groups follow in a static split.  A workgroup keeps a queue of
    // taken tiles, so the load side, which runs a few stages ahead, always
    // finds its next tile there: kTake0 are taken at the start and one more at
    // each epilogue, whose counter result is written to the queue one
    // epilogue later (so that waiting for it waits for nothing else).  Every
    // workgroup reaches the same decision from the same tables.
    int dyn = 0, gne = 0, tpg = ntm * ntn;
    if constexpr (DYN) {
        if (a.sched != nullptr && a.G <= kDynG && (int)gridDim.x <= NTHR) {
            const int G = (int)a.G;
            for (int g = tid; g < G; g += NTHR) {
                const int rows = rs[g + 1] - rs[g];
                gsteps[g] = rows > 0 ? (rows + KSR - 1) / KSR : 0;
            }
            __syncthreads();
            // thread w: the load of workgroup w in the static order; and the total
            int64_t load = 0, tot = 0;
            if (tid < (int)gridDim.x) {
                const int x = tid % kXCD, lo_w = x * per + tid / kXCD;
                const int hi_w = (x + 1) * per < nitems ? (x + 1) * per : nitems;
                for (int it = lo_w; it < hi_w; it += nj) load += gsteps[it / tpg] + kEpiCost;
            }
            for (int g = tid; g < G; g += NTHR) tot += (int64_t)(gsteps[g] + kEpiCost) * tpg;
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const int64_t ol = __shfl_xor(load, d, 64), ot = __shfl_xor(tot, d, 64);
                load = ol > load ? ol : load;
                tot += ot;
            }
            if (lane == 0) {
                red[wave] = load;
                red[4 + wave] = tot;
            }
            __syncthreads();
            int64_t mx = red[0], sum = red[4];
            for (int w = 1; w < 4; w++) {
                mx = red[w] > mx ? red[w] : mx;
                sum += red[4 + w];
            }
            dyn = 8 * mx > 9 * ((sum + gridDim.x - 1) / gridDim.x);
            if (dyn) {
                // rank of each group: more steps first, then the lower index
                for (int g = tid; g < G; g += NTHR) {
                    const int sg = gsteps[g];
                    int r = 0;
                    for (int h = 0; h < G; h++) {
                        const int sh = gsteps[h];
                        r += (sh > sg) | ((sh == sg) & (h < g));
                    }
                    gord[r] = g;
                }
                for (int g = 0; g < G; g++) gne += gsteps[g] > 0;
                // the first kTake0 rounds are dealt, one tile per workgroup per
                // round in alternating direction; the counter hands out the rest
                if (tid < kTake0) {
                    const int nw = (int)gridDim.x, w = (int)blockIdx.x;
                    dq[tid] = tid * nw + ((tid & 1) ? nw - 1 - w : w);
                }
                __syncthreads();
                lo = 0;
                hi = gne * tpg;   // positions past the taken tiles' range are never read
                istep = 1;
            }
        }
    }
    dyn = __builtin_amdgcn_readfirstlane(dyn);

    // tile of work item `item` (false: an m tile past its group's rows)
    auto describe = [&](int item, Tile &T, bool sorted = false) -> bool {
        const uint8_t *A = static_cast<const uint8_t *>(sa.A.data);
        const uint8_t *B = static_cast<const uint8_t *>(sa.B.data);
        int64_t m0, n0, r0, r1, g;
        if constexpr (MODE == MODE_TN) {
            const int per_g = ntm * ntn;
            int rem;
            if (DYN && dyn) {
                // queue position (or, from describe_sorted, the tile itself) ->
                // tile in the largest-first order -> group and tile
                const int t = sorted ? item : dq[item % kQueue];
                if (!sorted && t >= hi) return false;
                const int sg = t / per_g;
                g = gord[sg];
                rem = t - sg * per_g;
            } else {
                g = item / per_g;
                rem = item - (int)g * per_g;
            }
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
            T.x = B + r0 * ldb + n0 * ESZ;
            T.y = A + r0 * lda + m0 * ESZ;
            T.xs = sa.B.scales + blk0 * ldsb + n0;
            T.ys = sa.A.scales + blk0 * ldsa + m0;
            T.o = static_cast<uint8_t *>(sa.out) + (g * sa.out_gstride + m0 * sa.ld_out + n0) * OSZ;
            T.yv = (int)(sa.M - m0 < BT ? sa.M - m0 : BT);
            T.kext = (int)(r1 - r0);
            T.nblk = (T.kext + 31) / 32;
            T.ksteps = (T.kext + KSR - 1) / KSR;
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
                T.x = B + (g * sa.B.gstride + n0) * ESZ;
                T.xs = sa.B.scales + g * sa.B.scale_gstride + n0;
            }
            T.y = A + m0 * lda;
            T.ys = sa.A.scales + m0 * ldsa;
            T.o = static_cast<uint8_t *>(sa.out) + (m0 * sa.ld_out + n0) * OSZ;
            T.yv = (int)(r1 - m0 < BT ? r1 - m0 : BT);
            if constexpr (EPI != 0) {
                T.m0 = m0;
                T.n0 = n0;
                T.srow = (sa.epi_dirs & 2) ? sa.block_off[g] + (m0 - r0) / 32 : 0;
            }
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
    // the first tile at or after `from` (every one, or only those with steps)
    auto describe_sorted = [&](int t, Tile &T) { describe(t, T, true); };
    // (dynamic order: `from` is a queue position, and every taken tile of a
    // non-empty group has steps)
    auto next_tile = [&](int from, bool with_steps) {
        Tile T{};
        if (DYN && dyn) {
            if (describe(from, T)) return T;
        } else {
            for (int item = from; item < hi; item += nj)
                if (describe(item, T) && (!with_steps || T.ksteps > 0)) return T;
        }
        T.valid = 0;
        T.ksteps = 0;
        return T;
    };

    // scale-ring groups issued (load side) and begun (compute side)
    unsigned lgrp = 0, cgrp = 0, cgrp_slot = 0;
    const int nblk_k = (int)((a.K + 31) / 32);
    // (K-strided views count the contraction in rows and the valid columns in
    // bytes; T.kext is the group's rows for TN and K's bytes otherwise)
    auto src_x = [&](const Tile &T) {
        if constexpr (XKS) return Src{T.x, ldb, MODE == MODE_TN ? T.kext : T.kext / ESZ, T.xv * ESZ};
        else return Src{T.x, ldb, T.kext, T.xv};
    };
    auto src_y = [&](const Tile &T) {
        if constexpr (YKS) return Src{T.y, lda, T.kext, T.yv * ESZ};
        else return Src{T.y, lda, T.kext, T.yv};
    };
    // the load side's per-lane data-load offsets (of its current tile)
    const uint32_t lds_smem = lds_addr(smem);
    Feed fdx, fdy;
    // the load tile's operand and column-scale origins advanced to stage `ls`,
    // carried from stage to stage (per-stage strides are per launch)
    const uint8_t *sbx = nullptr, *sby = nullptr, *sbxs = nullptr, *sbys = nullptr;
    // (K-blocked codes: the next stage is the next 64-byte plane)
    const int64_t dsx = XKS ? (int64_t)KSR * ldb : (a.B.plane ? a.B.plane : BK);
    const int64_t dsy = YKS ? (int64_t)KSR * lda : (a.A.plane ? a.A.plane : BK);
    const int64_t dsxs = 2 * (int64_t)ldsb, dsys = 2 * (int64_t)ldsa;

    // Load instruction p of stage s of tile T into stage buffer st (live
    // false: a stage that carries nothing, with the same instruction count):
    // p = 0..3 the X operand, 4..7 the Y operand, then (MXFP8) the X and Y
    // per-stage scales where they do not come through the ring.
    auto issue_piece = [&](auto P, const Tile &T, int s, unsigned slot, bool live) {
        constexpr int p = decltype(P)::value;
        uint8_t *st = smem + slot * STAGE;
        const uint32_t dst = lds_smem + slot * STAGE + 4096 * wave;   // this wave's blocks
        if constexpr (p < 4) {
            if constexpr (XKS) stage_ks<p, ESZ>(src_x(T), sbx, fdx, s, dst, wave, lane, kOOB);
            else stage_kc<p>(src_x(T), sbx, fdx, s, dst, lane, kOOB);
        } else if constexpr (p < 8) {
            if constexpr (YKS) stage_ks<p - 4, ESZ>(src_y(T), sby, fdy, s, dst + OPB, wave, lane, kOOB);
            else stage_kc<p - 4>(src_y(T), sby, fdy, s, dst + OPB, lane, kOOB);
        } else if constexpr (p == 8 && XSB > 0) {
            if constexpr (XKS)
                stage_colscales(ColScales{T.xs, ldsb, T.nblk, T.xv}, sbxs, s, st + 2 * OPB, junk, wave, 0, lane, live);
            else
                stage_rowscales<SC == 1>(RowScales{T.xs, ldsb, T.nblk, T.xv}, s, tid, st + 2 * OPB, junk, live);
        } else if constexpr (YSB > 0) {
            if constexpr (YKS)
                stage_colscales(ColScales{T.ys, ldsa, T.nblk, T.yv}, sbys, s, st + 2 * OPB + XSB, junk, wave, 1, lane,
                                live);
            else
                stage_rowscales<SC == 1>(RowScales{T.ys, ldsa, T.nblk, T.yv}, s, tid, st + 2 * OPB + XSB, junk, live);
        }
    };
    // load instructions per wave per stage (at least: a group's first stage
    // adds its ring loads, which only makes the step waits stricter), and
    // epilogue memory instructions per wave
    constexpr int kStageOps = 8 + (XSB > 0 ? 1 : 0) + (YSB > 0 ? 1 : 0);
    static_assert(kStageOps == 8 + (F8 ? 2 - NRING : 0), "one load per operand's per-stage scales");
    constexpr int kEpiOps = OUT == MXQ_DTYPE_BF16 ? 32 : 64;

    f32x16_t acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; x++)
#pragma unroll
        for (int y = 0; y < 4; y++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[x][y][r] = 0.f;

    // ---- one stage's fragments (each wave's 128 x 128 quadrant as 4 x 4 MFMA
    // tiles of 32 x 32).  MFMA i: MXFP8 x = i / 4, y = i % 4 (16 per stage);
    // bf16 half kk = i / 16, then the same (32 per stage).  Fragment read j
    // (8 per stage and half) follows the order the MFMAs first need them:
    // x0, y0..y3, x1..x3.
    using Frags = std::conditional_t<F8, FragsF8, FragsBF16>;
    constexpr int kMfma = F8 ? 16 : 32;
    constexpr int kReads = F8 ? 8 : 16;
    // K-contiguous fragments: lane (g32, l32) of fragment i takes chunks g32
    // and 2 + g32 of row w + 32 i + l32 (w the wave's quadrant origin): fp8,
    // the two halves of its 32 bytes; bf16, its 8 elements of half 0 and of
    // half 1.  That row's swizzle is (l32 >> 2) & 3 for every i, so the four
    // fragments of an operand sit at fixed distances (i x 32 rows) from two
    // per-lane addresses, and their scale bytes likewise from one: the reads
    // take those distances as immediate offsets.
    struct StageView {
        const uint8_t *st;       // stage buffer
        const uint8_t *xl, *xh;  // K-contiguous X: the lane's chunks g32 and 2 + g32 of fragment row wx + l32
        const uint8_t *yl, *yh;  // the same for Y (row wy + l32)
        const uint8_t *xs, *ys;  // scale byte of fragment 0 (ring or per-stage words; K-strided: column-major)
        bool in_k;               // this lane's block lies inside the contraction
    };
    auto view = [&](const uint8_t *st, int s) {
        StageView v;
        v.st = st;
        const int sw = (l32 >> 2) & 3;
        const int lo = 16 * (g32 ^ sw), hi = 16 * ((2 + g32) ^ sw);
        v.xl = st + (wx + l32) * BK + lo;
        v.xh = st + (wx + l32) * BK + hi;
        v.yl = st + OPB + (wy + l32) * BK + lo;
        v.yh = st + OPB + (wy + l32) * BK + hi;
        const uint8_t *rg = ring + (cgrp_slot & 1) * NRING * RSLOT;
        const int sb = 2 * (s & 1) + g32, rb = 2 * (s % RGS) + g32;
        const uint8_t *scx = st + 2 * OPB, *scy = st + 2 * OPB + XSB;
        if constexpr (XKS) v.xs = scx + g32 * 256 + wx + l32;
        else if constexpr (XRING) v.xs = rg + (wx + l32) * 16 + rb;
        else v.xs = scx + (wx + l32) * 4 + sb;
        if constexpr (YKS) v.ys = scy + g32 * 256 + wy + l32;
        else if constexpr (YRING) v.ys = rg + (XRING ? RSLOT : 0) + (wy + l32) * 16 + rb;
        else v.ys = scy + (wy + l32) * 4 + sb;
        v.in_k = 2 * s + g32 < nblk_k;
        return v;
    };
    auto kc_f8 = [](const uint8_t *l, const uint8_t *h, int i) {
        const u32x4_t a = *reinterpret_cast<const u32x4_t *>(l + 32 * BK * i);
        const u32x4_t b = *reinterpret_cast<const u32x4_t *>(h + 32 * BK * i);
        return i32x8_t{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
    };
    auto kc_bf16 = [](const uint8_t *p, int i) {
        return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t *>(p + 32 * BK * i));
    };
    // scale byte of fragment i (32 rows or columns on)
    constexpr int XSTEP = XKS ? 32 : (XRING ? 32 * 16 : 32 * 4);
    constexpr int YSTEP = YKS ? 32 : (YRING ? 32 * 16 : 32 * 4);
    auto read_frag = [&](Frags &F, auto J, const StageView &v) {
        constexpr int j = decltype(J)::value;
        constexpr int jj = j % 8;
        constexpr bool isx = jj == 0 || jj >= 5;
        constexpr int idx = jj == 0 ? 0 : (jj < 5 ? jj - 1 : jj - 4);
        const uint8_t *tx = v.st, *ty = v.st + OPB;
        if constexpr (F8) {
            if constexpr (isx) {
                if constexpr (XKS) F.fx[idx] = frag_ks_f8(tx, wx + 32 * idx + 16 * ((lane >> 4) & 1), g32, l16);
                else F.fx[idx] = kc_f8(v.xl, v.xh, idx);
                F.sx[idx] = v.xs[XSTEP * idx];   // ring bytes past the row's end: see ring_scales
                if constexpr (XRING) F.in_k = v.in_k;
            } else {
                if constexpr (YKS) F.fy[idx] = frag_ks_f8(ty, wy + 32 * idx + 16 * ((lane >> 4) & 1), g32, l16);
                else F.fy[idx] = kc_f8(v.yl, v.yh, idx);
                F.sy[idx] = v.ys[YSTEP * idx];
                if constexpr (YRING) F.in_k = v.in_k;
            }
        } else {
            constexpr int kk = j / 8;
            if constexpr (isx) {
                if constexpr (XKS) F.fx[kk][idx] = frag_ks_bf16(tx, wx + 32 * idx + 16 * ((lane >> 4) & 1), kk, g32, l16);
                else F.fx[kk][idx] = kc_bf16(kk ? v.xh : v.xl, idx);
            } else {
                if constexpr (YKS) F.fy[kk][idx] = frag_ks_bf16(ty, wy + 32 * idx + 16 * ((lane >> 4) & 1), kk, g32, l16);
                else F.fy[kk][idx] = kc_bf16(kk ? v.yh : v.yl, idx);
            }
        }
    };
    // Ring scale bytes of blocks past the contraction are whatever follows
    // the row; such blocks have zero codes and take the unit scale, applied
    // here once the set's reads are complete (a select next to each read
    // would wait for it).
    auto ring_scales = [&](Frags &F) {
        if constexpr (F8 && (XRING || YRING)) {
#pragma unroll
            for (int x = 0; x < 4; x++) {
                if constexpr (XRING) F.sx[x] = F.in_k ? F.sx[x] : 127;
                if constexpr (YRING) F.sy[x] = F.in_k ? F.sy[x] : 127;
            }
        }
    };
    // MFMA i of a stage.  The empty asm statement after it takes its result,
    // so that the MFMA stays in its slot: a computation without side effects
    // could otherwise be sunk past the step's waits and barrier, off the
    // loads and reads it is meant to overlap.
    auto mfma = [&](const Frags &F, auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (F8) {
            constexpr int x = i / 4, y = i % 4;
            acc[x][y] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.fx[x], F.fy[y], acc[x][y], 0, 0, 0, F.sx[x],
                                                                         0, F.sy[y]);
            asm volatile("" ::"a"(acc[x][y]));
        } else {
            constexpr int kk = i / 16, x = (i % 16) / 4, y = i % 4;
            acc[x][y] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.fx[kk][x], F.fy[kk][y], acc[x][y], 0, 0, 0);
            asm volatile("" ::"a"(acc[x][y]));
        }
    };

    // ---- the fused SwiGLU epilogue.  Quarter h of a bf16 tile sits in the
    // staging buffer: 64 rows x 256 columns, staging row m < 32 being tile row
    // 32h + m and m >= 32 tile row 128 + 32h + m - 32 (so rows 0..31 and
    // 32..63 are two whole 32-row colwise blocks).  B's rows hold gate and up
    // interleaved in blocks of 128, so tile columns 0..127 are the gate and
    // 128..255 the up of activation columns n0/2 .. n0/2 + 127.  Thread t
    // takes the items (m, q) = (i / 16, i % 16), i = 256 it + t, it < 4: the 8
    // activation columns 8q .. 8q + 7 of staging row m.  The 4 lanes of a 1x32
    // block are then 4 consecutive lanes (a DPP quad), items 0-1 lie in the
    // first 32-row block and 2-3 in the second, and the lanes of a wave with
    // one q hold 8 rows of each block.  The arithmetic is the fused
    // activation kernels' (act_math.h), exact path included, so the codes and
    // scales are those of mxq_swiglu_quantize_fwd applied to the bf16 output.
    __shared__ uint32_t emx[EPI ? NTHR / 64 * 2 * 16 * 4 : 1];   // per-wave colwise maxima
    auto fused_act = [&](const Tile &T, const uint8_t *stg, int h, int yv) {
        if constexpr (EPI != 0) {
            constexpr int ACT = EPI == 2 ? ACT_CLAMPED : ACT_SWIGLU;
            const unsigned dirs = sa.epi_dirs;
            const float L = sa.epi_limit;
            const float *scale = sa.epi_scale;
            const int64_t j0 = T.n0 / 2, m0 = T.m0;
            const int q = tid & 15;
            uint32_t hv[4][4];
            uint32_t fix = 0;   // elements the fast path may round differently (bit 8 it + k)
#pragma unroll
            for (int it = 0; it < 4; it++) {
                const int m = (it * NTHR + tid) >> 4;
                const int tr = (m < 32 ? 32 * h : 128 + 32 * h - 32) + m;
                const bool valid = tr < yv;
                const u32x4_t gw = *reinterpret_cast<const u32x4_t *>(stg + m * 512 + 16 * (q ^ (m & 31)));
                const u32x4_t uw = *reinterpret_cast<const u32x4_t *>(stg + m * 512 + 16 * ((16 + q) ^ (m & 31)));
                const uint32_t g4[4] = {gw.x, gw.y, gw.z, gw.w}, u4[4] = {uw.x, uw.y, uw.z, uw.w};
                const float s = (valid && scale != nullptr) ? scale[m0 + tr] : 1.0f;
                uint32_t bits = 0u;
#pragma unroll
                for (int k = 0; k < 4; k++) bits |= fwd_pair<ACT>(g4[k], u4[k], s, L, hv[it][k]) << (2 * k);
                if (!normal_or_zero(s)) bits = 0xFFu;
#pragma unroll
                for (int k = 0; k < 4; k++) hv[it][k] = valid ? hv[it][k] : 0u;   // rows past the group
                fix |= (valid ? bits : 0u) << (8 * it);
            }
            // the flagged elements in fp64, one rolled loop (one copy of that code)
            while (fix) {
                const int idx = __builtin_ctz(fix);
                fix &= fix - 1u;
                const int it = idx >> 3, k = idx & 7;
                const int m = (it * NTHR + tid) >> 4;
                const int tr = (m < 32 ? 32 * h : 128 + 32 * h - 32) + m;
                const uint8_t *row = stg + m * 512;
                const float g = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(
                                                    row + 16 * (q ^ (m & 31)) + 2 * k) << 16);
                const float u = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(
                                                    row + 16 * ((16 + q) ^ (m & 31)) + 2 * k) << 16);
                const float s = scale != nullptr ? scale[m0 + tr] : 1.0f;
                const uint32_t v = fwd_elem_f64(g, u, s, L, ACT);
#pragma unroll
                for (int i2 = 0; i2 < 4; i2++)
#pragma unroll
                    for (int w = 0; w < 4; w++)
                        if (i2 == it && w == (k >> 1))
                            hv[i2][w] = (k & 1) ? ((hv[i2][w] & 0x0000FFFFu) | (v << 16))
                                                : ((hv[i2][w] & 0xFFFF0000u) | v);
            }
            if (dirs & 1) {
#pragma unroll
                for (int it = 0; it < 4; it++) {
                    const int m = (it * NTHR + tid) >> 4;
                    const int tr = (m < 32 ? 32 * h : 128 + 32 * h - 32) + m;
                    uint32_t mm = 0u;
#pragma unroll
                    for (int k = 0; k < 4; k++) mm = umax16x2(mm, hv[it][k] & 0x7FFF7FFFu);
                    mm = block_max<4>(max(mm & 0xFFFFu, mm >> 16));
                    const uint32_t E = e8m0_from_amax_bits(mm);
                    const u32x2_t c = {cvt4_same(hv[it][0], hv[it][1], E), cvt4_same(hv[it][2], hv[it][3], E)};
                    if (tr < yv) {
                        const int64_t r = m0 + tr;
                        __builtin_nontemporal_store(c, reinterpret_cast<u32x2_t *>(sa.epi_rc + r * sa.epi_ld_rc + j0 +
                                                                                   8 * q));
                        if ((q & 3) == 0) sa.epi_rs[r * sa.epi_ld_rs + (j0 + 8 * q) / 32] = (uint8_t)E;
                    }
                }
            }
            if (dirs & 2) {
                // column maxima of each 32-row block: the thread's two rows, the
                // wave's 8 (lanes q, q + 16, q + 32, q + 48), then the 4 waves
#pragma unroll
                for (int b = 0; b < 2; b++) {
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        uint32_t v = umax16x2(hv[2 * b][k] & 0x7FFF7FFFu, hv[2 * b + 1][k] & 0x7FFF7FFFu);
                        v = umax16x2(v, (uint32_t)__shfl_xor((int)v, 16, 64));
                        v = umax16x2(v, (uint32_t)__shfl_xor((int)v, 32, 64));
                        if (lane < 16) emx[((wave * 2 + b) * 16 + lane) * 4 + k] = v;
                    }
                }
                step_barrier<63>();
#pragma unroll
                for (int b = 0; b < 2; b++) {
                    uint32_t cm[4];
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        uint32_t v = emx[(b * 16 + q) * 4 + k];
#pragma unroll
                        for (int w = 1; w < NTHR / 64; w++) v = umax16x2(v, emx[((w * 2 + b) * 16 + q) * 4 + k]);
                        cm[k] = v;
                    }
                    uint32_t E[8];
                    float sc[8];
                    uint32_t nanm[2] = {0u, 0u};
#pragma unroll
                    for (int k = 0; k < 4; k++) {
                        E[2 * k] = e8m0_from_amax_bits(cm[k] & 0xFFFFu);
                        E[2 * k + 1] = e8m0_from_amax_bits(cm[k] >> 16);
                    }
#pragma unroll
                    for (int k = 0; k < 8; k++) {
                        sc[k] = scale_operand(E[k]);
                        nanm[k >> 2] |= (E[k] == 0xFFu ? 0xFFu : 0u) << (8 * (k & 3));
                    }
#pragma unroll
                    for (int i2 = 0; i2 < 2; i2++) {
                        const int it = 2 * b + i2;
                        const int m = (it * NTHR + tid) >> 4;
                        const int tr = (m < 32 ? 32 * h : 128 + 32 * h - 32) + m;
                        const u32x2_t c = {cvt4_cols(hv[it][0], hv[it][1], sc, nanm[0]),
                                           cvt4_cols(hv[it][2], hv[it][3], sc + 4, nanm[1])};
                        if (tr < yv)
                            __builtin_nontemporal_store(c, reinterpret_cast<u32x2_t *>(
                                                               sa.epi_cc + (m0 + tr) * sa.epi_ld_cc + j0 + 8 * q));
                    }
                    const int tb = b == 0 ? 32 * h : 128 + 32 * h;   // the block's first tile row
                    if (tid < 16 && tb < yv) {
                        const u32x2_t e = {E[0] | (E[1] << 8) | (E[2] << 16) | (E[3] << 24),
                                           E[4] | (E[5] << 8) | (E[6] << 16) | (E[7] << 24)};
                        __builtin_nontemporal_store(e, reinterpret_cast<u32x2_t *>(
                                                           sa.epi_cs + (T.srow + tb / 32) * sa.epi_ld_cs + j0 + 8 * q));
                    }
                }
            }
        }
    };

    // ---- epilogue: lane (g32, l32) holds C[m][n .. n+3] with m = wy + 32y + l32,
    // n = wx + 32x + 8q + 4 g32, in registers 4q .. 4q+3 of acc[x][y].
    const int ldo = (int)(a.ld_out * OSZ);   // output row pitch in bytes (< 2^23)
    const bool accumulate = a.accumulate != 0;
    auto epilogue = [&](const Tile &T, uint8_t *stg) {
        const __amdgpu_buffer_rsrc_t ro = rsrc(T.o, 0x7FFFFFF0);
        // The tile's extents and the pitch in registers, read once: the stores
        // below may alias the tile descriptor's LDS copy as far as the compiler
        // knows (it would read it again after each), and an opaque value used
        // under a condition would be computed in a branch of its own.
        const int yv = __builtin_amdgcn_readfirstlane(T.yv), xv = __builtin_amdgcn_readfirstlane(T.xv);
        const int ldo_r = opaque(ldo);
        if constexpr (OUT == MXQ_DTYPE_BF16) {
            // Through LDS, so that each output row leaves as 512 contiguous
            // bytes (16-byte nontemporal stores, 32 lanes per row): the buffer
            // of the stage just read holds a quarter of the tile, 64 rows x
            // 512 B with 16-byte chunk c of row m at c ^ (m & 31).  Quarter h
            // is fragment row y = h of every wave: rows 32h .. 32h + 31 (from
            // the two waves with wy = 0, staged as rows 0..31) and 128 + 32h ..
            // (from the other two, staged as rows 32..63), so all four waves
            // write each quarter, then all four store it.
            typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
            for (int h = 0; h < 4; h++) {
                step_barrier<63>();   // everyone is done reading stg (last step's fragments, or quarter h - 1)
                {
                    const int y = h;
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int x = 0; x < 4; x++) asm volatile("" : "+a"(acc[x][y]));
                    const int m = (wy >> 2) + l32;   // staging row
#pragma unroll
                    for (int x = 0; x < 4; x++)
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const int chunk = (wx + 32 * x + 8 * q) >> 3;
                            bf16x4_t b;
                            b.x = (__bf16)acc[x][y][4 * q];
                            b.y = (__bf16)acc[x][y][4 * q + 1];
                            b.z = (__bf16)acc[x][y][4 * q + 2];
                            b.w = (__bf16)acc[x][y][4 * q + 3];
                            *reinterpret_cast<bf16x4_t *>(stg + m * 512 + 16 * (chunk ^ (m & 31)) + 8 * g32) = b;
                        }
                    __builtin_amdgcn_sched_barrier(0);
                }
                step_barrier<63>();   // quarter h is in LDS
                // all eight reads first: the compiler keeps LDS reads behind
                // earlier buffer stores, so interleaving them would wait for
                // each read in turn
                u32x4_t v[8];
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int qd = j * NTHR + tid;
                    const int m = qd >> 5, c = qd & 31;
                    v[j] = *reinterpret_cast<const u32x4_t *>(stg + m * 512 + 16 * (c ^ (m & 31)));
                }
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const int qd = j * NTHR + tid;
                    const int m = qd >> 5, c = qd & 31;
                    const int row = (m < 32 ? 0 : 128 - 32) + 32 * h + m;   // tile row of staging row m
                    const uint32_t off = ((row < yv) & (8 * c < xv)) ? (uint32_t)(row * ldo_r + 16 * c) : kOOB;
                    __builtin_amdgcn_raw_buffer_store_b128(v[j], ro, off, 0, 2);   // nt
                }
                fused_act(T, stg, h, yv);
            }
        } else {
            // fp32: straight from the accumulators
#pragma unroll
            for (int y = 0; y < 4; y++) {
                // one row of fragments at a time, so that only its accumulators
                // are copied out of the matrix registers at once
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int x = 0; x < 4; x++) asm volatile("" : "+a"(acc[x][y]));
                const int ml = wy + 32 * y + l32;
                const uint32_t row = ml < yv ? (uint32_t)(ml * ldo_r + (wx + 4 * g32) * OSZ) : kOOB;
#pragma unroll
                for (int x = 0; x < 4; x++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        // columns past N (last n tile only) go out of range too
                        const uint32_t off = wx + 32 * x + 8 * q + 4 * g32 < xv ? row + (32 * x + 8 * q) * OSZ : kOOB;
                        f32x4_t w = f32x4_t{acc[x][y][4 * q], acc[x][y][4 * q + 1], acc[x][y][4 * q + 2],
                                            acc[x][y][4 * q + 3]};
                        if (accumulate)
                            w += __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, w), ro, off, 0, 0);
                    }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ---- the load side: tile `ld` (with steps), its next stage `ls`
    Tile ld = next_tile(lo, true);
    int ls = 0;
    auto make_feeds = [&]() {
        const bool live = ld.valid != 0;
        if constexpr (XKS) fdx = feed_ks<ESZ>(src_x(ld), live, wave, lane);
        else fdx = feed_kc(src_x(ld), live, wave, lane);
        if constexpr (YKS) fdy = feed_ks<ESZ>(src_y(ld), live, wave, lane);
        else fdy = feed_kc(src_y(ld), live, wave, lane);
        sbx = ld.x;
        sby = ld.y;
        sbxs = ld.xs;
        sbys = ld.ys;
    };
    make_feeds();
    unsigned issued = 0, consumed = 0;
    // epilogues run so far, and for each stage buffer that count when its
    // stage was issued (8 bits each): a stage's wait leaves in flight every
    // memory instruction issued after it
    unsigned epis = 0, epi_at = 0;
    bool pending = false;   // an issued stage the load side has not moved past yet
    // The scale ring: before the load side issues a group's first stage, the
    // group's 16 scale bytes per row go into slot lgrp & 1.
    auto ring_issue = [&]() {
        if constexpr (NRING > 0) {
            if (ld.valid && ls % RGS == 0) {
                uint8_t *slot = ring + (lgrp & 1) * NRING * RSLOT;
                const int row = 64 * wave + lane;
                if constexpr (XRING) {
                    const i32x4_t r = rsrc4(ld.xs, (int64_t)ld.xv * ldsb);
                    to_lds(r, slot + 1024 * wave, row < ld.xv ? (uint32_t)(row * ldsb + 2 * ls) : kOOB);
                }
                if constexpr (YRING) {
                    const i32x4_t r = rsrc4(ld.ys, (int64_t)ld.yv * ldsa);
                    to_lds(r, slot + (XRING ? RSLOT : 0) + 1024 * wave,
                           row < ld.yv ? (uint32_t)(row * ldsa + 2 * ls) : kOOB);
                }
                lgrp++;
            }
        }
    };
    auto issued_one = [&](unsigned slot) {
        epi_at = (epi_at & ~(0xFFu << (8 * slot))) | ((epis & 0xFFu) << (8 * slot));
        issued++;
        pending = true;
    };
    auto advance_load = [&]() {
        if (pending && ld.valid) {
            if (++ls == ld.ksteps) {
                ld = next_tile(ld.item + istep, true);
                ls = 0;
                make_feeds();
            } else {
                sbx += dsx;
                sby += dsy;
                if constexpr (XKS) sbxs += dsxs;
                if constexpr (YKS) sbys += dsys;
            }
        }
        pending = false;
    };
    // Wait until stage c has landed.  Vector memory operations of a wave
    // complete in issue order on this target, loads and stores alike (the
    // compiler's wait counts rely on the same), so it has once no more than
    // the later ones are in flight: the next two stages, plus an epilogue's
    // memory operations if one ran since stage c was issued (vmcnt saturates
    // at 63; more than that follows then).
    auto wait_stage = [&](unsigned c) {
        const unsigned slot = c & (NBUF - 1);
        const unsigned since = (epis - (epi_at >> (8 * slot))) & 0xFFu;
        if (opaque(__builtin_amdgcn_readfirstlane((int)since)) == 0) {
            constexpr int n = 2 * kStageOps;
            __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
        } else if (opaque(__builtin_amdgcn_readfirstlane((int)since)) == 1) {
            constexpr int n = 2 * kStageOps + kEpiOps < 63 ? 2 * kStageOps + kEpiOps : 63;
            __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
        } else {
            __builtin_amdgcn_s_waitcnt(0xCF7F);   // vmcnt(63)
        }
    };

    // ---- the pipeline.  Stage c is computed from registers while stage
    // c + 1 sits in LDS and stages c + 2 .. c + 4 load: in the shadow of
    // stage c's MFMAs a wave waits for stage c + 1, passes the step's barrier
    // (after which every wave has its stage-c fragments, so that buffer is
    // free), reads stage c + 1's fragments into the other register set and
    // issues stage c + 4 into stage c's buffer.  The load side walks the same
    // tile sequence (skipping tiles without steps), so at a tile's last step
    // the stage read is the next tile's first, and the epilogue stages the
    // output through that stage's buffer (its fragments are in registers; the
    // next step's barrier orders the buffer's reuse).
    static_for<0, NBUF>([&](auto) {
        ring_issue();
        const unsigned slot = issued & (NBUF - 1);
        static_for<0, kStageOps>([&](auto P) { issue_piece(P, ld, ls, slot, ld.valid != 0); });
        issued_one(slot);
        advance_load();
    });
    const Tile c0 = next_tile(lo, false);
    if (!c0.valid && !dyn) return;   // (the loads issued above carried nothing)
    tcur[wave] = c0;
    Frags FA, FB;
    {
        constexpr int n = 3 * kStageOps;   // stage 0 has landed: stages 1..3 may be in flight
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70);
        step_barrier<63>();
        if constexpr (NRING > 0) cgrp_slot = cgrp++;
        const StageView v = view(smem, 0);
        static_for<0, kReads>([&](auto J) { read_frag(FA, J, v); });
    }
    // step s of a K-step tile: MFMAs from P, the next stage's fragments into Q
    auto step = [&](Frags &P, Frags &Q, int s, int K) {
        advance_load();
        ring_scales(P);
        mfma(P, IC<0>{});
        mfma(P, IC<1>{});
        __builtin_amdgcn_sched_barrier(0);
        const unsigned cn = consumed + 1;
        wait_stage(cn);
        step_barrier<63>();   // stage cn has landed everywhere; stage `consumed` is read everywhere
        ring_issue();
        const int sn = s + 1 < K ? s + 1 : 0;   // stage cn's step within its tile
        if constexpr (NRING > 0) {
            if (sn % RGS == 0) cgrp_slot = cgrp++;
        }
        const StageView v = view(smem + (cn & (NBUF - 1)) * STAGE, sn);
        const unsigned slot = issued & (NBUF - 1);   // == consumed & (NBUF - 1)
        const bool live = ld.valid != 0;
        // One MFMA per slot; a wave issues in order, so the reads and loads
        // placed after an MFMA go out while the matrix core runs it.  The
        // fragment reads take the first slots (they must land by the next
        // step).  Where the stage's loads go was measured per mode
        // (alternating timings on one GPU): MXFP8 NT from slot 4 on, dgrad
        // from slot 2 (beside the reads), wgrad from slot 6, bf16 in every
        // other slot of the second half; packing them into the last slots
        // was 1-5 % slower, and moving the wgrad or bf16 loads earlier too.
        constexpr int kLoadStride = F8 ? 1 : 2;
        constexpr int kFirstLoad = MODE == MODE_NN ? 2 : (!F8 ? kMfma - 2 * kStageOps : (MODE == MODE_NT ? 4 : 6));
        static_assert(kFirstLoad >= 2 && kFirstLoad + (kStageOps - 1) * kLoadStride < kMfma,
                      "a load slot per stage load");
        static_for<2, kMfma>([&](auto I) {
            constexpr int i = decltype(I)::value;
            mfma(P, I);
            if constexpr (i - 2 < kReads) read_frag(Q, IC<i - 2>{}, v);
            constexpr int q = i - kFirstLoad;
            if constexpr (q >= 0 && q % kLoadStride == 0 && q / kLoadStride < kStageOps)
                issue_piece(IC<q / kLoadStride>{}, ld, ls, slot, live);
            __builtin_amdgcn_sched_barrier(0);
        });
        issued_one(slot);
        consumed++;
    };
    // Dynamic order: the counter value taken at an epilogue reaches the queue
    // at the start of the next one: the only memory operations the compiler
    // sees after it are that epilogue's stores, so its wait there leaves the
    // stage loads in flight alone.  (Only thread 0 takes and reads `taken`.)
    int taken = 0;
    bool have = false;
    int qfill = kTake0;   // queue entries written
    for (bool more = c0.valid != 0; more;) {
        refresh_lane();
        const int K = tcur[wave].ksteps;
        // two steps per iteration, so that the register sets alternate
        // without copies (an odd last step copies once)
        int s = 0;
        for (; s + 1 < K; s += 2) {
            step(FA, FB, s, K);
            step(FB, FA, s + 1, K);
        }
        if (s < K) {
            step(FA, FB, s, K);
            FA = FB;
        }
        if (DYN && dyn) {
            if (have) {
                if (tid == 0) dq[qfill % kQueue] = kTake0 * (int)gridDim.x + taken;
                qfill++;
            }
            if (tid == 0) taken = __hip_atomic_fetch_add(a.sched, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            have = true;
        }
        // the buffer of the stage just read (no load is headed for it)
        epilogue(tcur[wave], smem + (consumed & (NBUF - 1)) * STAGE);
        epis++;
        const Tile nc = next_tile(tcur[wave].item + istep, false);
        more = nc.valid != 0;
        if (!more) break;
        tcur[wave] = nc;
#pragma unroll
        for (int x = 0; x < 4; x++)
#pragma unroll
            for (int y = 0; y < 4; y++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[x][y][r] = 0.f;
    }
    // Dynamic order: the tiles of empty groups (zeros, or the output left as
    // it is when accumulating), split statically.
    if constexpr (DYN) {
        if (dyn) {
#pragma unroll
            for (int x = 0; x < 4; x++)
#pragma unroll
                for (int y = 0; y < 4; y++)
#pragma unroll
                    for (int r = 0; r < 16; r++) acc[x][y][r] = 0.f;
            const int ne = ((int)a.G - gne) * tpg;
            for (int e = (int)blockIdx.x; e < ne; e += (int)gridDim.x) {
                Tile T{};
                describe_sorted(gne * tpg + e, T);
                epilogue(T, smem + (consumed & (NBUF - 1)) * STAGE);
            }
        }
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
    // the row scales' path (see the kernel's SC)
    int sc = 1;
    if (DT == MXQ_DTYPE_MXFP8_E4M3 && MODE != MODE_TN) {
        const int64_t nblk = (g.K + 31) / 32, ks = (g.K + BK - 1) / BK;
        const bool ld4 = g.A.ld_scales % 4 == 0 && (MODE == MODE_NN || g.B.ld_scales % 4 == 0);
        const bool ring = ld4 && ks >= 3 && (ks % RGS == 0 || ks % RGS >= 3);
        sc = ring ? 2 : (ld4 && nblk % 4 == 0 ? 1 : 0);
    }
    const dim3 gd((unsigned)grid), bd(NTHR);
    const int a1 = (int)ntn, a2 = (int)ntm;
    const bool tab = g.G <= kTab;
    if (MODE == MODE_TN && g.sched != nullptr) hipLaunchKernelGGL(sched_reset, dim3(1), dim3(64), 0, stream, g.sched);
    if constexpr (MODE == MODE_NT && DT == MXQ_DTYPE_BF16 && OUT == MXQ_DTYPE_BF16) {
        if (g.epi_act != 0) {
            if (g.epi_act == 2) {
                if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 1, 2>), gd, bd, 0, stream, g, a1, a2);
                else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 1, 2>), gd, bd, 0, stream, g, a1, a2);
            } else {
                if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 1, 1>), gd, bd, 0, stream, g, a1, a2);
                else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 1, 1>), gd, bd, 0, stream, g, a1, a2);
            }
            return hipGetLastError();
        }
    }
    if constexpr (DT != MXQ_DTYPE_MXFP8_E4M3 || MODE == MODE_TN) {
        if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 1>), gd, bd, 0, stream, g, a1, a2);
        else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 1>), gd, bd, 0, stream, g, a1, a2);
        (void)sc;
    } else if (sc == 2) {
        if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 2>), gd, bd, 0, stream, g, a1, a2);
        else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 2>), gd, bd, 0, stream, g, a1, a2);
    } else if (sc == 1) {
        if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 1>), gd, bd, 0, stream, g, a1, a2);
        else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 1>), gd, bd, 0, stream, g, a1, a2);
    } else {
        if (tab) hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, true, 0>), gd, bd, 0, stream, g, a1, a2);
        else hipLaunchKernelGGL((gemm_kernel<MODE, DT, OUT, false, 0>), gd, bd, 0, stream, g, a1, a2);
    }
    return hipGetLastError();
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// bound on a K-blocked operand's planes (bytes), far below 2^62
constexpr int64_t kMaxPlaneExtent = int64_t(1) << 60;

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
    g.A = GemmOperand{in.A.dtype, in.A.data, in.A.ld, in.A.gstride, in.A.scales, in.A.ld_scales, in.A.scale_gstride,
                      in.A.kblock_plane};
    g.B = GemmOperand{in.B.dtype, in.B.data, in.B.ld, in.B.gstride, in.B.scales, in.B.ld_scales, in.B.scale_gstride,
                      in.B.kblock_plane};
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
    // K-blocked operands (64-byte contraction planes; either dtype): only the
    // operands read along the contraction.  A plane row is 64 bytes, i.e. ld
    // = 64 / element size, and the group stride counts elements too.
    const bool kba = in.A.kblock_plane != 0, kbb = in.B.kblock_plane != 0;
    if (kba || kbb) {
        if (in.A.kblock_plane < 0 || in.B.kblock_plane < 0) { err = "kblock_plane must be >= 0"; return MXQ_ERR_SHAPE; }
        if (in.mode == MXQ_GEMM_TN || (in.mode == MXQ_GEMM_NN && kbb)) {
            err = "only operands contiguous along the contraction (A of NT / NN, B of NT) can be K-blocked";
            return MXQ_ERR_UNSUPPORTED;
        }
        if ((in.K * esz) % 64 != 0) { err = "K-blocked operands need K a multiple of 64 bytes"; return MXQ_ERR_SHAPE; }
        if ((kba && in.A.ld * esz != 64) || (kbb && in.B.ld * esz != 64)) {
            err = "a K-blocked operand has ld = 64 bytes";
            return MXQ_ERR_SHAPE;
        }
        if ((kba && in.A.kblock_plane % 16 != 0) || (kbb && in.B.kblock_plane % 16 != 0)) {
            err = "kblock_plane must be a multiple of 16 bytes";
            return MXQ_ERR_ALIGN;
        }
        if (kba && in.A.kblock_plane < in.M * 64) { err = "A kblock_plane is smaller than its M rows of 64 bytes"; return MXQ_ERR_SHAPE; }
        if (kbb && (in.B.kblock_plane < (in.G - 1) * in.B.gstride * esz + in.N * 64 ||
                    (in.G > 1 && in.B.gstride * esz < in.N * 64))) {
            err = "B kblock_plane or group stride too small for G groups of N rows of 64 bytes";
            return MXQ_ERR_SHAPE;
        }
        const int64_t planes = in.K * esz / 64;
        if ((kba && in.A.kblock_plane > kMaxPlaneExtent / planes) || (kbb && in.B.kblock_plane > kMaxPlaneExtent / planes)) {
            err = "K-blocked operand extent too large";
            return MXQ_ERR_OVERFLOW;
        }
    }
    // operand extents
    if (in.mode == MXQ_GEMM_NT) {
        if ((!kba && in.A.ld < in.K) || (!kbb && in.B.ld < in.K) || in.ld_out < in.N) { err = "ld too small"; return MXQ_ERR_SHAPE; }
        if (!kbb && in.B.gstride < (in.N - 1) * in.B.ld + in.K && in.G > 1) { err = "B group stride too small"; return MXQ_ERR_SHAPE; }
        if (f8 && (in.A.ld_scales < (in.K + 31) / 32 || in.B.ld_scales < (in.K + 31) / 32)) { err = "ld_scales too small"; return MXQ_ERR_SHAPE; }
    } else if (in.mode == MXQ_GEMM_NN) {
        if ((!kba && in.A.ld < in.K) || in.B.ld < in.N || in.ld_out < in.N) { err = "ld too small"; return MXQ_ERR_SHAPE; }
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
            if (f8) return o32 ? launch_mode<MODE_NN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_F32>(g, stream)
                               : launch_mode<MODE_NN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_BF16>(g, stream);
            return o32 ? launch_mode<MODE_NN, MXQ_DTYPE_BF16, MXQ_DTYPE_F32>(g, stream)
                       : launch_mode<MODE_NN, MXQ_DTYPE_BF16, MXQ_DTYPE_BF16>(g, stream);
        default:
            if (f8) return o32 ? launch_mode<MODE_TN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_F32>(g, stream)
                               : launch_mode<MODE_TN, MXQ_DTYPE_MXFP8_E4M3, MXQ_DTYPE_BF16>(g, stream);
            return o32 ? launch_mode<MODE_TN, MXQ_DTYPE_BF16, MXQ_DTYPE_F32>(g, stream)
                       : launch_mode<MODE_TN, MXQ_DTYPE_BF16, MXQ_DTYPE_BF16>(g, stream);
    }
}

}  // namespace mxq
