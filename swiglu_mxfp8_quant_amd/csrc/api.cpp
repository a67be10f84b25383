// api.cpp -- the C ABI of libmxq (declared in include/mxq.h): argument
// validation, error reporting and dispatch to the HIP launchers.  Nothing here
// touches device memory; every launch is asynchronous on the caller's stream.
#include "mxq.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "gemm_internal.h"
#include "mxq_internal.h"

namespace {

thread_local std::string g_last_error;

mxq_status fail(mxq_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

mxq_status ok() {
    g_last_error.clear();
    return MXQ_OK;
}

mxq_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return ok();
    return fail(MXQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxExtent = int64_t(1) << 62;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte footprint of a strided 2-D array (rows x cols elements of esize bytes,
// row pitch ld elements): the interval [lo, hi) plus the pitch and row width,
// so that interleaved arrays with one pitch (e.g. the two halves of a packed
// [dgate | dup]) are not mistaken for overlapping ones.
struct Range {
    uintptr_t lo = 0, hi = 0;
    uintptr_t pitch = 0, width = 0;
    const char *name = "";
};

Range range2d(const void *p, int64_t rows, int64_t cols, int64_t ld, int64_t esize, const char *name) {
    Range r;
    r.name = name;
    if (p == nullptr || rows <= 0 || cols <= 0) return r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)(((rows - 1) * ld + cols) * esize);
    r.pitch = rows > 1 ? (uintptr_t)(ld * esize) : 0;
    r.width = (uintptr_t)(cols * esize);
    return r;
}

// Footprint of K-blocked codes: `planes` planes `plane` bytes apart, each
// holding `extent` bytes from its start.
Range range_kblock(const void *p, int64_t planes, int64_t plane, int64_t extent, const char *name) {
    Range r;
    r.name = name;
    if (p == nullptr || planes <= 0 || extent <= 0) return r;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)((planes - 1) * plane + extent);
    return r;
}

bool overlap(const Range &a, const Range &b) {
    if (!(a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi)) return false;
    if (a.pitch != 0 && a.pitch == b.pitch) {
        // same pitch: disjoint iff the row segments never meet modulo the pitch
        const uintptr_t d = (b.lo >= a.lo) ? (b.lo - a.lo) % a.pitch : (a.pitch - (a.lo - b.lo) % a.pitch) % a.pitch;
        if (d >= a.width && d + b.width <= a.pitch) return false;
    }
    return true;
}

// every output against every input and every other output
mxq_status check_alias(const std::vector<Range> &in, const std::vector<Range> &out) {
    for (size_t i = 0; i < out.size(); i++) {
        for (const Range &r : in)
            if (overlap(out[i], r)) return fail(MXQ_ERR_ALIAS, "output %s overlaps input %s", out[i].name, r.name);
        for (size_t j = i + 1; j < out.size(); j++)
            if (overlap(out[i], out[j]))
                return fail(MXQ_ERR_ALIAS, "output %s overlaps output %s", out[i].name, out[j].name);
    }
    return MXQ_OK;
}

// extent of rows x ld elements must stay far below 2^62 bytes
bool extent_ok(int64_t rows, int64_t ld, int64_t esize) {
    if (rows <= 0) return true;
    if (ld > kMaxExtent / esize) return false;
    return rows <= kMaxExtent / (ld * esize);
}

// Validate one MXFP8 output of `rows x cols` with `srows` scale rows.
mxq_status check_mx_out(const mxq_mx_out *o, bool rowwise, int64_t rows, int64_t cols, int64_t srows,
                        const char *name, std::vector<Range> &outs) {
    if (o == nullptr || o->codes == nullptr || o->scales == nullptr)
        return fail(MXQ_ERR_NULL, "%s output (codes and scales) is required for this direction", name);
    const int64_t plane = o->kblock_plane;
    if (plane != 0) {
        // K-blocked rowwise codes: (k / 64) plane + 64 r + k % 64, stored
        // with 32-bit offsets from each row's start
        if (!rowwise) return fail(MXQ_ERR_UNSUPPORTED, "%s: only rowwise codes can be K-blocked", name);
        if (plane < 0) return fail(MXQ_ERR_SHAPE, "%s kblock_plane %lld < 0", name, (long long)plane);
        if (o->ld_codes != 64) return fail(MXQ_ERR_SHAPE, "%s: K-blocked codes have ld_codes = 64", name);
        if (cols % 64 != 0) return fail(MXQ_ERR_SHAPE, "%s: K-blocked codes need a multiple of 64 columns", name);
        if (plane % 16 != 0 || !aligned(o->codes, 16))
            return fail(MXQ_ERR_ALIGN, "%s codes pointer and kblock_plane must be multiples of 16 bytes", name);
        if (plane < rows * 64) return fail(MXQ_ERR_SHAPE, "%s kblock_plane %lld < 64 x %lld rows", name, (long long)plane, (long long)rows);
        if (cols > 0 && (plane > (int64_t(1) << 31) || (cols / 64 - 1) * plane + 64 > int64_t(0x7FFFFFF0)))
            return fail(MXQ_ERR_OVERFLOW, "%s: K-blocked codes must span less than 2^31 bytes", name);
    } else if (o->ld_codes < cols) {
        return fail(MXQ_ERR_SHAPE, "%s ld_codes %lld < %lld", name, (long long)o->ld_codes, (long long)cols);
    }
    const int64_t scols = rowwise ? cols / 32 : cols;
    if (o->ld_scales < scols)
        return fail(MXQ_ERR_SHAPE, "%s ld_scales %lld < %lld", name, (long long)o->ld_scales, (long long)scols);
    if (!aligned(o->codes, 16) || o->ld_codes % 16 != 0)
        return fail(MXQ_ERR_ALIGN, "%s codes pointer and ld_codes must be multiples of 16 bytes", name);
    if (!rowwise && (!aligned(o->scales, 8) || o->ld_scales % 8 != 0))
        return fail(MXQ_ERR_ALIGN, "%s colwise scales pointer and ld_scales must be multiples of 8 bytes", name);
    if (!extent_ok(rows, o->ld_codes, 1) || !extent_ok(srows, o->ld_scales, 1))
        return fail(MXQ_ERR_OVERFLOW, "%s output extent too large", name);
    if (plane != 0) outs.push_back(range_kblock(o->codes, cols / 64, plane, rows * 64, "row codes"));
    else outs.push_back(range2d(o->codes, rows, cols, o->ld_codes, 1, rowwise ? "row codes" : "col codes"));
    outs.push_back(range2d(o->scales, srows, scols, o->ld_scales, 1, rowwise ? "row scales" : "col scales"));
    return MXQ_OK;
}

mxq_status check_bf16_in(const uint16_t *p, int64_t M, int64_t K, int64_t ld, const char *name,
                         std::vector<Range> &ins) {
    if (p == nullptr) return fail(MXQ_ERR_NULL, "%s is NULL", name);
    if (ld < K) return fail(MXQ_ERR_SHAPE, "%s ld %lld < K %lld", name, (long long)ld, (long long)K);
    if (!aligned(p, 16) || ld % 8 != 0)
        return fail(MXQ_ERR_ALIGN, "%s pointer and row pitch must be multiples of 16 bytes", name);
    if (!extent_ok(M, ld, 2)) return fail(MXQ_ERR_OVERFLOW, "%s extent too large", name);
    ins.push_back(range2d(p, M, K, ld, 2, name));
    return MXQ_OK;
}

struct GroupsOut {
    mxq::Groups g{0, nullptr, nullptr};
};

mxq_status check_groups(const mxq_groups *groups, bool need_blocks, GroupsOut &out, std::vector<Range> &ins) {
    if (groups == nullptr) return MXQ_OK;
    if (groups->G < 1 || groups->G > (int64_t(1) << 24))
        return fail(MXQ_ERR_SHAPE, "groups->G = %lld must be in [1, 2^24]", (long long)groups->G);
    if (groups->row_off == nullptr || (need_blocks && groups->block_off == nullptr))
        return fail(MXQ_ERR_NULL, "groups->row_off%s is NULL", need_blocks ? " or groups->block_off" : "");
    if (!aligned(groups->row_off, 8) || (groups->block_off && !aligned(groups->block_off, 8)))
        return fail(MXQ_ERR_ALIGN, "group offset arrays must be 8-byte aligned");
    out.g = mxq::Groups{groups->G, groups->row_off, groups->block_off};
    ins.push_back(range2d(groups->row_off, 1, groups->G + 1, groups->G + 1, 8, "row_off"));
    if (groups->block_off) ins.push_back(range2d(groups->block_off, 1, groups->G + 1, groups->G + 1, 8, "block_off"));
    return MXQ_OK;
}

// Checks the GLU interleave block il of an activation kind (0: none): only
// gated kinds take one, a positive multiple of 32 dividing K.
mxq_status check_interleave(int act_kind, int il, int64_t K) {
    if (il == 0) return MXQ_OK;
    if (act_kind != mxq::ACT_SWIGLU && act_kind != mxq::ACT_CLAMPED)
        return fail(MXQ_ERR_SHAPE, "glu_interleave applies to SwiGLU and clamped SwiGLU only");
    if (il < 0 || il % 32 != 0 || (K > 0 && K % il != 0))
        return fail(MXQ_ERR_SHAPE, "glu_interleave = %d must be a positive multiple of 32 dividing K = %lld", il,
                    (long long)K);
    return MXQ_OK;
}

// Columns one gate (or up) view spans in memory: K, or 2K - il interleaved.
int64_t gate_span(int64_t K, int il) { return il ? 2 * K - il : K; }

// Validate and pack the shared part of fwd / quantize.
mxq_status prepare_fwd(mxq::FwdArgs &a, int act_kind, float limit, int il, int64_t M, int64_t K,
                       const uint16_t *gate, int64_t ld_gate, const uint16_t *up, int64_t ld_up,
                       const float *row_scale, const mxq_groups *groups, uint32_t dirs,
                       const mxq_mx_out *row_out, const mxq_mx_out *col_out, bool *noop,
                       bool dense = false, uint16_t *h = nullptr, int64_t ld_h = 0) {
    *noop = false;
    if (M < 0 || K < 0) return fail(MXQ_ERR_SHAPE, "M = %lld and K = %lld must be >= 0", (long long)M, (long long)K);
    if (K % 32 != 0) return fail(MXQ_ERR_SHAPE, "K = %lld must be a multiple of 32", (long long)K);
    mxq_status si = check_interleave(act_kind, il, K);
    if (si != MXQ_OK) return si;
    if (act_kind == mxq::ACT_SRELU && up != nullptr) return fail(MXQ_ERR_SHAPE, "SReLU is unary: up must be NULL");
    if (dirs > 3 || (dirs == 0 && !dense))
        return fail(MXQ_ERR_SHAPE, "dirs = %u must be ROWWISE, COLWISE or both%s", dirs, dense ? ", or 0" : "");
    if (act_kind == mxq::ACT_CLAMPED && !(limit > 0.0f))
        return fail(MXQ_ERR_SHAPE, "clamped SwiGLU needs a limit > 0");
    if (act_kind != mxq::ACT_IDENTITY && row_scale != nullptr && !aligned(row_scale, 4))
        return fail(MXQ_ERR_ALIGN, "row_scale must be 4-byte aligned");
    std::vector<Range> ins, outs;
    GroupsOut go;
    mxq_status s = check_groups(groups, (dirs & 2) != 0, go, ins);
    if (s != MXQ_OK) return s;
    if (M == 0 || K == 0) {
        *noop = true;
        return MXQ_OK;
    }
    if (M > (int64_t(1) << 40) || K > (int64_t(1) << 30))
        return fail(MXQ_ERR_OVERFLOW, "M or K beyond the supported range");
    const bool gated = act_kind == mxq::ACT_SWIGLU || act_kind == mxq::ACT_CLAMPED;
    s = check_bf16_in(gate, M, gate_span(K, il), ld_gate, gated ? "gate" : "x", ins);
    if (s != MXQ_OK) return s;
    if (gated) {
        s = check_bf16_in(up, M, gate_span(K, il), ld_up, "up", ins);
        if (s != MXQ_OK) return s;
    }
    if (act_kind != mxq::ACT_IDENTITY && row_scale) ins.push_back(range2d(row_scale, 1, M, M, 4, "row_scale"));
    const int64_t G = go.g.G;
    if (dirs & 1) {
        s = check_mx_out(row_out, true, M, K, M, "rowwise", outs);
        if (s != MXQ_OK) return s;
    } else if (row_out != nullptr && row_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "row_out given but dirs has no ROWWISE");
    }
    if (dirs & 2) {
        // the exact scale-row count sum_g ceil(m_g/32) is known only on the
        // device; the alias check covers the ceil(M/32) rows that always exist
        s = check_mx_out(col_out, false, M, K, (M + 31) / 32, "colwise", outs);
        if (s != MXQ_OK) return s;
    } else if (col_out != nullptr && col_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "col_out given but dirs has no COLWISE");
    }
    if (dense) {
        if (h == nullptr) return fail(MXQ_ERR_NULL, "h is NULL (mxq_swiglu_quantize_fwd writes no dense output)");
        if (ld_h < K) return fail(MXQ_ERR_SHAPE, "h ld %lld < K %lld", (long long)ld_h, (long long)K);
        if (!aligned(h, 16) || ld_h % 8 != 0)
            return fail(MXQ_ERR_ALIGN, "h pointer and row pitch must be multiples of 16 bytes");
        if (!extent_ok(M, ld_h, 2)) return fail(MXQ_ERR_OVERFLOW, "h extent too large");
        outs.push_back(range2d(h, M, K, ld_h, 2, "h"));
    }
    // launch bound: HIP's grid x block must stay below 2^32 work-items
    if (mxq::act_quant_launch_threads(M, K, G, (dirs & 2) && G > 0, false) >= (int64_t(1) << 32))
        return fail(MXQ_ERR_OVERFLOW, "launch beyond 2^32 work-items");
    s = check_alias(ins, outs);
    if (s != MXQ_OK) return s;
    a.act = act_kind;
    a.limit = limit;
    a.M = M;
    a.K = K;
    a.gate = gate;
    a.ld_gate = ld_gate;
    a.up = gated ? up : nullptr;
    a.ld_up = ld_up;
    a.il = il;
    a.row_scale = act_kind == mxq::ACT_IDENTITY ? nullptr : row_scale;
    a.groups = go.g;
    a.dirs = dirs;
    a.row = (dirs & 1) ? mxq::MxOut{row_out->codes, row_out->ld_codes, row_out->scales, row_out->ld_scales, row_out->kblock_plane}
                       : mxq::MxOut{nullptr, 0, nullptr, 0, 0};
    a.col = (dirs & 2) ? mxq::MxOut{col_out->codes, col_out->ld_codes, col_out->scales, col_out->ld_scales, 0}
                       : mxq::MxOut{nullptr, 0, nullptr, 0, 0};
    a.h = h;
    a.ld_h = ld_h;
    return MXQ_OK;
}

int act_from(const mxq_act *act, float *limit, int *il) {
    *limit = 7.0f;
    *il = 0;
    if (act == nullptr) return mxq::ACT_SWIGLU;
    *limit = act->limit;
    *il = act->glu_interleave;
    switch (act->kind) {
        case MXQ_ACT_SWIGLU: return mxq::ACT_SWIGLU;
        case MXQ_ACT_CLAMPED_SWIGLU: return mxq::ACT_CLAMPED;
        case MXQ_ACT_SRELU: return mxq::ACT_SRELU;
        default: return -1;
    }
}

}  // namespace

namespace {

// Footprint of G stacked (rows x cols) arrays with row pitch ld and group
// stride gstride (elements): one 2-D range for a single group, else the whole
// interval from the first element to the last.
Range range_groups(const void *p, int64_t G, int64_t gstride, int64_t rows, int64_t cols, int64_t ld, int64_t esize,
                   const char *name) {
    if (G <= 1 || p == nullptr || rows <= 0 || cols <= 0) return range2d(p, rows, cols, ld, esize, name);
    Range r;
    r.name = name;
    r.lo = reinterpret_cast<uintptr_t>(p);
    r.hi = r.lo + (uintptr_t)(((G - 1) * gstride + (rows - 1) * ld + cols) * esize);
    return r;
}

// The output of a grouped GEMM must not overlap any input (its operands,
// their scales, the offsets).  With accumulate the output is read too, which
// is allowed: it is compared with the inputs only.
mxq_status check_gemm_alias(const mxq_gemm_args &a) {
    if (a.M == 0 || a.N == 0) return MXQ_OK;
    const bool f8 = a.A.dtype == MXQ_DTYPE_MXFP8_E4M3;
    const int64_t esz = f8 ? 1 : 2, osz = a.out_dtype == MXQ_DTYPE_F32 ? 4 : 2;
    std::vector<Range> ins;
    ins.push_back(range2d(a.row_off, 1, a.G + 1, a.G + 1, 8, "row_off"));
    if (a.block_off) ins.push_back(range2d(a.block_off, 1, a.G + 1, a.G + 1, 8, "block_off"));
    Range out;
    if (a.mode == MXQ_GEMM_TN) {
        // colwise scales: the ceil(rows/32) scale rows that always exist
        const int64_t nb = (a.rows + 31) / 32;
        ins.push_back(range2d(a.A.data, a.rows, a.M, a.A.ld, esz, "A"));
        ins.push_back(range2d(a.B.data, a.rows, a.N, a.B.ld, esz, "B"));
        if (f8) {
            ins.push_back(range2d(a.A.scales, nb, a.M, a.A.ld_scales, 1, "A scales"));
            ins.push_back(range2d(a.B.scales, nb, a.N, a.B.ld_scales, 1, "B scales"));
        }
        out = range_groups(a.out, a.G, a.out_gstride, a.M, a.N, a.ld_out, osz, "out");
    } else {
        const int64_t kb = (a.K + 31) / 32;
        if (a.A.kblock_plane > 0) ins.push_back(range_kblock(a.A.data, a.K * esz / 64, a.A.kblock_plane, a.M * 64, "A"));
        else ins.push_back(range2d(a.A.data, a.M, a.K, a.A.ld, esz, "A"));
        if (f8) ins.push_back(range2d(a.A.scales, a.M, kb, a.A.ld_scales, 1, "A scales"));
        if (a.mode == MXQ_GEMM_NT) {
            if (a.B.kblock_plane > 0)
                ins.push_back(range_kblock(a.B.data, a.K * esz / 64, a.B.kblock_plane,
                                           (a.G - 1) * a.B.gstride * esz + a.N * 64, "B"));
            else ins.push_back(range_groups(a.B.data, a.G, a.B.gstride, a.N, a.K, a.B.ld, esz, "B"));
            if (f8) ins.push_back(range_groups(a.B.scales, a.G, a.B.scale_gstride, a.N, kb, a.B.ld_scales, 1, "B scales"));
        } else {
            ins.push_back(range_groups(a.B.data, a.G, a.B.gstride, a.K, a.N, a.B.ld, esz, "B"));
            if (f8) ins.push_back(range_groups(a.B.scales, a.G, a.B.scale_gstride, kb, a.N, a.B.ld_scales, 1, "B scales"));
        }
        out = range2d(a.out, a.M, a.N, a.ld_out, osz, "out");
    }
    return check_alias(ins, {out});
}

}  // namespace

extern "C" {

const char *mxq_version(void) { return "mxq 0.1.0 (gfx950)"; }

const char *mxq_last_error_message(void) { return g_last_error.c_str(); }

const char *mxq_status_string(mxq_status s) {
    switch (s) {
        case MXQ_OK: return "MXQ_OK";
        case MXQ_ERR_NULL: return "MXQ_ERR_NULL";
        case MXQ_ERR_SHAPE: return "MXQ_ERR_SHAPE";
        case MXQ_ERR_ALIGN: return "MXQ_ERR_ALIGN";
        case MXQ_ERR_OVERFLOW: return "MXQ_ERR_OVERFLOW";
        case MXQ_ERR_ALIAS: return "MXQ_ERR_ALIAS";
        case MXQ_ERR_UNSUPPORTED: return "MXQ_ERR_UNSUPPORTED";
        case MXQ_ERR_HIP: return "MXQ_ERR_HIP";
        case MXQ_ERR_WORKSPACE: return "MXQ_ERR_WORKSPACE";
    }
    return "unknown mxq_status";
}

mxq_status mxq_splits_to_offsets(const int64_t *splits, int64_t G, int64_t *row_off, int64_t *block_off,
                                 int32_t *err_flag, void *stream) {
    if (splits == nullptr || row_off == nullptr) return fail(MXQ_ERR_NULL, "splits and row_off are required");
    if (G < 1 || G > (int64_t(1) << 20)) return fail(MXQ_ERR_SHAPE, "G = %lld must be in [1, 2^20]", (long long)G);
    if (!aligned(splits, 8) || !aligned(row_off, 8) || (block_off && !aligned(block_off, 8)) ||
        (err_flag && !aligned(err_flag, 4)))
        return fail(MXQ_ERR_ALIGN, "offset arrays must be 8-byte aligned (err_flag 4-byte)");
    std::vector<Range> ins{range2d(splits, 1, G, G, 8, "splits")};
    std::vector<Range> outs{range2d(row_off, 1, G + 1, G + 1, 8, "row_off")};
    if (block_off) outs.push_back(range2d(block_off, 1, G + 1, G + 1, 8, "block_off"));
    if (err_flag) outs.push_back(range2d(err_flag, 1, 1, 1, 4, "err_flag"));
    mxq_status s = check_alias(ins, outs);
    if (s != MXQ_OK) return s;
    return hip_status(mxq::launch_splits_to_offsets(splits, G, row_off, block_off, err_flag, (hipStream_t)stream),
                      "mxq_splits_to_offsets launch");
}

mxq_status mxq_swiglu_quantize_fwd(const mxq_act *act, int64_t M, int64_t K, const uint16_t *gate, int64_t ld_gate,
                                   const uint16_t *up, int64_t ld_up, const float *row_scale,
                                   const mxq_groups *groups, uint32_t dirs, const mxq_mx_out *row_out,
                                   const mxq_mx_out *col_out, void *stream) {
    float limit;
    int il;
    const int kind = act_from(act, &limit, &il);
    if (kind < 0) return fail(MXQ_ERR_UNSUPPORTED, "unknown activation kind %d", act->kind);
    mxq::FwdArgs a{};
    bool noop;
    mxq_status s = prepare_fwd(a, kind, limit, il, M, K, gate, ld_gate, up, ld_up, row_scale, groups, dirs, row_out,
                               col_out, &noop);
    if (s != MXQ_OK || noop) return s == MXQ_OK ? ok() : s;
    return hip_status(mxq::launch_act_quant_fwd(a, (hipStream_t)stream), "mxq_swiglu_quantize_fwd launch");
}

mxq_status mxq_swiglu_fwd_bf16(const mxq_act *act, int64_t M, int64_t K, const uint16_t *gate, int64_t ld_gate,
                               const uint16_t *up, int64_t ld_up, const float *row_scale, const mxq_groups *groups,
                               uint32_t dirs, const mxq_mx_out *row_out, const mxq_mx_out *col_out, uint16_t *h,
                               int64_t ld_h, void *stream) {
    float limit;
    int il;
    const int kind = act_from(act, &limit, &il);
    if (kind < 0) return fail(MXQ_ERR_UNSUPPORTED, "unknown activation kind %d", act->kind);
    mxq::FwdArgs a{};
    bool noop;
    mxq_status s = prepare_fwd(a, kind, limit, il, M, K, gate, ld_gate, up, ld_up, row_scale, groups, dirs, row_out,
                               col_out, &noop, true, h, ld_h);
    if (s != MXQ_OK || noop) return s == MXQ_OK ? ok() : s;
    return hip_status(mxq::launch_act_quant_fwd(a, (hipStream_t)stream), "mxq_swiglu_fwd_bf16 launch");
}

mxq_status mxq_quantize(int64_t M, int64_t K, const uint16_t *x, int64_t ld_x, const mxq_groups *groups,
                        uint32_t dirs, const mxq_mx_out *row_out, const mxq_mx_out *col_out, void *stream) {
    mxq::FwdArgs a{};
    bool noop;
    mxq_status s = prepare_fwd(a, mxq::ACT_IDENTITY, 0.0f, 0, M, K, x, ld_x, nullptr, 0, nullptr, groups, dirs,
                               row_out, col_out, &noop);
    if (s != MXQ_OK || noop) return s == MXQ_OK ? ok() : s;
    return hip_status(mxq::launch_act_quant_fwd(a, (hipStream_t)stream), "mxq_quantize launch");
}

mxq_status mxq_quantize_noop(int64_t M, int64_t K, const uint16_t *x, int64_t ld_x, const mxq_groups *groups,
                             uint32_t dirs, const mxq_mx_out *row_out, const mxq_mx_out *col_out,
                             const int32_t *noop_flag, void *stream) {
    if (noop_flag != nullptr && !aligned(noop_flag, 4)) return fail(MXQ_ERR_ALIGN, "noop_flag must be 4-byte aligned");
    mxq::FwdArgs a{};
    bool noop;
    mxq_status s = prepare_fwd(a, mxq::ACT_IDENTITY, 0.0f, 0, M, K, x, ld_x, nullptr, 0, nullptr, groups, dirs,
                               row_out, col_out, &noop);
    if (s != MXQ_OK || noop) return s == MXQ_OK ? ok() : s;
    if (noop_flag != nullptr) {
        // the flag is an input: no output may overlap it
        std::vector<Range> outs;
        if (dirs & 1) {
            if (row_out->kblock_plane > 0)
                outs.push_back(range_kblock(row_out->codes, K / 64, row_out->kblock_plane, M * 64, "row codes"));
            else outs.push_back(range2d(row_out->codes, M, K, row_out->ld_codes, 1, "row codes"));
            outs.push_back(range2d(row_out->scales, M, K / 32, row_out->ld_scales, 1, "row scales"));
        }
        if (dirs & 2) {
            outs.push_back(range2d(col_out->codes, M, K, col_out->ld_codes, 1, "col codes"));
            outs.push_back(range2d(col_out->scales, (M + 31) / 32, K, col_out->ld_scales, 1, "col scales"));
        }
        if ((s = check_alias({range2d(noop_flag, 1, 1, 1, 4, "noop_flag")}, outs)) != MXQ_OK) return s;
    }
    a.noop = noop_flag;
    return hip_status(mxq::launch_act_quant_fwd(a, (hipStream_t)stream), "mxq_quantize_noop launch");
}

mxq_status mxq_swiglu_quantize_bwd_workspace(int64_t M, int64_t K, uint32_t dirs, size_t *bytes) {
    (void)dirs;
    if (bytes == nullptr) return fail(MXQ_ERR_NULL, "bytes is NULL");
    if (M < 0 || K < 0 || K % 32 != 0) return fail(MXQ_ERR_SHAPE, "M, K must be >= 0 and K % 32 == 0");
    *bytes = (M == 0 || K == 0) ? 0 : mxq::bwd_workspace_bytes(M, K);
    return ok();
}

mxq_status mxq_swiglu_quantize_bwd(const mxq_act *act, int64_t M, int64_t K, const uint16_t *grad, int64_t ld_grad,
                                   const uint16_t *gate, int64_t ld_gate, const uint16_t *up, int64_t ld_up,
                                   const float *row_scale, const mxq_groups *groups, uint16_t *dgate,
                                   int64_t ld_dgate, uint16_t *dup, int64_t ld_dup, float *dscale, uint32_t dirs,
                                   const mxq_mx_out *row_out, const mxq_mx_out *col_out, void *ws,
                                   size_t ws_bytes, void *stream) {
    float limit;
    int il;
    const int kind = act_from(act, &limit, &il);
    if (kind < 0) return fail(MXQ_ERR_UNSUPPORTED, "unknown activation kind %d", act->kind);
    if (M < 0 || K < 0) return fail(MXQ_ERR_SHAPE, "M = %lld and K = %lld must be >= 0", (long long)M, (long long)K);
    if (K % 32 != 0) return fail(MXQ_ERR_SHAPE, "K = %lld must be a multiple of 32", (long long)K);
    if (dirs > 3) return fail(MXQ_ERR_SHAPE, "dirs = %u must be 0, ROWWISE, COLWISE or both", dirs);
    mxq_status si = check_interleave(kind, il, K);
    if (si != MXQ_OK) return si;
    const bool unary = kind == mxq::ACT_SRELU;
    if (unary) {
        if (up != nullptr || dup != nullptr) return fail(MXQ_ERR_SHAPE, "SReLU is unary: up and dup must be NULL");
    } else if ((dgate == nullptr) != (dup == nullptr)) {
        return fail(MXQ_ERR_NULL, "dgate and dup must both be given or both NULL");
    }
    if (il && dgate != nullptr && (dup != dgate + il || ld_dup != ld_dgate))
        return fail(MXQ_ERR_SHAPE, "with glu_interleave = %d the gradient is interleaved too: dup must be dgate + %d "
                    "with the same pitch", il, il);
    const int64_t KO = unary ? K : 2 * K;   // columns of the MXFP8 gradient
    if (dirs == 0 && dgate == nullptr && dscale == nullptr)
        return fail(MXQ_ERR_SHAPE, "nothing requested: dirs = 0 with no dense output and no dscale");
    if (kind == mxq::ACT_CLAMPED && !(limit > 0.0f)) return fail(MXQ_ERR_SHAPE, "clamped SwiGLU needs a limit > 0");
    std::vector<Range> ins, outs;
    GroupsOut go;
    mxq_status s = check_groups(groups, (dirs & 2) != 0, go, ins);
    if (s != MXQ_OK) return s;
    if (M == 0 || K == 0) return ok();
    if (M > (int64_t(1) << 40) || K > (int64_t(1) << 30))
        return fail(MXQ_ERR_OVERFLOW, "M or K beyond the supported range");
    if ((s = check_bf16_in(grad, M, K, ld_grad, "grad", ins)) != MXQ_OK) return s;
    if ((s = check_bf16_in(gate, M, gate_span(K, il), ld_gate, unary ? "x" : "gate", ins)) != MXQ_OK) return s;
    if (!unary && (s = check_bf16_in(up, M, gate_span(K, il), ld_up, "up", ins)) != MXQ_OK) return s;
    if (row_scale) {
        if (!aligned(row_scale, 4)) return fail(MXQ_ERR_ALIGN, "row_scale must be 4-byte aligned");
        ins.push_back(range2d(row_scale, 1, M, M, 4, "row_scale"));
    }
    if (dgate && unary) {
        if (ld_dgate < K) return fail(MXQ_ERR_SHAPE, "ld of dx must be >= K");
        if (!aligned(dgate, 16) || ld_dgate % 8 != 0)
            return fail(MXQ_ERR_ALIGN, "the dx pointer and pitch must be multiples of 16 bytes");
        if (!extent_ok(M, ld_dgate, 2)) return fail(MXQ_ERR_OVERFLOW, "dx extent too large");
        outs.push_back(range2d(dgate, M, K, ld_dgate, 2, "dx"));
    } else if (dgate) {
        const int64_t span = gate_span(K, il);
        if (ld_dgate < span || ld_dup < span) return fail(MXQ_ERR_SHAPE, "ld_dgate / ld_dup too small");
        if (!aligned(dgate, 16) || !aligned(dup, 16) || ld_dgate % 8 != 0 || ld_dup % 8 != 0)
            return fail(MXQ_ERR_ALIGN, "dgate / dup pointers and pitches must be multiples of 16 bytes");
        if (!extent_ok(M, ld_dgate, 2) || !extent_ok(M, ld_dup, 2))
            return fail(MXQ_ERR_OVERFLOW, "dgate / dup extent too large");
        if (il) {
            // the interleaved [dgate | dup] is one (M x 2K) output
            outs.push_back(range2d(dgate, M, 2 * K, ld_dgate, 2, "dgate|dup"));
        } else {
            outs.push_back(range2d(dgate, M, K, ld_dgate, 2, "dgate"));
            outs.push_back(range2d(dup, M, K, ld_dup, 2, "dup"));
        }
    }
    if (dscale) {
        if (!aligned(dscale, 4)) return fail(MXQ_ERR_ALIGN, "dscale must be 4-byte aligned");
        outs.push_back(range2d(dscale, 1, M, M, 4, "dscale"));
        const size_t need = mxq::bwd_workspace_bytes(M, K);
        if (need > 0) {
            if (ws == nullptr || ws_bytes < need)
                return fail(MXQ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws == nullptr ? (size_t)0 : ws_bytes);
            if (!aligned(ws, 4)) return fail(MXQ_ERR_ALIGN, "workspace must be 4-byte aligned");
            outs.push_back(range2d(ws, 1, (int64_t)need, (int64_t)need, 1, "workspace"));
        }
    }
    const int64_t G = go.g.G;
    if (dirs & 1) {
        if ((s = check_mx_out(row_out, true, M, KO, M, "rowwise", outs)) != MXQ_OK) return s;
    } else if (row_out != nullptr && row_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "row_out given but dirs has no ROWWISE");
    }
    if (dirs & 2) {
        if ((s = check_mx_out(col_out, false, M, KO, (M + 31) / 32, "colwise", outs)) != MXQ_OK)
            return s;
    } else if (col_out != nullptr && col_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "col_out given but dirs has no COLWISE");
    }
    if (mxq::act_quant_launch_threads(M, K, G, (dirs & 2) && G > 0, true) >= (int64_t(1) << 32))
        return fail(MXQ_ERR_OVERFLOW, "launch beyond 2^32 work-items");
    if ((s = check_alias(ins, outs)) != MXQ_OK) return s;

    mxq::BwdArgs a{};
    a.act = kind;
    a.limit = limit;
    a.M = M;
    a.K = K;
    a.grad = grad; a.ld_grad = ld_grad;
    a.gate = gate; a.ld_gate = ld_gate;
    a.up = unary ? nullptr : up; a.ld_up = ld_up;
    a.il = il;
    a.row_scale = row_scale;
    a.groups = go.g;
    a.dgate = dgate; a.ld_dgate = ld_dgate;
    a.dup = dup; a.ld_dup = ld_dup;
    a.dscale = dscale;
    a.dirs = dirs;
    a.row = (dirs & 1) ? mxq::MxOut{row_out->codes, row_out->ld_codes, row_out->scales, row_out->ld_scales, row_out->kblock_plane}
                       : mxq::MxOut{nullptr, 0, nullptr, 0, 0};
    a.col = (dirs & 2) ? mxq::MxOut{col_out->codes, col_out->ld_codes, col_out->scales, col_out->ld_scales, 0}
                       : mxq::MxOut{nullptr, 0, nullptr, 0, 0};
    a.partials = static_cast<float *>(ws);
    return hip_status(mxq::launch_act_quant_bwd(a, (hipStream_t)stream), "mxq_swiglu_quantize_bwd launch");
}

mxq_status mxq_swiglu_quantize_bwd_noalloc(const mxq_act *act, int64_t M, int64_t K, const uint16_t *grad,
                                           int64_t ld_grad, const uint16_t *gate, int64_t ld_gate,
                                           const uint16_t *up, int64_t ld_up, const float *row_scale,
                                           const mxq_groups *groups, uint16_t *dgate, int64_t ld_dgate,
                                           uint16_t *dup, int64_t ld_dup, float *dscale, uint32_t dirs,
                                           const mxq_mx_out *row_out, const mxq_mx_out *col_out, void *stream) {
    // the size check needs no device; the scratch's address is looked up
    // only for a call that fits it
    const size_t need = (dscale != nullptr && M > 0 && K > 0 && K % 32 == 0) ? mxq::bwd_workspace_bytes(M, K) : 0;
    const size_t cap = mxq::bwd_scratch_capacity();
    if (need > cap)
        return fail(MXQ_ERR_WORKSPACE,
                    "the allocation-free backward needs %zu bytes of scratch for dscale at M = %lld, K = %lld; "
                    "the library's scratch holds %zu (use mxq_swiglu_quantize_bwd with a workspace)",
                    need, (long long)M, (long long)K, cap);
    float *scratch = nullptr;
    if (need > 0) {
        const hipError_t e = mxq::bwd_scratch(&scratch);
        if (e != hipSuccess) return hip_status(e, "mxq_swiglu_quantize_bwd_noalloc scratch lookup");
    }
    return mxq_swiglu_quantize_bwd(act, M, K, grad, ld_grad, gate, ld_gate, up, ld_up, row_scale, groups, dgate,
                                   ld_dgate, dup, ld_dup, dscale, dirs, row_out, col_out, scratch,
                                   need > 0 ? cap : 0, stream);
}

// K-grouped launches keep one counter of their dynamic tile order in the
// workspace (256 bytes keep the allocation's alignment simple).
static size_t gemm_ws_bytes(const mxq_gemm_args &a) { return a.mode == MXQ_GEMM_TN ? 256 : 0; }


mxq_status mxq_grouped_gemm_workspace(const mxq_gemm_args *args, size_t *bytes) {
    if (args == nullptr || bytes == nullptr) return fail(MXQ_ERR_NULL, "args and bytes are required");
    *bytes = gemm_ws_bytes(*args);
    return ok();
}

mxq_status mxq_grouped_gemm(const mxq_gemm_args *args, void *ws, size_t ws_bytes, void *stream) {
    if (args == nullptr) return fail(MXQ_ERR_NULL, "args is NULL");
    mxq::GemmArgs g{};
    std::string err;
    const int st = mxq::gemm_prepare(*args, g, err);
    if (st != MXQ_OK) return fail((mxq_status)st, "%s", err.c_str());
    if (check_gemm_alias(*args) != MXQ_OK) return MXQ_ERR_ALIAS;
    const size_t need = gemm_ws_bytes(*args);
    if (need > 0) {
        if (ws == nullptr || ws_bytes < need)
            return fail(MXQ_ERR_WORKSPACE, "the workspace needs %zu bytes (got %zu)", need, ws == nullptr ? (size_t)0 : ws_bytes);
        if ((reinterpret_cast<uintptr_t>(ws) & 3u) != 0) return fail(MXQ_ERR_ALIGN, "the workspace must be 4-byte aligned");
        g.sched = static_cast<int *>(ws);
    }
    if (g.noop) return ok();
    return hip_status(mxq::launch_grouped_gemm(g, (hipStream_t)stream), "mxq_grouped_gemm launch");
}

mxq_status mxq_grouped_gemm_swiglu(const mxq_gemm_args *args, const mxq_act *act, const float *row_scale,
                                   uint32_t dirs, const mxq_mx_out *row_out, const mxq_mx_out *col_out,
                                   void *stream) {
    if (args == nullptr || act == nullptr) return fail(MXQ_ERR_NULL, "args and act are required");
    mxq::GemmArgs g{};
    std::string err;
    const int st = mxq::gemm_prepare(*args, g, err);
    if (st != MXQ_OK) return fail((mxq_status)st, "%s", err.c_str());
    if (args->mode != MXQ_GEMM_NT || args->A.dtype != MXQ_DTYPE_BF16 || args->out_dtype != MXQ_DTYPE_BF16)
        return fail(MXQ_ERR_UNSUPPORTED, "the fused SwiGLU epilogue is built for bf16 NT GEMMs with a bf16 output");
    float limit;
    int il;
    const int kind = act_from(act, &limit, &il);
    if (kind != mxq::ACT_SWIGLU && kind != mxq::ACT_CLAMPED)
        return fail(MXQ_ERR_UNSUPPORTED, "the fused epilogue computes SwiGLU or clamped SwiGLU");
    if (il != 128)
        return fail(MXQ_ERR_SHAPE, "the fused epilogue needs B's gate and up rows interleaved in blocks of 128 "
                    "(act->glu_interleave = 128), got %d", il);
    if (args->N % 256 != 0) return fail(MXQ_ERR_SHAPE, "N = %lld must be a multiple of 256", (long long)args->N);
    if (kind == mxq::ACT_CLAMPED && !(limit > 0.0f)) return fail(MXQ_ERR_SHAPE, "clamped SwiGLU needs a limit > 0");
    if (dirs < 1 || dirs > 3) return fail(MXQ_ERR_SHAPE, "dirs = %u must be ROWWISE, COLWISE or both", dirs);
    if ((dirs & 2) && args->block_off == nullptr)
        return fail(MXQ_ERR_NULL, "colwise output needs block_off (the groups' first colwise scale rows)");
    if (row_scale != nullptr && !aligned(row_scale, 4)) return fail(MXQ_ERR_ALIGN, "row_scale must be 4-byte aligned");
    const int64_t M = args->M, KA = args->N / 2;
    std::vector<Range> ins, outs;
    mxq_status s;
    if (dirs & 1) {
        if (row_out != nullptr && row_out->kblock_plane != 0)
            return fail(MXQ_ERR_UNSUPPORTED, "the fused FC1 epilogue writes row-major rowwise codes (kblock_plane 0)");
        if ((s = check_mx_out(row_out, true, M, KA, M, "rowwise", outs)) != MXQ_OK) return s;
    } else if (row_out != nullptr && row_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "row_out given but dirs has no ROWWISE");
    }
    if (dirs & 2) {
        if ((s = check_mx_out(col_out, false, M, KA, (M + 31) / 32, "colwise", outs)) != MXQ_OK) return s;
    } else if (col_out != nullptr && col_out->codes != nullptr) {
        return fail(MXQ_ERR_SHAPE, "col_out given but dirs has no COLWISE");
    }
    if (check_gemm_alias(*args) != MXQ_OK) return MXQ_ERR_ALIAS;
    // the activation's outputs against every input and the bf16 output
    ins.push_back(range2d(args->A.data, M, args->K, args->A.ld, 2, "A"));
    ins.push_back(range_groups(args->B.data, args->G, args->B.gstride, args->N, args->K, args->B.ld, 2, "B"));
    ins.push_back(range2d(args->row_off, 1, args->G + 1, args->G + 1, 8, "row_off"));
    if (args->block_off) ins.push_back(range2d(args->block_off, 1, args->G + 1, args->G + 1, 8, "block_off"));
    if (row_scale) ins.push_back(range2d(row_scale, 1, M, M, 4, "row_scale"));
    outs.push_back(range2d(args->out, M, args->N, args->ld_out, 2, "out"));
    if ((s = check_alias(ins, outs)) != MXQ_OK) return s;
    if (g.noop) return ok();
    g.epi_act = kind == mxq::ACT_CLAMPED ? 2 : 1;
    g.epi_limit = limit;
    g.epi_scale = row_scale;
    g.epi_dirs = dirs;
    if (dirs & 1) {
        g.epi_rc = row_out->codes; g.epi_ld_rc = row_out->ld_codes;
        g.epi_rs = row_out->scales; g.epi_ld_rs = row_out->ld_scales;
    }
    if (dirs & 2) {
        g.epi_cc = col_out->codes; g.epi_ld_cc = col_out->ld_codes;
        g.epi_cs = col_out->scales; g.epi_ld_cs = col_out->ld_scales;
    }
    return hip_status(mxq::launch_grouped_gemm(g, (hipStream_t)stream), "mxq_grouped_gemm_swiglu launch");
}

}  // extern "C"
