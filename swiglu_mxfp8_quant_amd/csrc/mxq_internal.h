// Internal interface between the C-ABI front end (api.cpp) and the HIP kernel
// translation units.  Not installed; the public interface is include/mxq.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace mxq {

// One direction of an MXFP8 output (device pointers, pitches in bytes).
struct MxOut {
    uint8_t *codes;
    int64_t ld_codes;
    uint8_t *scales;
    int64_t ld_scales;
    int64_t plane;      // rowwise only: 0 row-major; > 0 codes K-blocked by 64 (ld_codes 64), plane stride in bytes
};

// Row groups as seen by the kernels.  G == 0 means one implicit group of M rows.
struct Groups {
    int64_t G;
    const int64_t *row_off;
    const int64_t *block_off;
};

// ACT_SRELU is unary (x in `gate`, no `up`); ACT_IDENTITY is the plain quantizer.
enum Act { ACT_SWIGLU = 0, ACT_CLAMPED = 1, ACT_IDENTITY = 2, ACT_SRELU = 3 };

struct FwdArgs {
    int act;            // Act
    float limit;
    int64_t M, K;
    const uint16_t *gate; int64_t ld_gate;   // x for ACT_IDENTITY / ACT_SRELU
    const uint16_t *up; int64_t ld_up;       // unused for ACT_IDENTITY / ACT_SRELU
    int il;                                  // GLU interleave block (0: gate and up not interleaved)
    const float *row_scale;                  // NULL => 1
    Groups groups;
    unsigned dirs;
    MxOut row, col;
    const int32_t *noop;                     // device flag or NULL: non-zero => the launch does nothing
    uint16_t *h; int64_t ld_h;               // the activation as dense bf16 (logical columns), or NULL
};

struct BwdArgs {
    int act;
    float limit;
    int64_t M, K;
    const uint16_t *grad; int64_t ld_grad;
    const uint16_t *gate; int64_t ld_gate;
    const uint16_t *up; int64_t ld_up;       // unused for ACT_SRELU
    int il;                                  // GLU interleave block (0: none)
    const float *row_scale;
    Groups groups;
    uint16_t *dgate; int64_t ld_dgate;       // dx for ACT_SRELU
    uint16_t *dup; int64_t ld_dup;
    float *dscale;
    unsigned dirs;
    MxOut row, col;
    float *partials;    // workspace: per-row partial sums of dscale
};

// Host launchers (asynchronous on `stream`; return the hipGetLastError code).
hipError_t launch_splits_to_offsets(const int64_t *splits, int64_t G, int64_t *row_off,
                                    int64_t *block_off, int32_t *err_flag, hipStream_t stream);
hipError_t launch_act_quant_fwd(const FwdArgs &a, hipStream_t stream);
hipError_t launch_act_quant_bwd(const BwdArgs &a, hipStream_t stream);
size_t bwd_workspace_bytes(int64_t M, int64_t K);
// The allocation-free backward's scratch (a file-scope device array in
// act_quant.hip): its capacity in bytes, and its device address on the
// current device (looked up once per device).
size_t bwd_scratch_capacity();
hipError_t bwd_scratch(float **ptr);

// Work-items of the fused launch for these sizes (an upper bound when grouped;
// HIP needs grid x block below 2^32).
int64_t act_quant_launch_threads(int64_t M, int64_t K, int64_t G, bool grouped_colwise, bool backward);

// Upper bound of the number of colwise scale rows: sum_g ceil(m_g/32) <= ceil(M/32) + G.
inline int64_t colwise_block_bound(int64_t M, int64_t G) {
    return (M + 31) / 32 + (G > 0 ? G : 0);
}

}  // namespace mxq
