// Internal interface of the grouped GEMM (validation in gemm_prepare, kernels in
// grouped_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "mxq.h"

namespace mxq {

struct GemmOperand {
    int dtype;              // MXQ_DTYPE_BF16 / MXQ_DTYPE_MXFP8_E4M3
    const void *data;
    int64_t ld, gstride;
    const uint8_t *scales;
    int64_t ld_scales, scale_gstride;
};

struct GemmArgs {
    int mode;               // mxq_gemm_mode
    int64_t G;
    const int64_t *row_off, *block_off;
    int64_t M, N, K, rows;
    GemmOperand A, B;
    int out_dtype;
    void *out;
    int64_t ld_out, out_gstride;
    int accumulate;
    int max_workgroups;
    int *sched;             // K-grouped: device counter of the dynamic tile order (workspace)
    bool noop;
};

// Validates the public arguments; returns an mxq_status and an error text.
int gemm_prepare(const mxq_gemm_args &in, GemmArgs &out, std::string &err);
hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream);

}  // namespace mxq
