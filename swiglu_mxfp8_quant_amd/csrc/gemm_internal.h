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
    int64_t plane;          // 0: row-major; > 0: K-blocked (either dtype), bytes between 64-byte planes
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
    // The fused SwiGLU epilogue (bf16 NT launches whose B rows hold gate and
    // up interleaved in blocks of 128, so that every 256-column output tile
    // holds 128 gate and the matching 128 up columns): the activation of the
    // tile, quantized to MXFP8 rowwise and/or colwise, besides the bf16 output.
    int epi_act;            // 0: none; 1: SwiGLU; 2: clamped SwiGLU
    float epi_limit;
    const float *epi_scale; // row scale (NULL: 1)
    unsigned epi_dirs;      // 1 rowwise, 2 colwise (scale rows through block_off), 3 both
    uint8_t *epi_rc, *epi_rs, *epi_cc, *epi_cs;   // codes / scales of each direction
    int64_t epi_ld_rc, epi_ld_rs, epi_ld_cc, epi_ld_cs;
};

// Validates the public arguments; returns an mxq_status and an error text.
int gemm_prepare(const mxq_gemm_args &in, GemmArgs &out, std::string &err);
hipError_t launch_grouped_gemm(const GemmArgs &g, hipStream_t stream);

}  // namespace mxq
