// offsets.hip -- splits -> offsets on the device (page "Activation +
// GroupedLinear Fusion for MOE and other MOE optimizations", Greptile Summary
// and Sequence Diagram: every per-group offset array is computed once, up
// front, from the split sizes, instead of base-offset arithmetic at each use).
//
// One workgroup of 1024 lanes: each lane sums a contiguous run of splits,
// the run totals are scanned in LDS (Hillis-Steele, int64), and each lane
// writes the exclusive prefix sums of its run.  Integer arithmetic throughout,
// so the result is exact and independent of the lane count.
#include "mxq_internal.h"

namespace mxq {
namespace {

constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kScanThreads)
splits_to_offsets_kernel(const int64_t *splits, int64_t G, int64_t *row_off, int64_t *block_off,
                         int32_t *err_flag) {
    __shared__ int64_t s_rows[kScanThreads];
    __shared__ int64_t s_blks[kScanThreads];
    const int tid = threadIdx.x;
    const int64_t per = (G + kScanThreads - 1) / kScanThreads;
    const int64_t b = tid * per;
    const int64_t e = b + per < G ? b + per : G;
    int64_t sr = 0, sb = 0;
    bool neg = false;
    for (int64_t i = b; i < e; i++) {
        const int64_t v = splits[i];
        neg |= v < 0;
        sr += v;
        sb += (v + 31) / 32;  // ceil(v / 32) for v >= 0
    }
    s_rows[tid] = sr;
    s_blks[tid] = sb;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int64_t ar = tid >= off ? s_rows[tid - off] : 0;
        const int64_t ab = tid >= off ? s_blks[tid - off] : 0;
        __syncthreads();
        s_rows[tid] += ar;
        s_blks[tid] += ab;
        __syncthreads();
    }
    // exclusive prefix of this lane's run
    int64_t pr = tid > 0 ? s_rows[tid - 1] : 0;
    int64_t pb = tid > 0 ? s_blks[tid - 1] : 0;
    if (tid == 0) {
        row_off[0] = 0;
        if (block_off) block_off[0] = 0;
    }
    for (int64_t i = b; i < e; i++) {
        const int64_t v = splits[i];
        pr += v;
        pb += (v + 31) / 32;
        row_off[i + 1] = pr;
        if (block_off) block_off[i + 1] = pb;
    }
    if (neg && err_flag) *err_flag = 1;
}

}  // namespace

hipError_t launch_splits_to_offsets(const int64_t *splits, int64_t G, int64_t *row_off,
                                    int64_t *block_off, int32_t *err_flag, hipStream_t stream) {
    hipLaunchKernelGGL(splits_to_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, splits, G,
                       row_off, block_off, err_flag);
    return hipGetLastError();
}

}  // namespace mxq
