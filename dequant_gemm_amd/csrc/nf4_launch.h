// nf4_launch.h -- host-side launchers implemented by the kernel sources and
// called by the C ABI in nf4_api.hip.  All arguments are validated by the
// caller; launchers only configure grids and enqueue on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_common.h"

namespace nf4 {

// Workspace layout for quantization with double quantization: one row of
// kMeanSlots exact-mean accumulators per quantize workgroup (at most
// kQuantGridMax workgroups of kQuantThreads; the last workgroup's row also
// holds the partial block at the end), then the fp32 absmax of every block.
constexpr int kQuantThreads = 1024;
constexpr int kQuantGridMax = 512;
constexpr int kMeanSlots = 16;
constexpr size_t kPartialBytes = (size_t)kQuantGridMax * kMeanSlots * sizeof(unsigned long long);
constexpr size_t absmax_ws_offset() { return (kPartialBytes + 255) & ~(size_t)255; }
constexpr size_t quant_workspace_bytes(int64_t nblocks) {
  return (absmax_ws_offset() + (size_t)nblocks * sizeof(float) + 255) & ~(size_t)255;
}

// `lbs`: log2 of the block size (5..8); `fp4`: the FP4 level table instead of NF4's.
hipError_t launch_quantize(const void *w, int w_is_bf16, int64_t numel, int lbs, bool fp4, uint8_t *packed,
                           float *absmax_out, unsigned long long *partials, uint32_t *status,
                           int dq, int8_t *q_out, float *scale_out, float *mean_out,
                           hipStream_t stream);

hipError_t launch_dequantize(const uint8_t *packed, const AbsmaxSrc &src, int64_t numel,
                             void *out, int out_is_bf16, hipStream_t stream);

// `lr.r == 0`: no adapter term.
hipError_t launch_fwd(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                      const AbsmaxSrc &src, const LowRank &lr, void *y, int y_is_bf16, hipStream_t stream);

hipError_t launch_bwd_dx(const void *dy, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                         const AbsmaxSrc &src, const LowRank &lr, void *dx, int dx_is_bf16,
                         hipStream_t stream);

// C = alpha op(A) op(B), bf16 operands, fp32 accumulation (adapter.hip).
hipError_t launch_adapter_gemm(int ta, int tb, int64_t M, int64_t N, int64_t K, float alpha, const void *a,
                               int64_t lda, bool va, const void *b, int64_t ldb, bool vb, void *c, int64_t ldc,
                               bool c_bf16, hipStream_t stream);

}  // namespace nf4
