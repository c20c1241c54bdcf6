// dequantize.hip -- NF4 dequantization to bf16 (or fp32).
//
// "bitsandbytes" page, double-quantization paragraph: the scaling factors are
// dequantized first (a^ = fp32(fp32(q * s) + mu)) and then used to
// dequantize the weights, W^ = bf16_rne(fp32(level[code] * a^)).
// Streaming kernel: each lane turns one 32-bit word of packed codes (eight
// elements) into 16 bytes of bf16 (or 32 bytes of fp32).
#include "nf4_launch.h"

namespace nf4 {
namespace {

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ packed,
                                                         AbsmaxSrc src, int64_t numel,
                                                         void *__restrict__ out) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = level(threadIdx.x);
  __syncthreads();
  const float mu = src.dq ? *src.mean : 0.f;
  const int64_t n8 = numel / 8;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < n8; g += (int64_t)gridDim.x * 256) {
    const uint32_t d = *reinterpret_cast<const uint32_t *>(packed + g * 4);
    const float ah = block_ahat(src, g >> 3, mu);
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __fmul_rn(lv[(d >> (4 * j)) & 15u], ah);
    if (OUT_BF16) {
      uint4 o;
      o.x = pack_bf16x2(v[0], v[1]);
      o.y = pack_bf16x2(v[2], v[3]);
      o.z = pack_bf16x2(v[4], v[5]);
      o.w = pack_bf16x2(v[6], v[7]);
      reinterpret_cast<uint4 *>(out)[g] = o;
    } else {
      float4 *o = reinterpret_cast<float4 *>(out) + 2 * g;
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
  // the last numel % 8 elements
  if (blockIdx.x == 0) {
    for (int64_t e = n8 * 8 + threadIdx.x; e < numel; e += 256) {
      const uint8_t byte = packed[e >> 1];
      const uint32_t code = (e & 1) ? (byte >> 4) : (byte & 15u);
      const float v = __fmul_rn(lv[code], block_ahat(src, e / kBlock, mu));
      if (OUT_BF16)
        reinterpret_cast<uint16_t *>(out)[e] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
      else
        reinterpret_cast<float *>(out)[e] = v;
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t *packed, const AbsmaxSrc &src, int64_t numel,
                             void *out, int out_is_bf16, hipStream_t stream) {
  const int64_t n8 = numel / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  if (out_is_bf16)
    hipLaunchKernelGGL((dequantize_kernel<true>), dim3((unsigned)grid), dim3(256), 0, stream, packed, src, numel, out);
  else
    hipLaunchKernelGGL((dequantize_kernel<false>), dim3((unsigned)grid), dim3(256), 0, stream, packed, src, numel, out);
  return hipGetLastError();
}

}  // namespace nf4
