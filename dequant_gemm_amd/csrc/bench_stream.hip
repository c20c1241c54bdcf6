// bench_stream.hip -- the plain HBM read stream of libnf4_bench (include/nf4_bench.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nf4_bench.h"

namespace {

__global__ void read_stream_kernel(const uint4 *__restrict__ src, size_t n16, uint32_t *__restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  // four loads in flight per thread and pass
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = src[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

extern "C" int nf4bench_read_stream(const void *src, size_t bytes, uint32_t *sink, int grid, int block, void *stream) {
  if (!src || !sink || bytes == 0 || (bytes & 15) != 0) return 1;
  if (((uintptr_t)src & 15) != 0 || ((uintptr_t)sink & 15) != 0) return 1;
  if (!(block == 64 || block == 128 || block == 256 || block == 512 || block == 1024)) return 1;
  if (grid < 1 || grid > 65536) return 1;
  hipLaunchKernelGGL(read_stream_kernel, dim3((unsigned)grid), dim3((unsigned)block), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const uint4 *>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
