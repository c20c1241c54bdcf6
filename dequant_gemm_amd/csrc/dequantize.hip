// dequantize.hip -- NF4 dequantization to bf16 (or fp32).
//
// "bitsandbytes" page, double-quantization paragraph: the scaling factors are
// dequantized first (a^ = fp32(fp32(q * s) + mu)) and then used to
// dequantize the weights, W^ = bf16_rne(fp32(level[code] * a^)).
// Streaming kernels.  bf16 output: each lane turns 16 bytes of packed codes
// (32 elements, within one block of 32 or more) into 64 bytes of bf16 through the per-block
// register table of the 16 values bf16(level_i * a^), the same table the fused
// GEMMs use.  fp32 output: each lane turns one 32-bit word of codes (eight
// elements) into 32 bytes of fp32.
#include "nf4_launch.h"

namespace nf4 {
namespace {

// bf16 kernel: a wave works on tiles of 1 KiB of codes (2,048 elements).  Lane l
// loads the 16-byte chunk l of the tile (32 elements, inside one block) and
// dequantizes it into four 16-byte output chunks; these pass through LDS so
// that each store instruction of the wave writes 1 KiB contiguously (lane l
// stores output chunk 64j + l of the tile in store j).
constexpr int kDqTiles = 2;              // tiles per wave and iteration, all loaded first
constexpr int kDqWaves = 4;
constexpr int kDqRow = 5;                // LDS row of a lane: four chunks plus one of padding

// Orders this wave's LDS accesses before and after the call (wavefront scope).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <bool DQ, bool FP4>
__global__ __launch_bounds__(64 * kDqWaves) void dequantize_bf16_kernel(const uint8_t *__restrict__ packed,
                                                                        AbsmaxSrc src, int64_t n32,
                                                                        uint4 *__restrict__ out) {
  __shared__ uint4 stage[kDqWaves][64 * kDqRow];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint4 *st = stage[wave];
  const float mu = DQ ? *src.mean : 0.f;
  const int64_t ntiles = (n32 + 63) / 64;
  const int64_t nwaves = (int64_t)gridDim.x * kDqWaves;
  for (int64_t t0 = ((int64_t)blockIdx.x * kDqWaves + wave) * kDqTiles; t0 < ntiles; t0 += nwaves * kDqTiles) {
    uint4 c[kDqTiles];
    AbsmaxRaw r[kDqTiles];
#pragma unroll
    for (int u = 0; u < kDqTiles; ++u) {
      const int64_t g = (t0 + u) * 64 + lane;        // this lane's 16-byte code chunk
      const int64_t gc = g < n32 ? g : n32 - 1;
      c[u] = reinterpret_cast<const uint4 *>(packed)[gc];
      r[u] = load_raw<DQ>(src, gc >> (src.lbs - 5));   // chunk gc starts at element 32 gc
    }
    // every load is issued before the first conversion of an int8 absmax
    __builtin_amdgcn_sched_barrier(0);
    uint4 o[kDqTiles][4];
#pragma unroll
    for (int u = 0; u < kDqTiles; ++u) {
      const Lut tab = make_lut<FP4>(ahat_of(r[u], DQ, mu));
      const uint32_t w[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Sel4 sa, sb;
        select8(w[j], sa, sb);
        lookup4(sa, tab, o[u][j].x, o[u][j].y);
        lookup4(sb, tab, o[u][j].z, o[u][j].w);
      }
    }
    // Stores last: they count against the same counter as the loads, so a store
    // issued before a tile is dequantized would be waited for with that tile's
    // loads.  The empty asm pins every output word here, ahead of all stores.
#pragma unroll
    for (int u = 0; u < kDqTiles; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        asm volatile("" : "+v"(o[u][j].x), "+v"(o[u][j].y), "+v"(o[u][j].z), "+v"(o[u][j].w));
    const int64_t nout = 4 * n32;                    // 16-byte output chunks in total
#pragma unroll
    for (int u = 0; u < kDqTiles; ++u) {
      const int64_t t = t0 + u;                      // past the last tile every oi >= nout
#pragma unroll
      for (int j = 0; j < 4; ++j) st[lane * kDqRow + j] = o[u][j];
      wave_sync();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int src_lane = 16 * j + (lane >> 2);
        const uint4 v = st[src_lane * kDqRow + (lane & 3)];
        const int64_t oi = t * 256 + 64 * j + lane;
        if (oi < nout) out[oi] = v;
      }
      wave_sync();
    }
  }
}

template <bool OUT_BF16, bool FP4>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ packed,
                                                         AbsmaxSrc src, int64_t numel,
                                                         void *__restrict__ out, int64_t start) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = lvl<FP4>(threadIdx.x);
  __syncthreads();
  const float mu = src.dq ? *src.mean : 0.f;
  const int64_t n8 = numel / 8;
  for (int64_t g = start / 8 + (int64_t)blockIdx.x * 256 + threadIdx.x; g < n8; g += (int64_t)gridDim.x * 256) {
    const uint32_t d = *reinterpret_cast<const uint32_t *>(packed + g * 4);
    const float ah = block_ahat(src, (g * 8) >> src.lbs, mu);
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
      const float v = __fmul_rn(lv[code], block_ahat(src, e >> src.lbs, mu));
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
  if (out_is_bf16) {
    // whole 32-element chunks by the table kernel, the rest (fewer than 32
    // elements) by the element-wise kernel
    const int64_t n32 = numel / 32;
    if (n32 > 0) {
      const int64_t per_wg = 64 * kDqTiles * kDqWaves;   // 16-byte code chunks per workgroup and iteration
      int64_t grid = (n32 + per_wg - 1) / per_wg;
      if (grid > 65536) grid = 65536;
      auto kern = src.qt ? (src.dq ? dequantize_bf16_kernel<true, true> : dequantize_bf16_kernel<false, true>)
                         : (src.dq ? dequantize_bf16_kernel<true, false> : dequantize_bf16_kernel<false, false>);
      hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * kDqWaves), 0, stream, packed, src, n32,
                         reinterpret_cast<uint4 *>(out));
    }
    if (numel % 32) {
      const int64_t done = n32 * 32;
      auto tail = src.qt ? dequantize_kernel<true, true> : dequantize_kernel<true, false>;
      hipLaunchKernelGGL(tail, dim3(1), dim3(256), 0, stream, packed, src, numel, out, done);
    }
    return hipGetLastError();
  }
  const int64_t n8 = numel / 8;
  int64_t grid = (n8 + 255) / 256;
  if (grid > 16384) grid = 16384;
  if (grid < 1) grid = 1;
  auto kern = src.qt ? dequantize_kernel<false, true> : dequantize_kernel<false, false>;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), 0, stream, packed, src, numel, out,
                     (int64_t)0);
  return hipGetLastError();
}

}  // namespace nf4
