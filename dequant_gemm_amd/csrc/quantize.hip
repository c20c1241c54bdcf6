// quantize.hip -- NF4 blockwise quantization with double quantization.
//
// "Zenbit" page, section "What's inside", bullet zenbit.nf4 (NF4 blockwise
// quantization with double quantization); "bitsandbytes" page, NF4 data-type
// paragraph (absmax normalisation, nearest of 16 levels via lookup tables) and
// double-quantization paragraph (absmax per 64-weight block, the absmax values
// quantized to 8 bits with their own meta-scales).
//
// Kernels, in launch order:
//   zero_u64_kernel          clears the 256 exact-mean accumulators
//   quantize_blocks_kernel   full 64-blocks: absmax, codes, packing, accumulators
//   quantize_tail_kernel     the one partial block at the end, if any
//   mean_finalize_kernel     exact mean of all absmax values, one rounding
//   double_quant_kernel      int8 absmax and one fp32 scale per 256 blocks
#include "nf4_launch.h"

namespace nf4 {
namespace {

// ---------------------------------------------------------------- level search
//
// The normalised value n lies in [-1, 1].  [-1, 1+1/64) is cut into 129 cells
// of width 1/64; no cell holds more than one threshold and every threshold is
// more than 2e-4 away from a cell edge, so for n in cell j
//   code(n) = base_j + (n >= thr_j).
// A fast path forms n from one reciprocal per block (n' within 2^-22
// relative of the exact quotient); values n' within 2^-20 relative of the
// threshold of their cell are re-done with the IEEE division.

struct Cell {
  float thr;   // threshold inside the cell, +inf if none
  float lo;    // thr - tolerance
  float hi;    // thr + tolerance
  int base;    // code of the cell's lower edge
};

__device__ void build_cells(Cell *tab) {
  for (int j = threadIdx.x; j < 129; j += blockDim.x) {
    const float lo = -1.0f + (float)j * 0.015625f;
    const float hi = lo + 0.015625f;
    int base = 0;
    float thr = __builtin_inff();
#pragma unroll
    for (int i = 0; i < 15; ++i) {
      const float t = threshold(i);
      if (t <= lo)
        ++base;
      else if (t < hi)
        thr = t;
    }
    Cell c;
    c.thr = thr;
    c.base = base;
    if (thr == __builtin_inff()) {
      c.lo = thr;
      c.hi = thr;
    } else {
      const float tol = fabsf(thr) * 0x1p-20f;
      c.lo = thr - tol;
      c.hi = thr + tol;
    }
    tab[j] = c;
  }
}

__device__ __forceinline__ int classify(float n, const Cell *tab, bool &near) {
  const float f = (n + 1.0f) * 64.0f;
  int j = (int)f;
  j = j < 0 ? 0 : (j > 128 ? 128 : j);
  const Cell c = tab[j];
  near |= (n > c.lo) && (n < c.hi);
  return c.base + (n >= c.thr ? 1 : 0);
}

// Codes of eight values of one block with absmax bits `m` (finite, non-zero).
__device__ __forceinline__ uint32_t encode8(const float x[8], uint32_t m, const Cell *cells) {
  const float a = __uint_as_float(m);
  int code[8];
  bool near = false;
  if (m >= 0x01000000u && m < 0x7e000000u) {  // 2^-125 <= a < 2^125: 1/a is a normal float
    const float r = __builtin_amdgcn_rcpf(a);
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = classify(x[i] * r, cells, near);
  } else {
    near = true;
  }
  if (near) {
    bool unused = false;
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = classify(x[i] / a, cells, unused);
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)code[i] << (4 * i);
  return word;
}

__global__ void zero_u64_kernel(unsigned long long *p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0ull;
}

// Eight lanes per block, eight elements per lane.  Each lane's eight codes
// form one 32-bit word of the packed output (element 2j in the low nibble of
// byte j).  With double quantization the block absmax is also accumulated,
// exactly, as integer significand sums per binary exponent.
template <bool BF16, bool DQ>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(
    const void *__restrict__ w, int64_t nfull, uint8_t *__restrict__ packed,
    float *__restrict__ absmax, unsigned long long *__restrict__ buckets, uint32_t *status) {
  __shared__ Cell cells[129];
  __shared__ unsigned long long lbuck[256];
  build_cells(cells);
  if (DQ) lbuck[threadIdx.x] = 0ull;
  __syncthreads();

  const int part = threadIdx.x & 7;
  const int slot = threadIdx.x >> 3;
  bool bad = false;
  for (int64_t blk = (int64_t)blockIdx.x * 32 + slot; blk < nfull; blk += (int64_t)gridDim.x * 32) {
    float x[8];
    if (BF16) {
      const uint4 raw = *reinterpret_cast<const uint4 *>(
          reinterpret_cast<const uint16_t *>(w) + blk * kBlock + part * 8);
      x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
      x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
      x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
      x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
    } else {
      const float4 *p = reinterpret_cast<const float4 *>(
          reinterpret_cast<const float *>(w) + blk * kBlock + part * 8);
      const float4 u = p[0], v = p[1];
      x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
      x[4] = v.x; x[5] = v.y; x[6] = v.z; x[7] = v.w;
    }
    // absmax on the magnitude bits: integer order equals float order for
    // non-negative floats, and NaN/inf compare above every finite value
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    m = max(m, (uint32_t)__shfl_xor((int)m, 1));
    m = max(m, (uint32_t)__shfl_xor((int)m, 2));
    m = max(m, (uint32_t)__shfl_xor((int)m, 4));

    uint32_t word;
    if (m >= 0x7f800000u) {
      bad = true;
      word = 0x77777777u;
    } else if (m == 0) {
      word = 0x77777777u;  // all-zero block: every code is level 0.0
    } else {
      word = encode8(x, m, cells);
    }
    *reinterpret_cast<uint32_t *>(packed + blk * (kBlock / 2) + part * 4) = word;
    if (part == 0) {
      absmax[blk] = __uint_as_float(m);
      if (DQ && m < 0x7f800000u) {
        const uint32_t e = m >> 23;
        const unsigned long long sig = (m & 0x7fffffu) | (e ? 0x800000u : 0u);
        atomicAdd(&lbuck[e], sig);
      }
    }
  }
  if (DQ) {
    __syncthreads();
    const unsigned long long v = lbuck[threadIdx.x];
    if (v) atomicAdd(&buckets[threadIdx.x], v);
  }
  if (bad && status) atomicOr(status, 1u);
}

// The partial block at the end (fewer than 64 elements): one wave, one
// element per lane, exact division.
template <bool BF16, bool DQ>
__global__ __launch_bounds__(64) void quantize_tail_kernel(
    const void *__restrict__ w, int64_t numel, int64_t blk, uint8_t *__restrict__ packed,
    float *__restrict__ absmax, unsigned long long *__restrict__ buckets, uint32_t *status) {
  __shared__ Cell cells[129];
  build_cells(cells);
  __syncthreads();
  const int lane = threadIdx.x;
  const int64_t e = blk * kBlock + lane;
  const bool valid = e < numel;
  float x = 0.f;
  if (valid) {
    if (BF16)
      x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(w)[e] << 16);
    else
      x = reinterpret_cast<const float *>(w)[e];
  }
  uint32_t m = __float_as_uint(x) & 0x7fffffffu;
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, s));
  int code = 7;
  if (m != 0 && m < 0x7f800000u) {
    bool unused = false;
    code = classify(x / __uint_as_float(m), cells, unused);
  }
  if (!valid) code = 0;
  const int upper = __shfl_down(code, 1);
  if (valid && (lane & 1) == 0) packed[blk * (kBlock / 2) + lane / 2] = (uint8_t)(code | (upper << 4));
  if (lane == 0) {
    absmax[blk] = __uint_as_float(m);
    if (m >= 0x7f800000u) {
      if (status) atomicOr(status, 1u);
    } else if (DQ) {
      const uint32_t ex = m >> 23;
      atomicAdd(&buckets[ex], (unsigned long long)((m & 0x7fffffu) | (ex ? 0x800000u : 0u)));
    }
  }
}

// Exact mean of all block absmax values, rounded once to fp32 (nearest-even).
// Every finite fp32 is an integer number of 2^-149 units; bucket e holds the
// sum of the 24-bit significands of the values with biased exponent e, worth
// 2^(max(e,1)-1) units each.  The sum S (at most ~310 bits) is divided by the
// block count as a multi-word integer with 32 extra quotient bits, enough to
// reach below the smallest subnormal, then rounded on the remainder.
__global__ void mean_finalize_kernel(const unsigned long long *__restrict__ buckets,
                                     uint32_t nblocks, float *__restrict__ mean_out) {
  if (threadIdx.x != 0) return;
  constexpr int W = 13;
  uint32_t num[W];
#pragma unroll
  for (int i = 0; i < W; ++i) num[i] = 0;
  for (int e = 0; e < 256; ++e) {
    const unsigned long long v = buckets[e];
    if (!v) continue;
    const int sh = (e > 0 ? e : 1) - 1 + 32;  // S * 2^32
    const int wi = sh >> 5, bi = sh & 31;
    const unsigned long long lo = v << bi;
    const uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), bi ? (uint32_t)(v >> (64 - bi)) : 0u};
    unsigned long long carry = 0;
    for (int i = wi; i < W; ++i) {
      const unsigned long long add = (i - wi < 3) ? part[i - wi] : 0ull;
      const unsigned long long s = (unsigned long long)num[i] + add + carry;
      num[i] = (uint32_t)s;
      carry = s >> 32;
      if (i - wi >= 2 && carry == 0) break;
    }
  }
  uint32_t q[W];
  unsigned long long rem = 0;
  for (int i = W - 1; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | num[i];
    q[i] = (uint32_t)(cur / nblocks);
    rem = cur % nblocks;
  }
  int L = 0;
  for (int i = W - 1; i >= 0; --i)
    if (q[i]) {
      L = 32 * i + (32 - __clz(q[i]));
      break;
    }
  uint32_t bits = 0;
  if (L > 0) {
    int p = L - 24 > 32 ? L - 24 : 32;  // lsb kept: 24 bits, or the 2^-149 unit
    auto bit = [&](int i) -> uint32_t { return i < 0 ? 0u : (q[i >> 5] >> (i & 31)) & 1u; };
    uint32_t kept = 0;
    for (int b = 0; b < 24; ++b) kept |= bit(p + b) << b;
    const uint32_t round = bit(p - 1);
    uint32_t sticky = rem != 0 ? 1u : 0u;
    for (int i = 0; i < p - 1 && !sticky; ++i) sticky |= bit(i);
    if (round && (sticky || (kept & 1u))) ++kept;
    if (kept == (1u << 24)) {
      kept >>= 1;
      ++p;
    }
    // value = kept * 2^(p - 181)
    if (kept >= (1u << 23))
      bits = ((uint32_t)(p - 31) << 23) | (kept & 0x7fffffu);
    else
      bits = kept;  // subnormal (p == 32)
  }
  *mean_out = __uint_as_float(bits);
}

// One wave per group of 256 absmax values.
__global__ __launch_bounds__(64) void double_quant_kernel(const float *__restrict__ absmax,
                                                          int64_t nblocks,
                                                          const float *__restrict__ mean,
                                                          int8_t *__restrict__ q_out,
                                                          float *__restrict__ scale_out) {
  const int lane = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kGroup + lane * 4;
  const float mu = *mean;
  float ac[4];
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ac[i] = (base + i < nblocks) ? __fsub_rn(absmax[base + i], mu) : 0.f;
    m = fmaxf(m, fabsf(ac[i]));
  }
#pragma unroll
  for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
  const float s = __fdiv_rn(m, 127.0f);
  if (lane == 0) scale_out[blockIdx.x] = s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (base + i >= nblocks) break;
    int qv = 0;
    if (m != 0.f) {
      float r = rintf(__fdiv_rn(ac[i], s));
      r = fminf(fmaxf(r, -127.f), 127.f);
      qv = (int)r;
    }
    q_out[base + i] = (int8_t)qv;
  }
}

}  // namespace

hipError_t launch_quantize(const void *w, int w_is_bf16, int64_t numel, uint8_t *packed,
                           float *absmax_out, unsigned long long *buckets, uint32_t *status,
                           int dq, int8_t *q_out, float *scale_out, float *mean_out,
                           hipStream_t stream) {
  const int64_t nblocks = (numel + kBlock - 1) / kBlock;
  const int64_t nfull = numel / kBlock;
  if (dq) hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(256), 0, stream, buckets, 256);
  if (nfull > 0) {
    int64_t grid = (nfull + 31) / 32;
    if (grid > 8192) grid = 8192;
    const dim3 g((unsigned)grid), b(256);
    if (w_is_bf16) {
      if (dq) hipLaunchKernelGGL((quantize_blocks_kernel<true, true>), g, b, 0, stream, w, nfull, packed, absmax_out, buckets, status);
      else    hipLaunchKernelGGL((quantize_blocks_kernel<true, false>), g, b, 0, stream, w, nfull, packed, absmax_out, buckets, status);
    } else {
      if (dq) hipLaunchKernelGGL((quantize_blocks_kernel<false, true>), g, b, 0, stream, w, nfull, packed, absmax_out, buckets, status);
      else    hipLaunchKernelGGL((quantize_blocks_kernel<false, false>), g, b, 0, stream, w, nfull, packed, absmax_out, buckets, status);
    }
  }
  if (nfull < nblocks) {
    const dim3 g(1), b(64);
    if (w_is_bf16) {
      if (dq) hipLaunchKernelGGL((quantize_tail_kernel<true, true>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, buckets, status);
      else    hipLaunchKernelGGL((quantize_tail_kernel<true, false>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, buckets, status);
    } else {
      if (dq) hipLaunchKernelGGL((quantize_tail_kernel<false, true>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, buckets, status);
      else    hipLaunchKernelGGL((quantize_tail_kernel<false, false>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, buckets, status);
    }
  }
  if (dq) {
    hipLaunchKernelGGL(mean_finalize_kernel, dim3(1), dim3(64), 0, stream, buckets, (uint32_t)nblocks, mean_out);
    const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
    hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)ngroups), dim3(64), 0, stream, absmax_out, nblocks, mean_out, q_out, scale_out);
  }
  return hipGetLastError();
}

}  // namespace nf4
