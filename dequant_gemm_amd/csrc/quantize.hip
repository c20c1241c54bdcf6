// quantize.hip -- NF4 blockwise quantization with double quantization.
//
// "Zenbit" page, section "What's inside", bullet zenbit.nf4 (NF4 blockwise
// quantization with double quantization); "bitsandbytes" page, NF4 data-type
// paragraph (absmax normalisation, nearest of 16 levels via lookup tables) and
// double-quantization paragraph (absmax per 64-weight block, the absmax values
// quantized to 8 bits with their own meta-scales).
//
// Kernels, in launch order:
//   quantize_blocks_kernel   full 64-blocks: absmax, codes, packing; with double
//                            quantization also one row of exact-mean
//                            accumulators per workgroup (plain stores)
//   quantize_tail_kernel     the one partial block at the end, if any (its own
//                            accumulator row)
//   mean_reduce_kernel       one workgroup: sums the rows and forms the exact
//                            mean, one rounding
//   double_quant_kernel      int8 absmax and one fp32 scale per 256 blocks
//
// Exact mean.  Every finite fp32 is an integer number of 2^-149 units: a value
// with biased exponent e and 24-bit significand m is m * 2^(max(e,1)-1) units.
// A workgroup first sums significands per exponent (LDS, 64-bit), then folds
// the 256 exponent sums into the digits of one fixed-point integer: slot i
// accumulates (64-bit, carries left unresolved) the 32-bit digit of weight
// 2^(32 i) units of every term.  The ten used slots of all rows are summed in
// 64 bits (no overflow below 2^37 elements; tensors hold at most 2^36) and the carries resolved once at
// the end: integer sums, so the result does not depend on any order.
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

// FP4 code of a normalised value n: the magnitude index counts the
// thresholds |n| lies above (a tie goes to the smaller magnitude, the lower
// code), then the sign; zero of either sign takes code 0 (+0).
__device__ __forceinline__ int fp4_code(float n) {
  const float an = fabsf(n);
  int mi = 0;
#pragma unroll
  for (int i = 0; i < 7; ++i) mi += an > fp4_threshold(i) ? 1 : 0;
  return (n < 0.f && mi > 0) ? 8 + mi : mi;
}

// FP4 codes of eight values of one block with absmax bits `m` (finite,
// non-zero): exact IEEE division, then the thresholds.
__device__ __forceinline__ uint32_t encode8_fp4(const float x[8], uint32_t m) {
  const float a = __uint_as_float(m);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)fp4_code(x[i] / a) << (4 * i);
  return word;
}

// LPB lanes per block (block size 8 * LPB: 32, 64, 128 or 256), eight
// elements per lane.  Each lane's eight codes form one 32-bit word of the
// packed output (element 2j in the low nibble of byte j).  With double quantization each workgroup also sums the significands
// of its block absmax values per binary exponent (exact integer sums) and
// stores the 256 sums as its row of `partials`.  The next block's load is in
// flight while the current block is encoded.
// Adds the exponent-e sum `v` of significands to the digit slots (see above).
__device__ __forceinline__ void add_to_slots(unsigned long long *slot, int e, unsigned long long v) {
  const int sh = (e > 0 ? e : 1) - 1;
  const int wi = sh >> 5, bi = sh & 31;
  const unsigned long long lo = v << bi;
  atomicAdd(&slot[wi], (unsigned long long)(uint32_t)lo);
  atomicAdd(&slot[wi + 1], (unsigned long long)(uint32_t)(lo >> 32));
  if (bi) atomicAdd(&slot[wi + 2], (unsigned long long)(uint32_t)(v >> (64 - bi)));
}

template <bool BF16, bool DQ, int LPB, bool FP4>
__global__ __launch_bounds__(256) void quantize_blocks_kernel(
    const void *__restrict__ w, int64_t nfull, uint8_t *__restrict__ packed,
    float *__restrict__ absmax, unsigned long long *__restrict__ partials, uint32_t *status) {
  constexpr int BS = 8 * LPB;        // weights per block
  constexpr int BPI = 256 / LPB;     // blocks per workgroup and iteration
  __shared__ Cell cells[129];
  __shared__ unsigned long long lbuck[256];
  __shared__ unsigned long long lslot[kMeanSlots];
  const int part = threadIdx.x % LPB;
  const int slot = threadIdx.x / LPB;
  const int64_t stride = (int64_t)gridDim.x * BPI;
  auto load = [&](int64_t blk, uint4 &u, uint4 &v) {
    if (BF16) {
      u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(w) + blk * BS + part * 8);
    } else {
      const uint4 *p = reinterpret_cast<const uint4 *>(reinterpret_cast<const float *>(w) + blk * BS + part * 8);
      u = p[0];
      v = p[1];
    }
  };
  bool bad = false;
  int64_t blk = (int64_t)blockIdx.x * BPI + slot;
  uint4 cu = make_uint4(0, 0, 0, 0), cv = cu;
  if (blk < nfull) load(blk, cu, cv);   // in flight while the level table is built
  if (!FP4) build_cells(cells);
  if (DQ) {
    lbuck[threadIdx.x] = 0ull;
    if (threadIdx.x < kMeanSlots) lslot[threadIdx.x] = 0ull;
  }
  __syncthreads();

  for (; blk < nfull; blk += stride) {
    uint4 nu = make_uint4(0, 0, 0, 0), nv = nu;
    const int64_t nb = blk + stride < nfull ? blk + stride : nfull - 1;
    load(nb, nu, nv);
    float x[8];
    if (BF16) {
      x[0] = bf16_lo(cu.x); x[1] = bf16_hi(cu.x);
      x[2] = bf16_lo(cu.y); x[3] = bf16_hi(cu.y);
      x[4] = bf16_lo(cu.z); x[5] = bf16_hi(cu.z);
      x[6] = bf16_lo(cu.w); x[7] = bf16_hi(cu.w);
    } else {
      x[0] = __uint_as_float(cu.x); x[1] = __uint_as_float(cu.y);
      x[2] = __uint_as_float(cu.z); x[3] = __uint_as_float(cu.w);
      x[4] = __uint_as_float(cv.x); x[5] = __uint_as_float(cv.y);
      x[6] = __uint_as_float(cv.z); x[7] = __uint_as_float(cv.w);
    }
    // absmax on the magnitude bits: integer order equals float order for
    // non-negative floats, and NaN/inf compare above every finite value
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
#pragma unroll
    for (int sh = 1; sh < LPB; sh <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, sh));

    constexpr uint32_t kZeroWord = FP4 ? 0u : 0x77777777u;   // every code the +0 level
    uint32_t word;
    if (m >= 0x7f800000u) {
      bad = true;
      word = kZeroWord;
    } else if (m == 0) {
      word = kZeroWord;  // all-zero block
    } else {
      word = FP4 ? encode8_fp4(x, m) : encode8(x, m, cells);
    }
    *reinterpret_cast<uint32_t *>(packed + blk * (BS / 2) + part * 4) = word;
    if (part == 0) {
      absmax[blk] = __uint_as_float(m);
      if (DQ && m < 0x7f800000u) {
        const uint32_t e = m >> 23;
        const unsigned long long sig = (m & 0x7fffffu) | (e ? 0x800000u : 0u);
        atomicAdd(&lbuck[e], sig);
      }
    }
    cu = nu;
    cv = nv;
  }
  if (DQ) {
    __syncthreads();
    const unsigned long long v = lbuck[threadIdx.x];
    if (v) add_to_slots(lslot, threadIdx.x, v);
    __syncthreads();
    if (threadIdx.x < kMeanSlots) partials[(int64_t)blockIdx.x * kMeanSlots + threadIdx.x] = lslot[threadIdx.x];
  }
  if (bad && status) atomicOr(status, 1u);
}

// The partial block at the end (fewer than blocksize <= 256 elements): one
// workgroup of 256 threads, one element per thread, exact division.
template <bool BF16, bool DQ, bool FP4>
__global__ __launch_bounds__(256) void quantize_tail_kernel(
    const void *__restrict__ w, int64_t numel, int64_t blk, int bs, uint8_t *__restrict__ packed,
    float *__restrict__ absmax, unsigned long long *__restrict__ partial_row, uint32_t *status) {
  __shared__ Cell cells[129];
  __shared__ uint32_t wmax[4];
  if (!FP4) build_cells(cells);
  const int t = threadIdx.x;
  const int64_t e = blk * bs + t;
  const bool valid = t < bs && e < numel;
  float x = 0.f;
  if (valid) {
    if (BF16)
      x = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(w)[e] << 16);
    else
      x = reinterpret_cast<const float *>(w)[e];
  }
  uint32_t m = __float_as_uint(x) & 0x7fffffffu;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, sh));
  if ((t & 63) == 0) wmax[t >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  int code = FP4 ? 0 : 7;   // the +0 level
  if (m != 0 && m < 0x7f800000u) {
    bool unused = false;
    code = FP4 ? fp4_code(x / __uint_as_float(m)) : classify(x / __uint_as_float(m), cells, unused);
  }
  if (!valid) code = 0;
  const int upper = __shfl_down(code, 1);
  if (valid && (t & 1) == 0) packed[(blk * bs + t) / 2] = (uint8_t)(code | (upper << 4));
  if (DQ && t < kMeanSlots) {
    // this block's accumulator row: the digits of its absmax alone
    const uint32_t ex = m >> 23;
    const unsigned long long sig = (m & 0x7fffffu) | (ex ? 0x800000u : 0u);
    const int sh = (ex > 0 ? (int)ex : 1) - 1;
    const unsigned long long lo = sig << (sh & 31);     // below 2^55
    unsigned long long d = 0;
    if (m < 0x7f800000u) {
      if (t == (sh >> 5)) d = (uint32_t)lo;
      if (t == (sh >> 5) + 1) d = lo >> 32;
    }
    partial_row[t] = d;
  }
  if (t == 0) {
    absmax[blk] = __uint_as_float(m);
    if (m >= 0x7f800000u && status) atomicOr(status, 1u);
  }
}

// Exact mean of all block absmax values, rounded once to fp32 (nearest-even),
// from the total S (in 2^-149 units) given as 32-bit digits: digit[i] has
// weight 2^(32 i).  S is divided by the block count with 32 extra quotient
// bits -- enough to reach below the smallest subnormal -- and rounded on the
// remainder.
constexpr int kMeanWords = 13;   // S * 2^32 as 32-bit digits (S < 2^(10*32 + 24))

__device__ float mean_from_digits(const uint32_t num[kMeanWords], uint32_t nblocks) {
  constexpr int W = kMeanWords;
  // long division by nblocks, one 32-bit digit at a time: the digit
  // cur / nblocks (< 2^32 since rem < nblocks) is estimated in fp64 -- cur is
  // below nblocks * 2^32, so its rounding moves the estimate by less than one
  // -- and corrected exactly with an integer multiply-subtract
  uint32_t q[W];
  unsigned long long rem = 0;
  const double inv = 1.0 / (double)nblocks;
  int top = W - 1;            // digits above the highest non-zero one give zero quotient digits
  while (top > 0 && num[top] == 0) q[top--] = 0;
  for (int i = top; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | num[i];
    long long qe = (long long)((double)cur * inv);
    long long r = (long long)(cur - (unsigned long long)qe * nblocks);
    if (r < 0) {
      --qe;
      r += nblocks;
    } else if (r >= (long long)nblocks) {
      ++qe;
      r -= nblocks;
    }
    q[i] = (uint32_t)qe;
    rem = (unsigned long long)r;
  }
  int L = 0;
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (q[i]) L = 32 * i + (32 - __clz(q[i]));
  if (L == 0) return 0.f;
  int p = L - 24 > 32 ? L - 24 : 32;  // lsb kept: 24 bits, or the 2^-149 unit
  auto bits_at = [&](int pos) -> unsigned long long {  // 64 bits of q starting at bit pos
    const int w = pos >> 5, b = pos & 31;
    unsigned long long lo = 0, mid = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if (i == w) lo = q[i];
      if (i == w + 1) mid = q[i];
      if (i == w + 2) hi = q[i];
    }
    const unsigned long long x = lo | (mid << 32);
    return b ? (x >> b) | (hi << (64 - b)) : x;
  };
  uint32_t kept = (uint32_t)(bits_at(p) & 0xffffffu);
  const uint32_t round = (uint32_t)(bits_at(p - 1) & 1u);
  // sticky: any set bit below p-1, or a non-zero remainder
  bool sticky = rem != 0;
  const int sb = p - 1;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (32 * i + 32 <= sb) sticky |= q[i] != 0;
    else if (32 * i < sb) sticky |= (q[i] & ((1u << (sb - 32 * i)) - 1u)) != 0;
  }
  if (round && (sticky || (kept & 1u))) ++kept;
  if (kept == (1u << 24)) {
    kept >>= 1;
    ++p;
  }
  // value = kept * 2^(p - 181)
  const uint32_t bits = kept >= (1u << 23) ? (((uint32_t)(p - 31) << 23) | (kept & 0x7fffffu))
                                           : kept;  // subnormal (p == 32)
  return __uint_as_float(bits);
}

// One workgroup of 1024 threads: thread t sums the 16-byte piece t % 8 (slots
// 2(t%8) and 2(t%8)+1) of rows t/8, t/8 + 128, ... (at most 2049 rows: all of a
// thread's seventeen loads in flight at once), the 128 partial sums of each
// slot are added through LDS in two stages, and one thread resolves the
// carries and forms the mean.  Integer sums: the order does not matter.
// (Two dependent rounds of 8-byte loads took ~8.4 us.)  (Spreading the loads over
// several workgroups that meet through an arrival counter measured slower: the
// fence, the atomic and the re-read cost more than the loads.)
constexpr int kMeanThreads = 1024;

__global__ __launch_bounds__(kMeanThreads) void mean_reduce_kernel(const unsigned long long *__restrict__ partials,
                                                                  int nrows, uint32_t nblocks,
                                                                  float *__restrict__ mean_out) {
  static_assert(kMeanSlots == 16, "a row is eight 16-byte pieces of two slots");
  constexpr int RL = kMeanThreads / 8;                          // 128 rows per pass
  constexpr int P = (kQuantGridMax + 1 + RL - 1) / RL;          // passes for the most rows (17)
  __shared__ unsigned long long red[RL][kMeanSlots];
  const int t = threadIdx.x, pc = t & 7, rl = t >> 3;           // slots 2pc, 2pc+1 of rows rl + 128 i
  // every load of the thread in flight at once: one memory round trip
  ulonglong2 v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int r = rl + RL * i;
    v[i] = r < nrows ? reinterpret_cast<const ulonglong2 *>(partials + (int64_t)r * kMeanSlots)[pc]
                     : make_ulonglong2(0ull, 0ull);
  }
  unsigned long long a0 = 0, a1 = 0;   // every row slot is below 2^41 and there are at most 2049 rows
#pragma unroll
  for (int i = 0; i < P; ++i) {
    a0 += v[i].x;
    a1 += v[i].y;
  }
  red[rl][2 * pc] = a0;
  red[rl][2 * pc + 1] = a1;
  __syncthreads();
  // 128 partial rows -> 16 (threads 0..255: slot t%16, rows 8(t/16) .. +7), then -> 1
  unsigned long long w = 0;
  if (t < 16 * 16) {
    const int sl = t & 15, g = t >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) w += red[8 * g + i][sl];
  }
  __syncthreads();
  if (t < 16 * 16) red[t >> 4][t & 15] = w;
  __syncthreads();
  if (t == 0) {
    // S * 2^32: digit 0 is zero, digit i + 1 is slot i after the carries
    uint32_t num[kMeanWords];
    num[0] = 0;
    unsigned long long carry = 0;
#pragma unroll
    for (int i = 0; i < kMeanWords - 1; ++i) {
      unsigned long long slot = 0;
      if (i < kMeanSlots) {
#pragma unroll
        for (int g = 0; g < 16; ++g) slot += red[g][i];
      }
      const unsigned long long cur = slot + carry;
      num[i + 1] = (uint32_t)cur;
      carry = cur >> 32;
    }
    *mean_out = mean_from_digits(num, nblocks);
  }
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


template <bool BF16, bool DQ, bool FP4>
void launch_full(int lbs, int grid, int64_t numel, int64_t nfull, int bs, hipStream_t stream, const void *w,
                 uint8_t *packed, float *absmax_out, unsigned long long *partials, uint32_t *status) {
  if (nfull > 0) {
    const dim3 g((unsigned)grid), b(256);
    switch (lbs) {
      case 5: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 4, FP4>), g, b, 0, stream, w, nfull, packed, absmax_out, partials, status); break;
      case 6: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 8, FP4>), g, b, 0, stream, w, nfull, packed, absmax_out, partials, status); break;
      case 7: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 16, FP4>), g, b, 0, stream, w, nfull, packed, absmax_out, partials, status); break;
      default: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 32, FP4>), g, b, 0, stream, w, nfull, packed, absmax_out, partials, status); break;
    }
  }
  if (nfull * bs < numel) {   // the partial last block, with its own accumulator row
    unsigned long long *row = partials ? partials + (int64_t)grid * kMeanSlots : nullptr;
    hipLaunchKernelGGL((quantize_tail_kernel<BF16, DQ, FP4>), dim3(1), dim3(256), 0, stream, w, numel, nfull, bs,
                       packed, absmax_out, row, status);
  }
}

}  // namespace

hipError_t launch_quantize(const void *w, int w_is_bf16, int64_t numel, int lbs, bool fp4, uint8_t *packed,
                           float *absmax_out, unsigned long long *partials, uint32_t *status,
                           int dq, int8_t *q_out, float *scale_out, float *mean_out,
                           hipStream_t stream) {
  const int bs = 1 << lbs;
  const int64_t nblocks = (numel + bs - 1) / bs;
  const int64_t nfull = numel / bs;
  const int bpi = 256 / (bs / 8);   // blocks per quantize workgroup and iteration
  int grid = 0;
  if (nfull > 0) {
    const int64_t g64 = (nfull + bpi - 1) / bpi;
    grid = (int)(g64 < kQuantGridMax ? g64 : kQuantGridMax);
  }
  using L = void (*)(int, int, int64_t, int64_t, int, hipStream_t, const void *, uint8_t *, float *,
                     unsigned long long *, uint32_t *);
  static const L full[2][2][2] = {{{launch_full<false, false, false>, launch_full<false, false, true>},
                                   {launch_full<false, true, false>, launch_full<false, true, true>}},
                                  {{launch_full<true, false, false>, launch_full<true, false, true>},
                                   {launch_full<true, true, false>, launch_full<true, true, true>}}};
  full[w_is_bf16 ? 1 : 0][dq ? 1 : 0][fp4 ? 1 : 0](lbs, grid, numel, nfull, bs, stream, w, packed, absmax_out,
                                                   partials, status);
  const int rows = grid + (nfull < nblocks ? 1 : 0);
  if (dq) {
    hipLaunchKernelGGL(mean_reduce_kernel, dim3(1), dim3(kMeanThreads), 0, stream, partials, rows, (uint32_t)nblocks,
                       mean_out);
    const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
    hipLaunchKernelGGL(double_quant_kernel, dim3((unsigned)ngroups), dim3(64), 0, stream, absmax_out, nblocks, mean_out, q_out, scale_out);
  }
  return hipGetLastError();
}

}  // namespace nf4
