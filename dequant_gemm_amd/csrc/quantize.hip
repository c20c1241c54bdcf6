// quantize.hip -- NF4 blockwise quantization with double quantization.
//
// "Zenbit" page, section "What's inside", bullet zenbit.nf4 (NF4 blockwise
// quantization with double quantization); "bitsandbytes" page, NF4 data-type
// paragraph (absmax normalisation, nearest of 16 levels via lookup tables) and
// double-quantization paragraph (absmax per 64-weight block, the absmax values
// quantized to 8 bits with their own meta-scales).
//
// Kernels, in launch order:
//   quantize_blocks_kernel   absmax, codes and packing of every block (the
//                            last workgroup also takes the partial block at
//                            the end, if any); with double quantization also
//                            one row of exact-mean accumulators per workgroup
//                            (plain stores) and the fp32 absmax of every block
//   mean_dq_kernel           double quantization: each workgroup sums all the
//                            rows itself and forms the exact mean (one
//                            rounding; integer sums, so every workgroup gets
//                            the same bits), then quantizes its share of the
//                            256-block groups to int8 with one fp32 scale each
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
// relative of the exact quotient); each value n' within 2^-20 relative of the
// threshold of its cell is redone with the IEEE division.

struct Cell {
  float thr;   // threshold inside the cell, +inf if none
  int base;    // code of the cell's lower edge
};

// |n - thr| < |thr| * 2^-20: n is too close to the threshold for the fast
// quotient to decide (false for thr = +inf, where both sides are infinite).
__device__ __forceinline__ bool near_thr(float n, float thr) {
  return fabsf(n - thr) < fabsf(thr) * 0x1p-20f;
}

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
    tab[j] = c;
  }
}

__device__ __forceinline__ int classify(float n, const Cell *tab, bool &near) {
  const float f = (n + 1.0f) * 64.0f;
  int j = (int)f;
  j = j < 0 ? 0 : (j > 128 ? 128 : j);
  const Cell c = tab[j];
  near = near_thr(n, c.thr);
  return c.base + (n >= c.thr ? 1 : 0);
}

// Codes of eight values of one block with absmax bits `m` (finite, non-zero).
// An element whose fast quotient is near its cell's threshold is redone with
// the IEEE division on its own (the others keep the fast result).
__device__ __forceinline__ uint32_t encode8(const float x[8], uint32_t m, const Cell *cells) {
  const float a = __uint_as_float(m);
  int code[8];
  bool near[8];
  const bool fast = m >= 0x01000000u && m < 0x7e000000u;  // 2^-125 <= a < 2^125: 1/a is a normal float
  const float r = __builtin_amdgcn_rcpf(a);
  bool any = false;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    code[i] = classify(x[i] * r, cells, near[i]);
    near[i] = near[i] || !fast;
    any = any || near[i];
  }
  if (any) {                // rare: one branch around the per-element redo
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (near[i]) {
        bool unused;
        code[i] = classify(x[i] / a, cells, unused);
      }
    }
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)code[i] << (4 * i);
  return word;
}

// FP4: the normalised magnitude |n| in [0, 1] is cut into 25 cells of width
// 1/24 centred on multiples of 1/24.  The seven decision thresholds (the
// largest fp32 values not above the midpoints of adjacent magnitudes 1/24,
// 3/24, 5/24, 7/24, 10/24, 14/24, 20/24) each sit at a cell's centre, so a cell
// holds at most one and every one is 1/48 from its cell's edges; then
//   magnitude index(|n|) = base_j + (|n| > thr_j)
// (strictly above: a tie goes to the smaller magnitude, the lower code).  The
// sign is applied after; zero of either sign takes code 0 (+0).
//
// The comparison itself needs no quotient.  For q = |x| / a and an fp32
// threshold t, fl(q) > t exactly when q lies above the midpoint tm between t
// and the next float (or on it, when t's significand is odd: the tie rounds to
// the even neighbour).  With tm2 = tm (t even) or a double just below tm (t
// odd: no fp32 |x| lies between a * tm2 and a * tm), the decision is
// fma(-a, tm2, |x|) > 0 in fp64: the fused product-difference is rounded
// once, which keeps its sign exact.  Bit-exact ratios such as 5/24 = 160/768
// are common among bf16 weights and land on thresholds; this decides them
// without the IEEE division.
constexpr int kFp4Cells = 25;

struct Fp4Cell {
  double tm2;   // decision point (+inf if the cell holds no threshold)
  float thr;    // the threshold itself, for exact quotients
  int base;     // magnitude index of the cell's lower edge
};

__device__ void build_cells_fp4(Fp4Cell *tab) {
  for (int j = threadIdx.x; j < kFp4Cells; j += blockDim.x) {
    const float lo = ((float)j - 0.5f) * (1.0f / 24.0f);
    const float hi = ((float)j + 0.5f) * (1.0f / 24.0f);
    int base = 0;
    float thr = __builtin_inff();
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const float t = fp4_threshold(i);
      if (t < lo)
        ++base;
      else if (t < hi)
        thr = t;
    }
    Fp4Cell c;
    c.thr = thr;
    c.base = base;
    c.tm2 = __builtin_inf();
    if (thr != __builtin_inff()) {
      const uint32_t tb = __float_as_uint(thr);
      const double tm = 0.5 * ((double)thr + (double)__uint_as_float(tb + 1u));   // exact in fp64
      c.tm2 = (tb & 1u) ? tm * (1.0 - 0x1p-40) : tm;
    }
    tab[j] = c;
  }
}

// Magnitude-and-sign code of an exact quotient n.
__device__ __forceinline__ int classify_fp4(float n, const Fp4Cell *tab) {
  const float an = fabsf(n);
  int j = (int)(an * 24.0f + 0.5f);
  j = j > kFp4Cells - 1 ? kFp4Cells - 1 : j;
  const Fp4Cell c = tab[j];
  const int mi = c.base + (an > c.thr ? 1 : 0);
  return (n < 0.f && mi > 0) ? 8 + mi : mi;
}

// FP4 codes of eight values of one block with absmax bits `m` (finite,
// non-zero).  One reciprocal per block locates each value's cell (n' within
// 2^-22 relative of the quotient: the cell may be the neighbour of the exact
// one only near a cell edge, where both give the same index); the threshold
// decision is the exact fp64 test above.  A block whose reciprocal is not a
// normal float takes the IEEE division.
__device__ __forceinline__ uint32_t encode8_fp4(const float x[8], uint32_t m, const Fp4Cell *cells) {
  const float a = __uint_as_float(m);
  const bool fast = m >= 0x01000000u && m < 0x7e000000u;   // 2^-125 <= a < 2^125
  int code[8];
  if (fast) {
    const float r = __builtin_amdgcn_rcpf(a);
    const double na = -(double)a;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float ax = fabsf(x[i]);
      int j = (int)(ax * r * 24.0f + 0.5f);
      j = j > kFp4Cells - 1 ? kFp4Cells - 1 : j;
      const Fp4Cell c = cells[j];
      const int mi = c.base + (__fma_rn(na, c.tm2, (double)ax) > 0.0 ? 1 : 0);
      code[i] = (x[i] < 0.f && mi > 0) ? 8 + mi : mi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) code[i] = classify_fp4(x[i] / a, cells);
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) word |= (uint32_t)code[i] << (4 * i);
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
__global__ __launch_bounds__(kQuantThreads) void quantize_blocks_kernel(
    const void *__restrict__ w, int64_t numel, int64_t nfull, uint8_t *__restrict__ packed,
    float *__restrict__ absmax, unsigned long long *__restrict__ partials, uint32_t *status) {
  constexpr int BS = 8 * LPB;        // weights per block
  constexpr int BPI = kQuantThreads / LPB;     // blocks per workgroup and iteration
  constexpr int kWaves = kQuantThreads / 64;
  __shared__ __attribute__((aligned(16))) uint8_t celltab[129 * sizeof(Cell)];   // NF4: 129 Cells, FP4: 25 Fp4Cells
  static_assert(kFp4Cells * sizeof(Fp4Cell) <= sizeof(celltab), "FP4 cell table exceeds its buffer");
  Cell *cells = reinterpret_cast<Cell *>(celltab);
  Fp4Cell *cells4 = reinterpret_cast<Fp4Cell *>(celltab);
  __shared__ unsigned long long lbuck[256];
  __shared__ unsigned long long lslot[kMeanSlots];
  __shared__ uint32_t wmax[kWaves];
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
  auto add_absmax = [&](uint32_t m) {   // this block's absmax into the exponent sums
    const uint32_t e = m >> 23;
    const unsigned long long sig = (m & 0x7fffffu) | (e ? 0x800000u : 0u);
    atomicAdd(&lbuck[e], sig);
  };
  bool bad = false;
  int64_t blk = (int64_t)blockIdx.x * BPI + slot;
  uint4 cu = make_uint4(0, 0, 0, 0), cv = cu;
  if (blk < nfull) load(blk, cu, cv);   // in flight while the level table is built
  if (FP4)
    build_cells_fp4(cells4);
  else
    build_cells(cells);
  if (DQ) {
    if (threadIdx.x < 256) lbuck[threadIdx.x] = 0ull;
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
    if (BF16) {
      // eight bf16 magnitudes as four pairs of 16-bit integers, their maximum
      // shifted into the fp32 position (the fp32 bits of a bf16 value are its
      // bits << 16)
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      const u16x2 p0 = __builtin_bit_cast(u16x2, cu.x & 0x7fff7fffu), p1 = __builtin_bit_cast(u16x2, cu.y & 0x7fff7fffu);
      const u16x2 p2 = __builtin_bit_cast(u16x2, cu.z & 0x7fff7fffu), p3 = __builtin_bit_cast(u16x2, cu.w & 0x7fff7fffu);
      const u16x2 pm = __builtin_elementwise_max(__builtin_elementwise_max(p0, p1), __builtin_elementwise_max(p2, p3));
      m = (uint32_t)(pm.x > pm.y ? pm.x : pm.y) << 16;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, __float_as_uint(x[i]) & 0x7fffffffu);
    }
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
      word = FP4 ? encode8_fp4(x, m, cells4) : encode8(x, m, cells);
    }
    *reinterpret_cast<uint32_t *>(packed + blk * (BS / 2) + part * 4) = word;
    if (part == 0) {
      absmax[blk] = __uint_as_float(m);
      if (DQ && m < 0x7f800000u) add_absmax(m);
    }
    cu = nu;
    cv = nv;
  }

  // The partial block at the end (fewer than BS <= 256 elements), in the last
  // workgroup: one element per thread, exact division.
  if (blockIdx.x == gridDim.x - 1 && nfull * BS < numel) {
    const int t = threadIdx.x;
    const int64_t e = nfull * BS + t;
    const bool valid = t < BS && e < numel;
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
    m = wmax[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = max(m, wmax[i]);
    int code = FP4 ? 0 : 7;   // the +0 level
    if (m != 0 && m < 0x7f800000u) {
      bool unused = false;
      const float n = x / __uint_as_float(m);
      code = FP4 ? classify_fp4(n, cells4) : classify(n, cells, unused);
    }
    if (!valid) code = 0;
    const int upper = __shfl_down(code, 1);
    if (valid && (t & 1) == 0) packed[e / 2] = (uint8_t)(code | (upper << 4));
    if (t == 0) {
      absmax[nfull] = __uint_as_float(m);
      if (m >= 0x7f800000u) bad = true;
      else if (DQ) add_absmax(m);
    }
  }
  if (DQ) {
    __syncthreads();
    if (threadIdx.x < 256) {
      const unsigned long long v = lbuck[threadIdx.x];
      if (v) add_to_slots(lslot, threadIdx.x, v);
    }
    __syncthreads();
    if (threadIdx.x < kMeanSlots) partials[(int64_t)blockIdx.x * kMeanSlots + threadIdx.x] = lslot[threadIdx.x];
  }
  if (bad && status) atomicOr(status, 1u);
}

// Exact mean of all block absmax values, rounded once to fp32 (nearest-even),
// from N = S * 2^32 (S the total in 2^-149 units) given as 32-bit digits:
// num[i] has weight 2^(32 i), num[0] = 0.  The quotient N / nblocks is wanted
// to 24 significant bits, a round bit and a sticky bit.  Let T be the three
// digits from the highest non-zero one down (T >= 2^64) and R the digits below
// them, so N = T 2^k + R with k = 32 (top - 2) and R < 2^k (for top < 2, k < 0
// and R = 0).  With T = Q nblocks + rem, the true quotient is
// Q 2^k + (rem 2^k + R) / nblocks, the last term below 2^k: the quotient's bits
// from position k up are Q's, and Q has at least 33 bits (T >= 2^64,
// nblocks < 2^32), so its top 24 bits and the round bit all come from Q, and
// the sticky bit is Q's lower bits or a non-zero rem or R.  Three digit steps
// of long division instead of one per digit, and no indexing of the digits
// by a run-time value.
constexpr int kMeanWords = 13;   // S * 2^32 as 32-bit digits (S < 2^(10*32 + 24))

__host__ __device__ inline float mean_from_digits(const uint32_t num[kMeanWords], uint32_t nblocks) {
  constexpr int W = kMeanWords;
  int top = -1;
#pragma unroll
  for (int i = 0; i < W; ++i)
    if (num[i]) top = i;
  if (top < 0) return 0.f;
  uint32_t t[3] = {0u, 0u, 0u};   // T's digits, low to high
  bool rnz = false;               // R != 0
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (i == top) t[2] = num[i];
    if (i == top - 1) t[1] = num[i];
    if (i == top - 2) t[0] = num[i];
    if (i < top - 2 && num[i]) rnz = true;
  }
  const int k = 32 * (top - 2);
  // T / nblocks one 32-bit digit at a time: the digit cur / nblocks (< 2^32
  // since rem < nblocks) is estimated in fp64 -- cur is below nblocks * 2^32,
  // so its rounding moves the estimate by less than one -- and corrected
  // exactly with an integer multiply-subtract
  const double inv = 1.0 / (double)nblocks;
  uint32_t q[3];
  unsigned long long rem = 0;
#pragma unroll
  for (int i = 2; i >= 0; --i) {
    const unsigned long long cur = (rem << 32) | t[i];
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
  const unsigned long long lo = ((unsigned long long)q[1] << 32) | q[0];
  const unsigned long long hi = q[2];
  const int lq = q[2] ? 64 + 32 - __builtin_clz(q[2])
                      : (q[1] ? 32 + 32 - __builtin_clz(q[1]) : 32 - __builtin_clz(q[0]));   // >= 33
  // lsb kept: 24 bits below the leading one, or the 2^-149 unit (position 32 of the quotient)
  int p = lq + k - 24 > 32 ? lq + k - 24 : 32;
  const int pq = p - k;           // the same position in Q, >= 9
  auto bits_at = [&](int pos) -> unsigned long long {   // bits pos .. pos+63 of Q (zeros past 96)
    if (pos >= 96) return 0ull;
    if (pos >= 64) return hi >> (pos - 64);
    if (pos == 0) return lo;
    return (lo >> pos) | (hi << (64 - pos));
  };
  uint32_t kept = (uint32_t)(bits_at(pq) & 0xffffffu);
  const uint32_t round = (uint32_t)(bits_at(pq - 1) & 1u);
  const int sb = pq - 1;          // sticky: Q's bits below sb, rem, R
  bool sticky = rem != 0 || rnz;
  if (sb >= 96)
    sticky = sticky || lo != 0 || hi != 0;
  else if (sb >= 64)
    sticky = sticky || lo != 0 || (hi & ((1ull << (sb - 64)) - 1ull)) != 0;
  else if (sb > 0)
    sticky = sticky || (lo & ((1ull << sb) - 1ull)) != 0;
  if (round && (sticky || (kept & 1u))) ++kept;
  if (kept == (1u << 24)) {
    kept >>= 1;
    ++p;
  }
  // value = kept * 2^(p - 181)
  const uint32_t bits = kept >= (1u << 23) ? (((uint32_t)(p - 31) << 23) | (kept & 0x7fffffu))
                                           : kept;  // subnormal (p == 32)
  float f;
  __builtin_memcpy(&f, &bits, 4);
  return f;
}

// The exact mean of the rows' total, in every thread of a workgroup of 1024
// threads: thread t sums the 16-byte piece t % 8 (slots 2(t%8) and 2(t%8)+1)
// of rows t/8, t/8 + 128, ... (at most 512 rows: all of a thread's loads in
// flight at once), the 128 partial sums of each slot are added through LDS in
// two stages, and one thread resolves the carries and forms the mean, which
// it hands to the others through LDS.  Integer sums: the order does not
// matter, so every workgroup that runs this gets the same bits.
constexpr int kMeanThreads = 1024;

__device__ float mean_of_rows(const unsigned long long *__restrict__ partials, int nrows, uint32_t nblocks) {
  static_assert(kMeanSlots == 16, "a row is eight 16-byte pieces of two slots");
  constexpr int RL = kMeanThreads / 8;                          // 128 rows per pass
  constexpr int P = (kQuantGridMax + RL - 1) / RL;              // passes for the most rows (4)
  __shared__ unsigned long long red[RL][kMeanSlots];
  __shared__ unsigned long long slot_sum[kMeanSlots];
  __shared__ float mean_lds;
  const int t = threadIdx.x, pc = t & 7, rl = t >> 3;           // slots 2pc, 2pc+1 of rows rl + 128 i
  ulonglong2 v[P];
#pragma unroll
  for (int i = 0; i < P; ++i) {
    const int r = rl + RL * i;
    v[i] = r < nrows ? reinterpret_cast<const ulonglong2 *>(partials + (int64_t)r * kMeanSlots)[pc]
                     : make_ulonglong2(0ull, 0ull);
  }
  unsigned long long a0 = 0, a1 = 0;   // a row slot is below 96 * 2^32 and there are at most 512 rows
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
  if (t < kMeanSlots) {          // slot t over the 16 partial rows
    unsigned long long slot = 0;
#pragma unroll
    for (int g = 0; g < 16; ++g) slot += red[g][t];
    slot_sum[t] = slot;
  }
  __syncthreads();
  if (t == 0) {
    // S * 2^32: digit 0 is zero, digit i + 1 is slot i after the carries
    uint32_t num[kMeanWords];
    num[0] = 0;
    unsigned long long carry = 0;
#pragma unroll
    for (int i = 0; i < kMeanWords - 1; ++i) {
      const unsigned long long cur = (i < kMeanSlots ? slot_sum[i] : 0ull) + carry;
      num[i + 1] = (uint32_t)cur;
      carry = cur >> 32;
    }
    mean_lds = mean_from_digits(num, nblocks);
  }
  __syncthreads();
  return mean_lds;
}

// Double quantization with the mean formed in place: every workgroup (1024
// threads) computes the exact mean from the rows, workgroup 0 stores it, and
// wave w of workgroup b quantizes groups b * 16 + w, b * 16 + w + 16 * grid,
// ... of 256 absmax values: a' = fp32(a - mu), s = fp32(max|a'| / 127),
// q = clamp(rint(fp32(a' / s)), -127, 127); an all-zero group has s = 0, q = 0.
__global__ __launch_bounds__(kMeanThreads) void mean_dq_kernel(const unsigned long long *__restrict__ partials,
                                                              int nrows, const float *__restrict__ absmax,
                                                              int64_t nblocks, int8_t *__restrict__ q_out,
                                                              float *__restrict__ scale_out,
                                                              float *__restrict__ mean_out) {
  const int lane = threadIdx.x & 63;
  const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
  const int64_t step = (int64_t)gridDim.x * (kMeanThreads / 64);
  const int64_t g0 = (int64_t)blockIdx.x * (kMeanThreads / 64) + (threadIdx.x >> 6);
  // the lane's four absmax values of group g (zeros past the last block)
  auto load4 = [&](int64_t g) {
    const int64_t base = g * kGroup + lane * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (base + 3 < nblocks) {
      a = *reinterpret_cast<const float4 *>(absmax + base);
    } else {
      if (base < nblocks) a.x = absmax[base];
      if (base + 1 < nblocks) a.y = absmax[base + 1];
      if (base + 2 < nblocks) a.z = absmax[base + 2];
    }
    return a;
  };
  // the first group's values are in flight while the mean is formed
  float4 pre = make_float4(0.f, 0.f, 0.f, 0.f);
  if (g0 < ngroups) pre = load4(g0);
  const float mu = mean_of_rows(partials, nrows, (uint32_t)nblocks);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mean_out = mu;
  for (int64_t g = g0; g < ngroups; g += step) {
    const int64_t base = g * kGroup + lane * 4;
    const float4 a = g == g0 ? pre : load4(g);
    float ac[4];
    float m = 0.f;
    ac[0] = __fsub_rn(a.x, mu); ac[1] = __fsub_rn(a.y, mu);
    ac[2] = __fsub_rn(a.z, mu); ac[3] = __fsub_rn(a.w, mu);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (base + i >= nblocks) ac[i] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(ac[i]));
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) m = fmaxf(m, __shfl_xor(m, sh));
    const float s = __fdiv_rn(m, 127.0f);
    if (lane == 0) scale_out[g] = s;
    int qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] = 0;
      if (m != 0.f) {
        float r = rintf(__fdiv_rn(ac[i], s));
        r = fminf(fmaxf(r, -127.f), 127.f);
        qv[i] = (int)r;
      }
    }
    if (base + 3 < nblocks) {
      *reinterpret_cast<uint32_t *>(q_out + base) =
          (uint32_t)(qv[0] & 0xff) | (uint32_t)(qv[1] & 0xff) << 8 | (uint32_t)(qv[2] & 0xff) << 16 |
          (uint32_t)(qv[3] & 0xff) << 24;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (base + i < nblocks) q_out[base + i] = (int8_t)qv[i];
    }
  }
}

// Workgroups of the double-quantization launch: each one re-derives the mean
// from the rows (at most 512 x 128 bytes), so they are kept few.
constexpr int kDqGridMax = 256;

template <bool BF16, bool DQ, bool FP4>
void launch_blocks(int lbs, int grid, int64_t numel, int64_t nfull, hipStream_t stream, const void *w,
                   uint8_t *packed, float *absmax_out, unsigned long long *partials, uint32_t *status) {
  const dim3 g((unsigned)grid), b(kQuantThreads);
  switch (lbs) {
    case 5: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 4, FP4>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, partials, status); break;
    case 6: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 8, FP4>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, partials, status); break;
    case 7: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 16, FP4>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, partials, status); break;
    default: hipLaunchKernelGGL((quantize_blocks_kernel<BF16, DQ, 32, FP4>), g, b, 0, stream, w, numel, nfull, packed, absmax_out, partials, status); break;
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
  const int bpi = kQuantThreads / (bs / 8);   // blocks per quantize workgroup and iteration
  // at least one workgroup: the last one also takes the partial block at the end
  const int64_t g64 = (nfull + bpi - 1) / bpi;
  const int grid = (int)(g64 < 1 ? 1 : (g64 < kQuantGridMax ? g64 : kQuantGridMax));
  using L = void (*)(int, int, int64_t, int64_t, hipStream_t, const void *, uint8_t *, float *,
                     unsigned long long *, uint32_t *);
  static const L blocks[2][2][2] = {{{launch_blocks<false, false, false>, launch_blocks<false, false, true>},
                                     {launch_blocks<false, true, false>, launch_blocks<false, true, true>}},
                                    {{launch_blocks<true, false, false>, launch_blocks<true, false, true>},
                                     {launch_blocks<true, true, false>, launch_blocks<true, true, true>}}};
  blocks[w_is_bf16 ? 1 : 0][dq ? 1 : 0][fp4 ? 1 : 0](lbs, grid, numel, nfull, stream, w, packed, absmax_out,
                                                     partials, status);
  if (dq) {
    const int64_t ngroups = (nblocks + kGroup - 1) / kGroup;
    const int64_t dq_need = (ngroups + kMeanThreads / 64 - 1) / (kMeanThreads / 64);
    const int dq_grid = (int)(dq_need < kDqGridMax ? dq_need : kDqGridMax);
    hipLaunchKernelGGL(mean_dq_kernel, dim3((unsigned)dq_grid), dim3(kMeanThreads), 0, stream, partials, grid,
                       absmax_out, nblocks, q_out, scale_out, mean_out);
  }
  return hipGetLastError();
}

}  // namespace nf4
