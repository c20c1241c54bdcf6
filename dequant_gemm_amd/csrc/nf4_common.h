// nf4_common.h -- device-side constants and helpers shared by the libnf4 kernels.
//
// NF4 levels: "bitsandbytes" page, NF4 data-type paragraph (16 levels from the
// inverse normal CDF, denser near zero).  The values are QLoRA's asymmetric
// construction (8 positive and 7 negative standard-normal quantiles, offset
// 0.9677083, plus 0, normalised by the largest) rounded once to fp32; they are
// stored here as bit patterns.  The decision thresholds are derived from the
// levels: t_i is the smallest fp32 strictly above the midpoint of levels i and
// i+1, so code(n) = #{i : n >= t_i} is the nearest level with ties going to
// the lower index.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace nf4 {

// f(std::integral_constant<int, i>{}) for i = 0 .. n-1, each a separate
// instance: the index is a constant wherever f uses it, however large the body
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_seq(f, std::make_integer_sequence<int, N>{});
}


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBlock = 64;     // weights per absmax block
constexpr int kGroup = 256;    // absmax values per double-quantization scale

constexpr uint32_t kLevelBits[16] = {
    0xbf800000u, 0xbf3239b3u, 0xbf066b30u, 0xbeca32a0u, 0xbe91a24cu, 0xbe3d353fu,
    0xbdba786bu, 0x00000000u, 0x3da2fb03u, 0x3e24cae1u, 0x3e7c04dcu, 0x3ead0338u,
    0x3ee1a4b7u, 0x3f1007aau, 0x3f3913b1u, 0x3f800000u};

constexpr uint32_t kThresholdBits[15] = {
    0xbf591cd9u, 0xbf1c5271u, 0xbeeb847fu, 0xbeadea75u, 0xbe703cebu, 0xbe0d38bau,
    0xbd3a786au, 0x3d22fb04u, 0x3df64863u, 0x3e5067dfu, 0x3e9582d4u, 0x3ec753f8u,
    0x3f006d03u, 0x3f248daeu, 0x3f5c89d9u};

__host__ __device__ constexpr float level(int i) { return __builtin_bit_cast(float, kLevelBits[i]); }
__host__ __device__ constexpr float threshold(int i) { return __builtin_bit_cast(float, kThresholdBits[i]); }

// FP4 ("bitsandbytes" page, 4-bit training paragraph: FP4, standard
// floating-point 4-bit): the E2M1 4-bit float.  A code is the format's own bit
// pattern -- bit 3 the sign, bits 2-1 the exponent with bias 1 (field 0
// subnormal), bit 0 the mantissa -- and its level is the value divided by 6,
// the largest magnitude, rounded once to fp32 (the division by 6 of an exact
// magnitude is one rounding).
__host__ __device__ constexpr float fp4_level(int code) {
  const int e = (code >> 1) & 3, m = code & 1;
  const float mag = e == 0 ? 0.5f * (float)m : (float)(1 << (e - 1)) * (1.0f + 0.5f * (float)m);
  return (code & 8) ? -(mag / 6.0f) : mag / 6.0f;
}
// Decision threshold between FP4 magnitudes i and i+1 (i = 0..6): the largest
// fp32 value not above their exact midpoint, so that for every fp32 |n|,
// |n| > t exactly when |n| lies above the midpoint (a tie goes to the smaller
// magnitude, the lower code).
__host__ __device__ constexpr float fp4_threshold(int i) {
  const double mid = ((double)fp4_level(i) + (double)fp4_level(i + 1)) * 0.5;   // exact in fp64
  const float t = (float)mid;
  return (double)t > mid ? __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, t) - 1u) : t;
}

// ------------------------------------------------------------------ small helpers

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding and leaves the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | (7 << 4) | (0xF << 8) | (((n >> 4) & 3) << 14);
}

// The same for the LDS/scalar-memory counter: at most n outstanding.
__host__ __device__ constexpr int lgkm_imm(int n) {
  return 0xF | (7 << 4) | ((n & 0xF) << 8) | (3 << 14);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  // Byte permute of the 8-byte value {hi, lo}: selector bytes 0-3 pick bytes of
  // `lo`, 4-7 bytes of `hi`, 12 gives 0x00 and 13 or more gives 0xFF.
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t bitsel(uint32_t mask, uint32_t a, uint32_t b) {
  return (mask & a) | (~mask & b);
}

// Two fp32 values rounded to bf16 (nearest-even), packed low then high.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Dequantized block absmax: a^ = fp32(fp32(q * s) + mu) with double
// quantization ("bitsandbytes" page, double-quantization paragraph: the scale
// factors are dequantized first), else the stored fp32 absmax.
struct AbsmaxSrc {
  const float *absmax;        // fp32 per block (no double quantization)
  const int8_t *q;            // int8 per block
  const float *scale;         // fp32 per group of 256 blocks
  const float *mean;          // one fp32
  int dq;
  int lbs;                    // log2 of the block size (5..8: 32..256 weights per block)
  int qt;                     // level table: 0 NF4, 1 FP4 (the launchers pick the kernel instantiation)
};

// Level of code i in the NF4 or FP4 table (a compile-time choice: every kernel
// that builds tables is instantiated for both, so each keeps its constants).
template <bool FP4>
__host__ __device__ constexpr float lvl(int i) { return FP4 ? fp4_level(i) : level(i); }

__device__ __forceinline__ float block_ahat(const AbsmaxSrc &s, int64_t blk, float mu) {
  if (!s.dq) return s.absmax[blk];
  float qs = __fmul_rn((float)s.q[blk], s.scale[blk >> 8]);
  return __fadd_rn(qs, mu);
}

// The raw per-block state, loaded early and turned into a^ only when used, so
// that a prefetch does not force an early wait on its own loads.
struct AbsmaxRaw {
  float v;     // fp32 absmax (no double quantization) or the group scale
  int q;       // int8 absmax (double quantization)
};

__device__ __forceinline__ AbsmaxRaw load_absmax_raw(const AbsmaxSrc &s, int64_t blk) {
  AbsmaxRaw r;
  if (s.dq) {
    r.q = s.q[blk];
    r.v = s.scale[blk >> 8];
  } else {
    r.q = 0;
    r.v = s.absmax[blk];
  }
  return r;
}

// The same with the storage form fixed at compile time, so that no branch sits
// between a lane's loads (a load inside a runtime branch is waited for before
// the branch ends, which would serialise it with the loads issued after it).
template <bool DQ>
__device__ __forceinline__ AbsmaxRaw load_raw(const AbsmaxSrc &s, int64_t blk) {
  AbsmaxRaw r;
  if (DQ) {
    r.q = s.q[blk];
    r.v = s.scale[blk >> 8];
  } else {
    r.q = 0;
    r.v = s.absmax[blk];
  }
  return r;
}

__device__ __forceinline__ float ahat_of(const AbsmaxRaw &r, int dq, float mu) {
  return dq ? __fadd_rn(__fmul_rn((float)r.q, r.v), mu) : r.v;
}

// The state of two adjacent blocks 2i and 2i+1 (one 64-element chunk at block
// size 32), loaded as one access: the two int8 absmax values as 16 bits (the
// pair never straddles a group of 256, so one scale serves both) or the two
// fp32 absmax values as 8 bytes.  Kept packed until used: unpacking right
// after the load would wait for it there.
struct AbsmaxRaw2 {
  float v0, v1;   // fp32 absmax values (no double quantization), or the group scale in v0
  uint32_t q2;    // the two int8 absmax values, block 2i in the low byte
};

template <bool DQ>
__device__ __forceinline__ AbsmaxRaw2 load_raw2(const AbsmaxSrc &s, int64_t blk) {   // blk even
  AbsmaxRaw2 r;
  if (DQ) {
    r.q2 = *reinterpret_cast<const uint16_t *>(s.q + blk);
    r.v0 = s.scale[blk >> 8];
    r.v1 = r.v0;
  } else {
    const float2 a = *reinterpret_cast<const float2 *>(s.absmax + blk);
    r.v0 = a.x;
    r.v1 = a.y;
    r.q2 = 0;
  }
  return r;
}

// a^ of block 2i + u
__device__ __forceinline__ float ahat2_of(const AbsmaxRaw2 &r, int u, int dq, float mu) {
  if (!dq) return u ? r.v1 : r.v0;
  const int q = (int)(int8_t)(uint8_t)(u ? (r.q2 >> 8) : r.q2);
  return __fadd_rn(__fmul_rn((float)q, r.v0), mu);
}

// The per-chunk absmax state of a 64-element chunk: one block, or two at size 32.
template <bool BS32>
struct ChunkAbsmax;
template <>
struct ChunkAbsmax<false> {
  AbsmaxRaw r;
  template <bool DQ>
  __device__ __forceinline__ void load(const AbsmaxSrc &s, int64_t blk) { r = load_raw<DQ>(s, blk); }
  __device__ __forceinline__ float ahat(int, int dq, float mu) const { return ahat_of(r, dq, mu); }
};
template <>
struct ChunkAbsmax<true> {
  AbsmaxRaw2 r;
  template <bool DQ>
  __device__ __forceinline__ void load(const AbsmaxSrc &s, int64_t blk) { r = load_raw2<DQ>(s, blk); }
  __device__ __forceinline__ float ahat(int u, int dq, float mu) const { return ahat2_of(r, u, dq, mu); }
};

// ------------------------------------------------------------------ low-rank adapter term
//
// "bitsandbytes" page, 4-bit/LoRA paragraph: a frozen 4-bit base weight with
// small trainable adapters.  The GEMMs can add a rank-r product U V^T to their
// accumulators before the results are stored: U is bf16 [M, r] (the adapter's
// activations on the reduction side), V is bf16 [output columns, r], both
// row-major, r a multiple of 16.  The adapter rank index plays the role of the
// reduction index in extra MFMA K-slices.
struct LowRank {
  const uint16_t *u;
  const uint16_t *v;
  int r;
};

// For the 32x32x16 kernels with four waves (256 threads), each owning 64
// output columns as two halves of 32 over the workgroup's 256 rows: adds U V^T
// to a wave's 8 x 2 tiles, half h at the columns col[h] (lane l: row l%32 of
// each 32-row tile, column col[h] of half h; lane group kg = l/32 takes ranks
// 16s + 8kg .. +7 of slice s from both operands).  Every wave needs the same
// 256 rows of U, so the workgroup stages them in LDS (`buf`, 256 rows of
// 2 CH + 16 bytes that no wave still reads), a chunk of CH ranks (a multiple
// of 16) at a time; each A fragment read from it feeds both halves.  The V
// fragments of a whole chunk are loaded before its U rows are staged, so that
// their latencies overlap.  Rows past M read row M-1 and the columns must
// already be clamped to existing ones: those outputs are never stored.  All
// waves of the workgroup must call this together (it synchronises them).
template <int CH>
__device__ __forceinline__ void add_lowrank_wide(f32x16 acc[8][2], const LowRank &lr, int64_t m0, int64_t M,
                                                 const int64_t col[2], int bl, int kg, uint8_t *buf) {
  static_assert(CH % 16 == 0, "chunks of whole MFMA slices");
  constexpr int ROW = 2 * CH + 16;   // bytes per staged row (16 of padding against bank conflicts)
  const uint16_t *vrow0 = lr.v + col[0] * lr.r + 8 * kg;
  const uint16_t *vrow1 = lr.v + col[1] * lr.r + 8 * kg;
  for (int r0 = 0; r0 < lr.r; r0 += CH) {
    const int rc = lr.r - r0 < CH ? lr.r - r0 : CH;   // a multiple of 16
    const int cpr = rc / 8;                            // 16-byte chunks per row
    uint4 bv0[CH / 16], bv1[CH / 16];
    static_for<CH / 16>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if (16 * s < rc) {
        bv0[s] = *reinterpret_cast<const uint4 *>(vrow0 + r0 + 16 * s);
        bv1[s] = *reinterpret_cast<const uint4 *>(vrow1 + r0 + 16 * s);
      }
    });
    // U rows into the buffer: piece c = threadIdx.x + 256 k (k < cpr, a
    // condition the whole workgroup shares) is row c / cpr, 16-byte chunk
    // c % cpr.  Every load is issued before the first store, so that the loads'
    // latencies overlap (with a store after each load, each waited for its own).
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 up[CH / 8];
    uint32_t poff[CH / 8];   // the pieces' byte offsets in the buffer
    {
      const int q = 256 / cpr, rm = 256 - q * cpr;      // 256 threads = q rows + rm chunks
      int row = (int)threadIdx.x / cpr, ch = (int)threadIdx.x - row * cpr;
      static_for<CH / 8>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        poff[k] = (uint32_t)(row * ROW + 16 * ch);
        // (a piece past the chunk loads U's first 16 bytes instead, never stored:
        // no branch around the load)
        const int64_t grow = m0 + row < M ? m0 + row : M - 1;
        const int64_t eoff = k < cpr ? grow * lr.r + r0 + 8 * ch : 0;
        up[k] = *reinterpret_cast<const u32x4 *>(lr.u + eoff);
        row += q;
        ch += rm;
        if (ch >= cpr) {
          ch -= cpr;
          ++row;
        }
      });
    }
    __syncthreads();   // the buffer is free
    static_for<CH / 8>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if (k < cpr) *reinterpret_cast<u32x4 *>(buf + poff[k]) = up[k];
    });
    __syncthreads();
    static_for<CH / 16>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      if (16 * s < rc) {
        uint4 av[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          av[i] = *reinterpret_cast<const uint4 *>(buf + (32 * i + bl) * ROW + 16 * (2 * s + kg));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                              __builtin_bit_cast(bf16x8, bv0[s]), acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, av[i]),
                                                              __builtin_bit_cast(bf16x8, bv1[s]), acc[i][1], 0, 0, 0);
        }
      }
    });
  }
}

// ------------------------------------------------------------------ register LUT dequant
//
// For one block, the 16 possible dequantized values bf16(level_i * a^) are
// computed once and held as byte planes: lo[q] holds the low bytes of entries
// 4q..4q+3, hi[q] the high bytes.  A byte-permute then looks up four codes at
// a time; bit 3 of each code picks the upper or lower half of the table.

struct Lut {
  uint32_t lo[4];
  uint32_t hi[4];
};

template <bool FP4>
__device__ __forceinline__ Lut make_lut(float ahat) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    p[j] = pack_bf16x2(__fmul_rn(lvl<FP4>(2 * j), ahat), __fmul_rn(lvl<FP4>(2 * j + 1), ahat));
  Lut t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// Four codes (one per byte of `sel`, values 0..15) -> low and high bytes of
// their bf16 values.
__device__ __forceinline__ void lut_lookup4(uint32_t sel, const Lut &t, uint32_t &lo, uint32_t &hi) {
  const uint32_t s7 = sel & 0x07070707u;
  const uint32_t upper = perm(0u, 0u, sel + 0x05050505u);  // 0xFF in bytes whose code >= 8
  lo = bitsel(upper, perm(t.lo[3], t.lo[2], s7), perm(t.lo[1], t.lo[0], s7));
  hi = bitsel(upper, perm(t.hi[3], t.hi[2], s7), perm(t.hi[1], t.hi[0], s7));
}

// Eight packed codes (element 2j in the low nibble of byte j) -> eight bf16
// values in element order, as four bf16x2 words.
__device__ __forceinline__ void dequant8(uint32_t d, const Lut &t, uint32_t out[4]) {
  const uint32_t even = d & 0x0f0f0f0fu;          // codes of elements 0, 2, 4, 6
  const uint32_t odd = (d >> 4) & 0x0f0f0f0fu;    // codes of elements 1, 3, 5, 7
  const uint32_t sa = perm(odd, even, 0x05010400u);  // codes 0, 1, 2, 3
  const uint32_t sb = perm(odd, even, 0x07030602u);  // codes 4, 5, 6, 7
  uint32_t lo, hi;
  lut_lookup4(sa, t, lo, hi);
  out[0] = perm(hi, lo, 0x05010400u);
  out[1] = perm(hi, lo, 0x07030602u);
  lut_lookup4(sb, t, lo, hi);
  out[2] = perm(hi, lo, 0x05010400u);
  out[3] = perm(hi, lo, 0x07030602u);
}

// The same lookup with the two table halves combined by AND instead of a
// bit-3 mask.  For four codes c the lower-half selector is c (codes 0..7) or
// c + 8 (codes 8..15, selector 16..23, which makes the byte-permute emit 0xFF);
// the upper-half selector is that value with bit 4 flipped: c + 16 (0xFF) for
// codes 0..7 and c - 8 for codes 8..15.  Each half's lookup therefore yields
// the table byte where it owns the code and 0xFF elsewhere, and the AND of the
// two is the entry.
struct Sel4 {
  uint32_t lo;   // selectors into entries 0..7
  uint32_t hi;   // selectors into entries 8..15
};

// Eight packed codes (element 2j in the low nibble of byte j) -> selectors for
// elements 0..3 (a) and 4..7 (b), in element order.
__device__ __forceinline__ void select8(uint32_t d, Sel4 &a, Sel4 &b) {
  const uint32_t even = d & 0x0f0f0f0fu;
  const uint32_t odd = (d >> 4) & 0x0f0f0f0fu;
  const uint32_t ea = even + (d & 0x08080808u);
  const uint32_t oa = odd + (odd & 0x08080808u);
  a.lo = perm(oa, ea, 0x05010400u);
  b.lo = perm(oa, ea, 0x07030602u);
  a.hi = a.lo ^ 0x10101010u;
  b.hi = b.lo ^ 0x10101010u;
}

// The same selectors without putting the elements back in order: (a) for the
// even elements 0, 2, 4, 6 and (b) for the odd elements 1, 3, 5, 7.  Looked up,
// they give a B fragment in the K order 0, 2, 4, 6, 1, 3, 5, 7, which an A
// fragment must match (xfrag_even_odd); two byte permutes fewer per eight codes.
__device__ __forceinline__ void select8_even_odd(uint32_t d, Sel4 &a, Sel4 &b) {
  const uint32_t even = d & 0x0f0f0f0fu;
  const uint32_t odd = (d >> 4) & 0x0f0f0f0fu;
  a.lo = even + (d & 0x08080808u);
  b.lo = odd + (odd & 0x08080808u);
  a.hi = a.lo ^ 0x10101010u;
  b.hi = b.lo ^ 0x10101010u;
}

// Eight consecutive bf16 values (element order) -> K order 0, 2, 4, 6, 1, 3, 5, 7.
__device__ __forceinline__ uint4 xfrag_even_odd(uint4 x) {
  return make_uint4(perm(x.y, x.x, 0x05040100u), perm(x.w, x.z, 0x05040100u), perm(x.y, x.x, 0x07060302u),
                    perm(x.w, x.z, 0x07060302u));
}

// Four selected codes -> their bf16 values as two bf16x2 words (element order).
__device__ __forceinline__ void lookup4(const Sel4 &s, const Lut &t, uint32_t &w0, uint32_t &w1) {
  const uint32_t lo = perm(t.lo[1], t.lo[0], s.lo) & perm(t.lo[3], t.lo[2], s.hi);
  const uint32_t hi = perm(t.hi[1], t.hi[0], s.lo) & perm(t.hi[3], t.hi[2], s.hi);
  w0 = perm(hi, lo, 0x05010400u);
  w1 = perm(hi, lo, 0x07030602u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t w[4]) {
  uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

}  // namespace nf4
