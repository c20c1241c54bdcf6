// gemm_fwd.hip -- fused NF4-dequant GEMM, forward: Y = X W^T.
//
// "Zenbit" page, section "What's inside", bullet zenbit.pallas_nf4: the
// weight streams compressed and is dequantized on chip, never materialised
// at full precision in device memory.  "bitsandbytes" page, quantized-GEMM
// paragraph: on-the-fly dequantization, fp32 multiply and fp32 output.
//
// X is bf16 [M, K]; the weight is NF4 [N, K] (nn.Linear's [out, in]); Y is
// fp32 (or bf16) [M, N].  W^ is formed in registers as bf16 and fed to bf16
// MFMA with fp32 accumulation.
//
// Kernels, chosen by M and the weight's layout:
//   fwd_rows_kernel   M <= 16 over many weight rows: one 16-wave workgroup per
//                     CU walks a run of 16-row groups with X in registers.
//   fwd_small_kernel  M <= 16 otherwise, streaming-bound: one workgroup per 16
//                     weight rows, its eight waves split K; every weight byte is
//                     read once, all of a lane's loads are issued together.
//   fwd_wide_kernel   M > 16, block size 64, no adapter term, K % 256 == 0:
//                     256x256 output tiles, four waves of 64 weight rows (one
//                     wave per SIMD), a lane dequantizing whole 64-blocks.
//   fwd_large_kernel  M > 16 otherwise, matrix-core-bound: 256x256 output
//                     tiles, eight waves; X staged through LDS (three stages,
//                     filled by buffer-to-LDS loads), each wave dequantizes its
//                     own 32 weight rows straight into MFMA operand registers
//                     (no LDS round trip, no duplicate dequantization inside
//                     the workgroup).
#include <utility>

#include "nf4_launch.h"

namespace nf4 {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// ----------------------------------------------------------------- small M
//
// MFMA 16x16x32: lane l feeds A row l%16 (an X row) and B column l%16 (a
// weight row), eight K values each per MFMA.  K is walked in superchunks of
// 256 (four 64-blocks); lane group kg = l/16 owns block kg of each
// superchunk outright -- its 64 codes (two 16-byte loads) and its a^ -- so one
// 16-entry LUT serves 64 elements, and MFMA j of the superchunk takes elements
// 8j..8j+7 of every lane's block.  A and B lanes of the same kg hold the same K
// indices, which is all the MFMA requires.  Eight waves split K; all of a
// wave's loads are issued before any of its arithmetic.

constexpr int kSmallCols = 16;
constexpr int kSmallWaves = 8;
constexpr int kNonTemporal = 2;    // buffer-load cache policy: bit 1 = nt (streaming)
constexpr size_t kSmallXldsBytes = 131456;   // X staged in LDS: at most 16 rows of 4096 (+16 bytes), a zero pad

template <bool Y_BF16, bool DQ, bool LR, bool BS32, bool FP4, bool XLDS>
__global__ __launch_bounds__(64 * kSmallWaves) void fwd_small_kernel(
    const uint16_t *__restrict__ X, int M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ Y) {
  __shared__ f32x4 red[kSmallWaves - 1][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * kSmallCols;
  const int64_t n = n0 + col;
  const bool nvalid = n < N;
  const int64_t nc = nvalid ? n : N - 1;       // columns past N compute garbage, never stored
  const bool mvalid = col < M;
  const float mu = DQ ? *src.mean : 0.f;
  const int kchunks = (int)(K / kBlock);       // 64-element chunks per weight row
  const int nsc = (int)((K + 255) / 256);
  const int per = (nsc + kSmallWaves - 1) / kSmallWaves;
  const int s0 = wave * per;
  const int s1 = s0 + per < nsc ? s0 + per : nsc;

  // All loads go through buffer descriptors based at the workgroup's first
  // weight row, with 32-bit per-lane offsets (K < 2^24 and 16 rows): no 64-bit
  // address arithmetic per lane, and a lane whose offset lies past a
  // descriptor's end reads zeros.  That is how the X loads of rows past M
  // yield the zeros those lanes feed (their products land in output rows
  // that are never stored): at M = 1 this removes 15/16 of the X loads, four
  // times the code bytes, with no masking.  Weight rows past N get zero codes
  // (their outputs are never stored either).
  const int rows = (int)(N - n0 < kSmallCols ? N - n0 : kSmallCols);
  const uint32_t rowb = (uint32_t)(K / 2);
  const __amdgpu_buffer_rsrc_t wrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(packed + n0 * (K / 2)), (short)0,
                                        (int)(rows * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(X), (short)0, (int)(M * K * 2), 0x00020000);
  // Blocks: the block of flat element e is e >> lbs.  The workgroup's first
  // element n0 K is a multiple of 16 * 64, so its block fb = n0 K >> lbs is
  // exact and a lane's block is fb + ((col K + k) >> lbs).
  const int64_t nblocks = (N * K + (1 << src.lbs) - 1) >> src.lbs;
  const int64_t fb = (n0 * K) >> src.lbs;
  const int64_t fg = fb >> 8;                   // the group of block fb
  const int fbo = (int)(fb & 255);              // fb's place in its group
  const int64_t blks = nblocks - fb;            // blocks from fb to the end (descriptor sizes clamp at 2^31 - 1)
  auto nrec = [](int64_t bytes) { return (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff); };
  __amdgpu_buffer_rsrc_t ars, srs;              // fp32 absmax, group scales
  if (DQ) {
    srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src.scale + fg), (short)0,
                                            nrec(4 * (((nblocks + 255) >> 8) - fg)), 0x00020000);
  } else {
    ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src.absmax + fb), (short)0, nrec(4 * blks), 0x00020000);
  }
  // (the int8 absmax is a plain load, clamped to the last block: a sign-extended
  // buffer byte load gets moved behind every other load)
  const int8_t *qwg = DQ ? src.q + fb : nullptr;
  const uint32_t qlast = (uint32_t)(blks - 1 < 0x7fffffff ? blks - 1 : 0x7fffffff);
  auto load_abs = [&](uint32_t rb) {            // rb: block relative to fb
    AbsmaxRaw a;
    if (DQ) {
      a.q = qwg[rb < qlast ? rb : qlast];
      a.v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, ((uint32_t)fbo + rb) >> 8 << 2, 0, 0));
    } else {
      a.q = 0;
      a.v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, rb << 2, 0, 0));
    }
    return a;
  };
  const uint32_t wlane = (uint32_t)col * rowb;             // the lane's row within the descriptor
  const uint32_t elane = (uint32_t)col * (uint32_t)K;      // its first flat element, relative to n0 K
  const uint32_t xlane = mvalid ? (uint32_t)col * (uint32_t)K * 2 : 0x80000000u;

  // XLDS: X [M, K] staged in LDS by buffer-to-LDS loads issued before any
  // weight load (row m at m * (2K + 16) bytes, padded against bank
  // conflicts), one 1 KiB piece per wave instruction; fragments are then read
  // from LDS by the lanes whose X row exists.  Against per-lane X loads from
  // L2 (each instruction touching 64 different 128-byte lines) this took a
  // 4096x4096 call from 5.83 / 7.88 to 5.66 / 7.16 us at M = 4 / 16.  The
  // launcher uses it only when every wave owns at least one superchunk (the
  // hand-over barrier is inside the first iteration) and K % 512 == 0.
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const uint32_t xstride = (uint32_t)(K * 2 + 16);
  const uint32_t xzero = (uint32_t)M * xstride;     // 128 zero bytes after the M rows
  if (XLDS) {
    if (threadIdx.x < 8) *reinterpret_cast<uint4 *>(xs + xzero + 16 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    const int cpr = (int)(K / 8);                   // 16-byte pieces per X row, a multiple of 64
    const int total = M * cpr;
    for (int c0 = 64 * wave; c0 < total; c0 += 64 * kSmallWaves) {
      const int m = c0 / cpr, ch0 = c0 - m * cpr;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void *)(xs + m * xstride + 16 * ch0), 16,
                                               (uint32_t)((m * K + (int64_t)(ch0 + lane) * 8) * 2), 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int sc = s0; sc < s1; sc += 2) {
    uint4 c[2][2];
    AbsmaxRaw r[2], r2[2];   // r2: the second 32-element block of the chunk (block size 32)
    uint4 xa[2][8];
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int bi = 4 * (sc + u) + kg;        // 64-element chunk of the weight row
      ok[u] = (sc + u < s1) && (bi < kchunks);
      const uint32_t bic = ok[u] ? (uint32_t)bi : 0u;
      const uint32_t wo = wlane + bic * (kBlock / 2);
      // codes are read once per call: non-temporal (cache-policy bit nt).  X, which
      // every workgroup reads, and the absmax state keep the default policy (nt on the
      // absmax state measured slower).
      c[u][0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, 0, kNonTemporal));
      c[u][1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo + 16, 0, kNonTemporal));
      const uint32_t rb = (elane + bic * kBlock) >> src.lbs;
      r[u] = load_abs(rb);
      if (BS32) r2[u] = load_abs(rb + 1);
      if (!XLDS) {
        const uint32_t xo = xlane + bic * (kBlock * 2);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xa[u][j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * j, 0, 0));
      }
      // every load before any arithmetic, chunk 0's before chunk 1's (left to itself
      // the compiler sinks the X loads next to their MFMAs to save registers, or
      // puts both chunks' absmax loads last; either serialises the latencies)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    if (XLDS) {
      if (sc == s0) {
        // the X pieces were issued before this iteration's weight loads: two
        // chunks of two code loads and the absmax state (1 or 2 loads per block)
        constexpr int kAfterX = 2 * (2 + (DQ ? 2 : 1) * (BS32 ? 2 : 1));
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAfterX));
        __builtin_amdgcn_s_waitcnt(lgkm_imm(0));      // the zero pad's stores
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // lanes whose X row or chunk does not exist read the zero pad (no
        // branch, no register zeroing)
        const int bi = 4 * (sc + u) + kg;
        const uint32_t xo = (mvalid && ok[u]) ? col * xstride + (uint32_t)bi * (kBlock * 2) : xzero;
#pragma unroll
        for (int j = 0; j < 8; ++j) xa[u][j] = *reinterpret_cast<const uint4 *>(xs + xo + 16 * j);
      }
    }
    // (a chunk past the wave's range has ok = false: a zero table, so its
    // MFMAs add exact zeros; no branch, so no load is sunk into one)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const Lut t = make_lut<FP4>(ok[u] ? ahat_of(r[u], DQ, mu) : 0.f);
      Lut t2;
      if (BS32) t2 = make_lut<FP4>(ok[u] ? ahat_of(r2[u], DQ, mu) : 0.f);
      const uint32_t words[8] = {c[u][0].x, c[u][0].y, c[u][0].z, c[u][0].w,
                                 c[u][1].x, c[u][1].y, c[u][1].z, c[u][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t b[4];
        Sel4 sa, sb;
        const Lut &tj = (BS32 && j >= 4) ? t2 : t;
        select8(words[j], sa, sb);
        lookup4(sa, tj, b[0], b[1]);
        lookup4(sb, tj, b[2], b[3]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u][j]), as_bf16x8(b), acc, 0, 0, 0);
      }
    }
  }
  if (LR) {
    // adapter term: rank slices of 32 dealt to the waves; lane group kg takes
    // ranks 32s + 8kg .. +7 of both operands (zeros past r)
    for (int s = wave; 32 * s < lr.r; s += kSmallWaves) {
      const int rk = 32 * s + 8 * kg;
      uint4 av = make_uint4(0u, 0u, 0u, 0u), bv = make_uint4(0u, 0u, 0u, 0u);
      if (rk < lr.r) {
        bv = *reinterpret_cast<const uint4 *>(lr.v + nc * lr.r + rk);
        if (mvalid) av = *reinterpret_cast<const uint4 *>(lr.u + (int64_t)col * lr.r + rk);
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kSmallWaves - 1; ++w) {
    const f32x4 o = red[w][lane];
    acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
  }
  if (!nvalid) return;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int mm = 4 * kg + rr;
    if (mm < M) {
      if (Y_BF16)
        reinterpret_cast<uint16_t *>(Y)[(int64_t)mm * N + n] = (uint16_t)(pack_bf16x2(acc[rr], 0.f) & 0xffffu);
      else
        reinterpret_cast<float *>(Y)[(int64_t)mm * N + n] = acc[rr];
    }
  }
}

// ----------------------------------------------------------------- small M, many weight rows
//
// For weights of many 16-row groups (at least six per CU) the small-M kernel
// above re-reads X for every group, which at M = 16 and N = 28672, K = 8192
// is 458 MB through L2 per call.  Here a workgroup of 16 waves owns a
// contiguous run of row groups and keeps X in registers for all of them: wave
// w and lane group kg = l/16 form slot s = 4w + kg, which takes the 64-blocks
// s, s + 64, ... of every weight row (XJ = 1 or 2 of them, K <= 8192); lane l
// feeds MFMA 16x16x32 with A = X row l%16 (zeros past M) and B = weight row
// l%16 of the group, MFMA w of a block taking elements 8w .. 8w+7 on both
// sides.  Units (row group, block round) are double buffered: the next unit's
// codes and absmax are in flight while the current one is dequantized.  After
// the last unit of a row group, the adapter term (if any) is added, the 16
// waves' partial sums go through LDS (double buffered, one barrier per row
// group) and wave t % 16 adds them and stores.  Measured on the 28672 x 8192
// weight (three weights rotating, per call): 40.3 / 47.1 / 78.2 us with the
// kernel above against 37.5 / 38.6 / 44.4 us at M = 1 / 4 / 16; with fewer
// row groups per workgroup (4096 x 4096: one, 11008 x 4096: two or three) it
// was slower, so the launcher uses it from six row groups per CU on.
constexpr int kRowsWaves = 16;
constexpr int kRowsGrid = 256;             // one workgroup per CU of the MI355X
constexpr int64_t kRowsMinGroups = 6 * kRowsGrid;

struct DecUnit {
  uint4 c0, c1;      // 64 codes
  int q, q2;         // int8 absmax (q2: second 32-block, block size 32)
  float s, s2;       // group scale (or fp32 absmax without double quantization)
};

template <int XJ, bool DQ, bool BS32, bool FP4>
__global__ __launch_bounds__(64 * kRowsWaves) void fwd_rows_kernel(
    const uint16_t *__restrict__ X, int M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ Y, int y_bf16, int rg_base, int rg_extra) {
  constexpr int kDecWaves = kRowsWaves;
  constexpr int kDecSlots = 4 * kRowsWaves;
  __shared__ f32x4 red[2][kDecWaves][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int slot = 4 * wave + kg;
  const int bid = blockIdx.x;
  const int g0 = bid * rg_base + (bid < rg_extra ? bid : rg_extra);
  const int T = rg_base + (bid < rg_extra ? 1 : 0);
  const int KB = (int)(K >> 6);
  static_assert(XJ == 1 || XJ == 2, "one or two 64-blocks per lane and row");
  constexpr int J = XJ;
  const int U = T * J;
  const float mu = DQ ? *src.mean : 0.f;
  const int64_t n0 = (int64_t)g0 * 16;
  const int64_t rows = (N - n0 < (int64_t)T * 16) ? N - n0 : (int64_t)T * 16;
  const uint32_t rowb = (uint32_t)(K / 2);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(packed + n0 * (K / 2)), (short)0, (int)(rows * rowb), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(X), (short)0, (int)(M * K * 2), 0x00020000);
  const int lbs = src.lbs;
  const int64_t nblocks = (N * K + (1 << lbs) - 1) >> lbs;
  const int64_t fb = (n0 * K) >> lbs;         // first block of the workgroup (n0 K is a multiple of 1024)
  const int64_t fg = fb >> 8;
  const int fbo = (int)(fb & 255);
  const int64_t blks = nblocks - fb;
  auto nrec = [](int64_t bytes) { return (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff); };
  __amdgpu_buffer_rsrc_t ars, srs;
  if (DQ) {
    srs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src.scale + fg), (short)0,
                                            nrec(4 * (((nblocks + 255) >> 8) - fg)), 0x00020000);
  } else {
    ars = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(src.absmax + fb), (short)0, nrec(4 * blks),
                                            0x00020000);
  }
  __amdgpu_buffer_rsrc_t qrs;                 // int8 absmax from the workgroup's first block
  if (DQ)
    qrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t *>(src.q + fb), (short)0, nrec(blks), 0x00020000);
  const uint32_t xrow = col < M ? (uint32_t)col * (uint32_t)K * 2 : 0x80000000u;
  // Y as one range (the launcher keeps M N 4 below 2^31)
  const __amdgpu_buffer_rsrc_t yrs =
      __builtin_amdgcn_make_buffer_rsrc(Y, (short)0, (int)((int64_t)M * N * (y_bf16 ? 2 : 4)), 0x00020000);

  auto load_abs = [&](uint32_t rb, int &q, float &s) {
    if (DQ) {
      q = (int)(int8_t)__builtin_amdgcn_raw_buffer_load_b8(qrs, rb, 0, 0);
      s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(srs, ((uint32_t)fbo + rb) >> 8 << 2, 0, 0));
    } else {
      q = 0;
      s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, rb << 2, 0, 0));
    }
  };
  // unit u = (row group t, block round j); XJ > 0 gives j at compile time
  auto load_unit = [&](int u, DecUnit &d) {
    const int uc = u < U ? u : U - 1;
    const int t = uc / J, j = uc - t * J;
    const int b = slot + kDecSlots * j;
    const bool ok = b < KB;
    const uint32_t bc = ok ? (uint32_t)b : 0u;
    const uint32_t r = (uint32_t)(t * 16 + col);
    const uint32_t wo = ok ? r * rowb + bc * 32 : 0x80000000u;
    d.c0 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo, 0, 2));
    d.c1 = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrs, wo + 16, 0, 2));
    const uint32_t rb = (r * (uint32_t)K + bc * 64) >> lbs;
    load_abs(rb, d.q, d.s);
    if (BS32) load_abs(rb + 1, d.q2, d.s2);
  };
  auto unit_ok = [&](int u) {
    const int t = u / J, j = u - t * J;
    return slot + kDecSlots * j < KB;
  };

  // resident X
  uint4 xr[XJ][8];
  {
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int b = slot + kDecSlots * j;
      const uint32_t xo = b < KB ? xrow + (uint32_t)b * 128 : 0x80000000u;
#pragma unroll
      for (int w = 0; w < 8; ++w)
        xr[j][w] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xo + 16 * w, 0, 0));
    }
    // into the K order of the weight fragments (once; reused for every row group)
#pragma unroll
    for (int j = 0; j < XJ; ++j)
#pragma unroll
      for (int w = 0; w < 8; ++w) xr[j][w] = xfrag_even_odd(xr[j][w]);
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const DecUnit &d, const uint4 *xa, bool ok) {
    const float ah = ok ? (DQ ? __fadd_rn(__fmul_rn((float)d.q, d.s), mu) : d.s) : 0.f;
    const Lut t = make_lut<FP4>(ah);
    Lut t2;
    if (BS32) t2 = make_lut<FP4>(ok ? (DQ ? __fadd_rn(__fmul_rn((float)d.q2, d.s2), mu) : d.s2) : 0.f);
    const uint32_t words[8] = {d.c0.x, d.c0.y, d.c0.z, d.c0.w, d.c1.x, d.c1.y, d.c1.z, d.c1.w};
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t bw[4];
      Sel4 sa, sb;
      const Lut &tw = (BS32 && w >= 4) ? t2 : t;
      select8_even_odd(words[w], sa, sb);
      lookup4(sa, tw, bw[0], bw[1]);
      lookup4(sb, tw, bw[2], bw[3]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[w]), as_bf16x8(bw), acc, 0, 0, 0);
    }
  };
  // end of row group t: adapter term, partial sums through LDS; wave t % 16
  // adds the 16 parts and stores (row group t's outputs: rows m < M of
  // columns n0 + 16t .. +15)
  auto finish = [&](int t) {
    if (lr.r > 0) {
      const int64_t nt = n0 + (int64_t)t * 16;                     // wave-uniform
      const int64_t nlast = N - 1 - nt;                            // lanes past N read row N-1
      const uint16_t *vbase = lr.v + nt * lr.r;
      const uint32_t vrow = (uint32_t)((col < nlast ? col : nlast) * lr.r);
      for (int s = wave; 32 * s < lr.r; s += kDecWaves) {
        const int rk = 32 * s + 8 * kg;
        uint4 av = make_uint4(0u, 0u, 0u, 0u), bv = make_uint4(0u, 0u, 0u, 0u);
        if (rk < lr.r) {
          bv = *reinterpret_cast<const uint4 *>(vbase + vrow + rk);
          if (col < M) av = *reinterpret_cast<const uint4 *>(lr.u + col * lr.r + rk);
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc, 0, 0, 0);
      }
    }
    red[t & 1][wave][lane] = acc;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    if (wave == (t & (kDecWaves - 1))) {
      f32x4 s = red[t & 1][0][lane];
#pragma unroll 5
      for (int w = 1; w < kDecWaves; ++w) {
        const f32x4 o = red[t & 1][w][lane];
        s[0] += o[0]; s[1] += o[1]; s[2] += o[2]; s[3] += o[3];
      }
      // element (m, nt + col) of Y; rows past M and columns past N get an
      // offset beyond the descriptor's range, where stores are dropped
      const uint32_t nt = (uint32_t)(n0 + 16 * t);
      const bool cok = nt + (uint32_t)col < (uint32_t)N;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * kg + r;
        const uint32_t e = (uint32_t)m * (uint32_t)N + nt + (uint32_t)col;
        const bool ok = cok && m < M;
        const float v = s[r];     // a scalar copy: bit_cast of a vector element reads element 0 here
        if (y_bf16)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu), yrs,
                                                ok ? 2 * e : 0x80000000u, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), yrs, ok ? 4 * e : 0x80000000u, 0,
                                                0);
      }
    }
  };

  DecUnit A, B;
  load_unit(0, A);
  load_unit(1, B);
  if (XJ == 2) {
    for (int t = 0; t < T; ++t) {
      compute(A, xr[0], unit_ok(2 * t));
      load_unit(2 * t + 2, A);
      compute(B, xr[XJ - 1], unit_ok(2 * t + 1));
      load_unit(2 * t + 3, B);
      finish(t);
    }
  } else {
    for (int t = 0; t < T; t += 2) {
      compute(A, xr[0], unit_ok(t));
      load_unit(t + 2, A);
      finish(t);
      if (t + 1 < T) {
        compute(B, xr[0], unit_ok(t + 1));
        finish(t + 1);
      }
      load_unit(t + 3, B);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// ----------------------------------------------------------------- large M
//
// Workgroup tile 256 (M) x 256 (N), eight waves, two per SIMD; wave w owns the
// 32 output columns n0 + 32w .. +31 over all 256 rows: 8 MFMA 32x32x16 tiles
// stacked along M, 128 accumulator registers.  Each wave dequantizes only its
// own columns (the weight never passes through LDS, and no column is
// dequantized twice in a workgroup); each dequantized B fragment feeds 8
// MFMAs.  While one wave of a SIMD waits on a load issue or a barrier, the
// other keeps the matrix core busy.
//
// K advances in steps of 64 (one quantization block): per step a lane holds
// one 16-byte code chunk (32 codes) and one LUT.  Lane group kg = l/32 owns K
// range 32kg .. 32kg+31 of the step and MFMA slice j (0..3) takes elements
// 8j .. 8j+7 of it from both operands (A and B only have to agree on the K
// index of each slot).
//
// X tiles (256 rows x 64 K, 32 KiB) reach LDS by buffer-to-LDS loads through
// three stages: the tile two steps ahead loads during a whole step.  The
// barrier that hands a tile over sits in the middle of the last slice, so the
// slice's second half covers the next step's first A-fragment reads.
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NWAVE = 8;
constexpr int XROW = BK * 2;                 // 128-byte LDS rows
constexpr int XTILE = BM * XROW;             // 32 KiB

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// takes a contiguous run of tiles, then walk tiles in groups of 4 M-tiles so
// that the workgroups an XCD runs together share X tiles and weight codes in
// its L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + idx;
  constexpr int G = 4;
  const int per_group = G * tiles_n;
  const int group = t / per_group;
  const int first_m = group * G;
  const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
  const int in_group = t % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// A lane's weight state for one K-step: 32 codes and the block's absmax state.
struct StepCodes {
  uint4 w;
  AbsmaxRaw r;
};

__device__ __forceinline__ void sched_cut() { __builtin_amdgcn_sched_barrier(0); }

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

template <typename T>
__device__ __forceinline__ const uint8_t *uniform_ptr(const T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void mfma2(f32x16 &c0, f32x16 &c1, const uint4 &a0, const uint4 &a1, const uint32_t b[4]) {
  const bf16x8 bv = as_bf16x8(b);
  c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a0), bv, c0, 0, 0, 0);
  c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a1), bv, c1, 0, 0, 0);
}

// Entries 4q .. 4q+3 of the LUT of bf16(level_i * a^) (one quarter, so that
// the work can be spread between MFMAs).
template <bool FP4>
__device__ __forceinline__ void make_lut_quarter(float ahat, int q, Lut &t) {
  const uint32_t p0 = pack_bf16x2(__fmul_rn(lvl<FP4>(4 * q), ahat), __fmul_rn(lvl<FP4>(4 * q + 1), ahat));
  const uint32_t p1 = pack_bf16x2(__fmul_rn(lvl<FP4>(4 * q + 2), ahat), __fmul_rn(lvl<FP4>(4 * q + 3), ahat));
  t.lo[q] = perm(p1, p0, 0x06040200u);
  t.hi[q] = perm(p1, p0, 0x07050301u);
}

// Scheduling-group masks for __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// Interleave a scheduling region as `n` repetitions of: one MFMA, `nds` LDS
// reads, `nv` VALU instructions and, every `vm_every`-th time, one vector
// memory load.  A few vector-ALU instructions after each MFMA overlap the
// matrix core almost completely; a burst after one MFMA does not, even with
// a second wave on the SIMD.
template <int n, int nds, int nv, int vm_every>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int i = 0; i < n; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if (nds) __builtin_amdgcn_sched_group_barrier(SG_DS_READ, nds, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VALU, nv, 0);
    if (vm_every && i % (vm_every ? vm_every : 1) == 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
  }
}

template <bool Y_BF16, bool DQ, bool LR, bool GBS, bool FP4>
__global__ __launch_bounds__(64 * NWAVE) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_large_kernel(
    const uint16_t *__restrict__ X, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ Y, int tiles_m, int tiles_n) {
  // separate arrays (not one indexed by stage) so that the compiler can tell
  // the tile being read from the tiles being loaded
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[XTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[XTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs2[XTILE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const float mu = DQ ? *src.mean : 0.f;
  const int bl = lane & 31, kg = lane >> 5;

  // B operand: this lane's weight row; a column past N loads row N-1 (its
  // outputs are never stored).
  const int64_t ncol = n0 + 32 * wave + bl;
  const int64_t nc = ncol < N ? ncol : N - 1;
  const uint8_t *wq = packed + nc * (K / 2) + kg * 16;
  // block of step k: blk0 + k (block size 64), else the flat index of the lane's
  // 32-element chunk shifted by log2(block size) -- a chunk never straddles a block
  const int64_t blk0 = nc * (K / kBlock);
  const int64_t flat0 = nc * K + 32 * kg;

  // X tile loads, buffer-to-LDS: wave w's load i (0..3) fills LDS bytes
  // (4w + i) * 1024 .. +1023, i.e. tile rows 8(4w + i) .. +7; lane l takes row
  // 8(4w + i) + l/8 and physical 16-byte chunk l%8, which holds logical chunk
  // (l%8) ^ ((row/2) & 7).  One buffer descriptor per wave and step, based at
  // the wave's first row and sized to its rows that exist: lanes of rows past
  // M fall outside it and load zeros.  Offsets and sizes are 32-bit (K < 2^24,
  // checked by the API); the descriptor fields are made explicitly
  // wave-uniform since a descriptor lives in SGPRs.
  const int64_t wrow0 = m0 + 32 * wave;
  const int64_t wrows = M - wrow0 < 0 ? 0 : (M - wrow0 > 32 ? 32 : M - wrow0);
  const int wbytes = __builtin_amdgcn_readfirstlane((int)(uint32_t)(wrows * K * 2));
  const uint8_t *xwave = uniform_ptr(X + (wrows > 0 ? wrow0 : 0) * K);
  uint32_t xvoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 8 * i + (lane >> 3);                             // row within the wave's 32
    xvoff[i] = (uint32_t)(r * K * 2) + ((uint32_t)((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  // A fragments: lane l reads row 32i + l%32, logical chunk 4kg + j of slice j,
  // stored at chunk (4kg + j) ^ ((row/2) & 7) (the row's low five bits are l%32).
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = bl * XROW + (((4 * kg + j) ^ ((bl >> 1) & 7)) << 4);

  const int64_t nk = K / BK;
  auto clampk = [&](int64_t k) { return k < nk ? k : nk - 1; };
  auto xrsrc = [&](int64_t kt) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xwave + clampk(kt) * (BK * 2)), (short)0,
                                             wbytes, 0x00020000);
  };
  auto issue_x1 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t *dst, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (4 * wave + i) * 1024), 16, xvoff[i], 0, 0, 0);
  };
  auto issue_codes = [&](int64_t kt, StepCodes &c) {
    const int64_t k = clampk(kt);
    c.w = *reinterpret_cast<const uint4 *>(wq + k * (BK / 2));
    c.r = load_raw<DQ>(src, GBS ? (flat0 + k * BK) >> src.lbs : blk0 + k);
  };
  auto ahat_at = [&](int64_t kt, const StepCodes &c) { return kt < nk ? ahat_of(c.r, DQ, mu) : 0.f; };

  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  uint4 a[8];      // A fragments; each is refilled for the next slice right after its MFMA issues
  // B fragments rotate through three buffers: step k's slices 0..3 take
  // p0, p1, p2, p0 with (p0, p1, p2) = (k, k+1, k+2) mod 3, and step k+1's
  // first word goes to p1, so every word can be dequantized a slice or more
  // ahead into a buffer no MFMA is reading.
  uint32_t bb0[4], bb1[4], bb2[4];
  uint4 cw;        // codes of the current step
  Lut lut;         // LUT of the current step
  // codes of the next two steps, in flight: step kt + 1 + i sits in slot
  // (kt + 1 + i) % 3, so that with three steps per loop iteration every
  // slot keeps its registers (a loop-carried copy would wait for the load)
  StepCodes cs0, cs1, cs2;

  // prologue: the codes of steps 0 and 1 and tiles 0 and 1; all complete
  // before the barrier (the compiler may reorder these loads, so the wait
  // counts none of them as outstanding)
  {
    StepCodes c0;
    issue_codes(0, c0);
    const __amdgpu_buffer_rsrc_t r0 = xrsrc(0), r1 = xrsrc(1);
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_x1(r0, xs0, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) issue_x1(r1, xs1, i);
    issue_codes(1, cs1);
    cw = c0.w;
    const float ah = ahat_at(0, c0);
#pragma unroll
    for (int q = 0; q < 4; ++q) make_lut_quarter<FP4>(ah, q, lut);
    Sel4 sa, sb;
    select8(cw.x, sa, sb);
    lookup4(sa, lut, bb0[0], bb0[1]);
    lookup4(sb, lut, bb0[2], bb0[3]);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  sched_cut();
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4 *>(xs0 + aoff[0] + i * 32 * XROW);

  // One K-step: four slices of 8 MFMAs (one per 32-row tile), each a
  // scheduling region whose other work is interleaved evenly between its
  // MFMAs (about four vector-ALU instructions each):
  //   slice j < 3   A fragments of slice j+1 (each refilled right after its
  //                 MFMA); one load of the tile two steps ahead into `ld`
  //                 (free since the previous hand-over)
  //   dequant       slice 0: word 1 and word 2's selectors; slice 1: word
  //                 2's lookups and half of word 3; slice 2: the rest of word
  //                 3, the next step's a^ and three quarters of its LUT (in
  //                 place, after word 3's last lookup); slice 3: the last
  //                 quarter and the next step's first word
  //   hand-over     after four MFMAs of slice 3: this wave's LDS reads and
  //                 the next tile's loads complete (only the four loads of the
  //                 tile two steps ahead may be outstanding), the barrier, the
  //                 codes two steps ahead; the slice's last four MFMAs cover
  //                 the reads of the next step's slice-0 fragments from `nx`
  auto step = [&](int64_t kt, uint8_t *rd, uint8_t *nx, uint8_t *ld, const StepCodes &cn, StepCodes &cfill,
                  uint32_t *p0, uint32_t *p1, uint32_t *p2) {
    Sel4 sa, sb, sc, sd;
    const __amdgpu_buffer_rsrc_t rsl = xrsrc(kt + 2);
    // slice 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(p0), acc[i], 0, 0, 0);
      a[i] = *reinterpret_cast<const uint4 *>(rd + aoff[1] + i * 32 * XROW);
    }
    issue_x1(rsl, ld, 0);
    select8(cw.y, sa, sb);
    lookup4(sa, lut, p1[0], p1[1]);
    lookup4(sb, lut, p1[2], p1[3]);
    select8(cw.z, sc, sd);
    interleave<8, 1, 5, 8>();
    sched_cut();
    // slice 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(p1), acc[i], 0, 0, 0);
      a[i] = *reinterpret_cast<const uint4 *>(rd + aoff[2] + i * 32 * XROW);
    }
    issue_x1(rsl, ld, 1);
    lookup4(sc, lut, p2[0], p2[1]);
    lookup4(sd, lut, p2[2], p2[3]);
    select8(cw.w, sa, sb);
    lookup4(sa, lut, p0[0], p0[1]);
    interleave<8, 1, 5, 8>();
    sched_cut();
    // slice 2
    const float ahn = ahat_at(kt + 1, cn);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(p2), acc[i], 0, 0, 0);
      a[i] = *reinterpret_cast<const uint4 *>(rd + aoff[3] + i * 32 * XROW);
    }
    issue_x1(rsl, ld, 2);
    lookup4(sb, lut, p0[2], p0[3]);
    make_lut_quarter<FP4>(ahn, 0, lut);
    make_lut_quarter<FP4>(ahn, 1, lut);
    make_lut_quarter<FP4>(ahn, 2, lut);
    interleave<8, 1, 5, 8>();
    sched_cut();
    // slice 3, first half
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(p0), acc[i], 0, 0, 0);
    issue_x1(rsl, ld, 3);
    make_lut_quarter<FP4>(ahn, 3, lut);
    cw = cn.w;
    select8(cw.x, sa, sb);
    interleave<4, 0, 5, 4>();
    sched_cut();
    // hand-over
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(4) & ~(0xF << 8));   // vmcnt(4) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    sched_cut();
    issue_codes(kt + 2, cfill);
    sched_cut();
    // slice 3, second half
#pragma unroll
    for (int i = 4; i < 8; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(p0), acc[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4 *>(nx + aoff[0] + i * 32 * XROW);
    lookup4(sa, lut, p1[0], p1[1]);
    lookup4(sb, lut, p1[2], p1[3]);
    interleave<4, 2, 4, 0>();
    sched_cut();
  };
  // steps run in threes (one per LDS stage, code slot and B-buffer rotation); the last one or two after the loop
  int64_t kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    step(kt, xs0, xs1, xs2, cs1, cs2, bb0, bb1, bb2);
    step(kt + 1, xs1, xs2, xs0, cs2, cs0, bb1, bb2, bb0);
    step(kt + 2, xs2, xs0, xs1, cs0, cs1, bb2, bb0, bb1);
  }
  if (kt < nk) step(kt, xs0, xs1, xs2, cs1, cs2, bb0, bb1, bb2);
  if (kt + 1 < nk) step(kt + 1, xs1, xs2, xs0, cs2, cs0, bb1, bb2, bb0);
  __builtin_amdgcn_s_waitcnt(0);
  if (LR) add_lowrank_32x8(acc, lr, m0, M, nc, bl, kg, xs0);

  // epilogue: lane l, register r of a 32x32 tile holds row 8(r/4)+4(l/32)+r%4, column l%32
  if (m0 + BM <= M && n0 + BN <= N && N < ((int64_t)1 << 27)) {
    // a full tile: every store is a wave-uniform row address (scalar arithmetic) plus the
    // lane's 32-bit byte offset (row 4kg, column l%32), with no per-store bounds test
    constexpr int ES = Y_BF16 ? 2 : 4;
    const uint32_t voff = (uint32_t)((4 * kg) * (uint32_t)N + bl) * ES;
    uint8_t *ycol = reinterpret_cast<uint8_t *>(Y) + (m0 * N + n0 + 32 * wave) * ES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        uint8_t *rowp = ycol + (int64_t)(32 * i + 8 * (r / 4) + (r % 4)) * N * ES;
        if (Y_BF16)
          *reinterpret_cast<uint16_t *>(rowp + voff) = (uint16_t)(pack_bf16x2(acc[i][r], 0.f) & 0xffffu);
        else
          *reinterpret_cast<float *>(rowp + voff) = acc[i][r];
      }
    }
  } else if (ncol < N) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * i + 8 * (r / 4) + 4 * kg + (r % 4);
        if (row < M) {
          const int64_t off = row * N + ncol;
          if (Y_BF16)
            reinterpret_cast<uint16_t *>(Y)[off] = (uint16_t)(pack_bf16x2(acc[i][r], 0.f) & 0xffffu);
          else
            reinterpret_cast<float *>(Y)[off] = acc[i][r];
        }
      }
    }
  }
}

// ----------------------------------------------------------------- large M, one wave per SIMD
//
// The forward with four waves, each owning 64 output columns (two halves h of
// 32: weight rows n0 + 64w + 32h + l%32) over all 256 rows of the tile: 256
// fp32 accumulators per lane, one wave per SIMD, each A fragment feeding two
// MFMAs.  K advances in double steps of 128 in which lane group kg = l/32
// owns 64-block 2d + kg of both its weight rows, so a lane builds one table per
// 64 weights of a row (the eight-wave kernel above: per 32).  MFMA slice j
// (0..7) takes elements 8j .. 8j+7 of that block from both operands; the A
// fragment of lane group kg comes from the X tile of its block, so a double
// step reads two 64-K tiles at once: four LDS stages, one pair read while the
// other loads.  A double step is 64 groups of two MFMAs (group g of a slice:
// M-tile g against both halves); the other work:
//   A reads     after its MFMAs, group g refills a[g] for the next slice; the
//               next double step's slice 0 after the hand-over
//   B words     the next slice's fragments (word j+1 of both rows) in groups
//               0-5 of slice j < 7; the next double step's two tables once
//               word 7 is done (slice 6 groups 6-7, slice 7 groups 0-1, in
//               place), then its word 0 (slice 7 groups 2-7)
//   X loads     the next double step's two tiles into the other pair of
//               stages: groups 0, 2, ..., 30
//   hand-over   before group 60: all loads and this wave's LDS reads complete,
//               barrier, codes two double steps ahead (into the slot of this
//               double step's own codes)
// Used for block size 64 without an adapter term, K a multiple of 256 (double
// steps in pairs: a loop body with a conditional second double step spills).
constexpr int NWAVE_W = 4;

struct DoubleCodes {
  uint4 w[2][2];    // [row half][16-byte piece]: the 64 codes of each row's block
  AbsmaxRaw r[2];   // the two blocks' absmax state
};

template <bool Y_BF16, bool DQ, bool FP4>
__global__ __launch_bounds__(64 * NWAVE_W) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_wide_kernel(
    const uint16_t *__restrict__ X, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, void *__restrict__ Y, int tiles_m, int tiles_n) {
  // two pairs of stages (tile 2d, then tile 2d + 1), one array per pair so
  // that the compiler can tell the pair being read from the pair being loaded
  // (a pointer chosen per lane between two arrays would make every LDS read
  // wait for all loads in flight)
  __shared__ __attribute__((aligned(1024))) uint8_t xp0[2 * XTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t xp1[2 * XTILE];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const float mu = DQ ? *src.mean : 0.f;
  const int bl = lane & 31, kg = lane >> 5;

  // B operands: this lane's two weight rows; a column past N loads row N-1
  // (its outputs are never stored)
  const uint8_t *wq[2];
  int64_t blk0[2], ncol[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ncol[h] = n0 + 64 * wave + 32 * h + bl;
    const int64_t nc = ncol[h] < N ? ncol[h] : N - 1;
    wq[h] = packed + nc * (K / 2) + kg * 32;   // block kg of each double step
    blk0[h] = nc * (K / kBlock) + kg;
  }

  // X tile loads: a 64-K tile is 256 rows x 128 bytes; wave w's load i (0..7)
  // covers tile rows 8(8w + i) .. +7, swizzled and bounded as in the kernel above
  const int64_t wrow0 = m0 + 64 * wave;
  const int64_t wrows = M - wrow0 < 0 ? 0 : (M - wrow0 > 64 ? 64 : M - wrow0);
  const int wbytes = __builtin_amdgcn_readfirstlane((int)(uint32_t)(wrows * K * 2));
  const uint8_t *xwave = uniform_ptr(X + (wrows > 0 ? wrow0 : 0) * K);
  uint32_t xvoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 8 * i + (lane >> 3);
    xvoff[i] = (uint32_t)(r * K * 2) + ((uint32_t)((lane & 7) ^ ((r >> 1) & 7)) << 4);
  }
  // A fragments: lane l reads row 32i + l%32 of the tile of its block, logical
  // chunk j of slice j, stored at chunk j ^ ((row/2) & 7)
  int aoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) aoff[j] = bl * XROW + ((j ^ ((bl >> 1) & 7)) << 4);

  const int64_t nd = K / (2 * BK);
  auto clampd = [&](int64_t d) { return d < nd ? d : nd - 1; };
  auto xrsrc = [&](int64_t t) {   // the 64-K tile t
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xwave + t * (BK * 2)), (short)0, wbytes,
                                             0x00020000);
  };
  auto issue_x1 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t *dst, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (8 * wave + i) * 1024), 16, xvoff[i], 0, 0, 0);
  };
  auto issue_codes = [&](int64_t d, DoubleCodes &c) {
    const int64_t dc = clampd(d);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 *p = reinterpret_cast<const uint4 *>(wq[h] + dc * BK);
      c.w[h][0] = p[0];
      c.w[h][1] = p[1];
      c.r[h] = load_raw<DQ>(src, blk0[h] + 2 * dc);
    }
  };
  auto ahat_at = [&](int64_t d, const DoubleCodes &c, int h) { return d < nd ? ahat_of(c.r[h], DQ, mu) : 0.f; };
  auto word = [&](const DoubleCodes &c, int h, int j) {
    const uint4 &w = c.w[h][j >> 2];
    return (j & 3) == 0 ? w.x : ((j & 3) == 1 ? w.y : ((j & 3) == 2 ? w.z : w.w));
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][h][r] = 0.f;

  uint4 a[8];
  uint32_t B0[2][4], B1[2][4];   // B fragments [row half] of the current and the next slice
  Lut lut[2];
  DoubleCodes cs0, cs1;          // double step d's codes sit in slot d % 2

  // prologue: codes of double steps 0 and 1, the tiles of double step 0; its
  // tables and slice-0 fragments
  issue_codes(0, cs0);
  {
    const __amdgpu_buffer_rsrc_t r0 = xrsrc(0), r1 = xrsrc(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_x1(r0, xp0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_x1(r1, xp0 + XTILE, i);
  }
  issue_codes(1, cs1);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float ah = ahat_at(0, cs0, h);
#pragma unroll
    for (int q = 0; q < 4; ++q) make_lut_quarter<FP4>(ah, q, lut[h]);
    Sel4 sa, sb;
    select8(word(cs0, h, 0), sa, sb);
    lookup4(sa, lut[h], B0[h][0], B0[h][1]);
    lookup4(sb, lut[h], B0[h][2], B0[h][3]);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  sched_cut();
  {
    const uint8_t *base = xp0 + kg * XTILE;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4 *>(base + aoff[0] + i * 32 * XROW);
  }

  // rdp: the pair read (tiles 2d, 2d+1); ldp: the pair loaded (2d+2, 2d+3)
  auto dstep = [&](int64_t d, uint8_t *rdp, uint8_t *ldp, DoubleCodes &cc, const DoubleCodes &cn) {
    Sel4 sa[2], sb[2];
    float ahn[2] = {0.f, 0.f};
    const uint8_t *rd = rdp + kg * XTILE;
    const uint8_t *nx = ldp + kg * XTILE;
    const int64_t t1 = 2 * clampd(d + 1);
    const __amdgpu_buffer_rsrc_t rl0 = xrsrc(t1), rl1 = xrsrc(t1 + 1);
    static_for<64>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int slice = r / 8, g = r % 8;
      uint32_t(*bc)[4] = (slice & 1) ? B1 : B0;
      uint32_t(*bn)[4] = (slice & 1) ? B0 : B1;
      if (r == 60) {
        __builtin_amdgcn_s_waitcnt(0);   // the next tiles landed, this wave's LDS reads done
        __builtin_amdgcn_s_barrier();
        sched_cut();
        issue_codes(d + 2, cc);
        sched_cut();
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[g][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[g]), as_bf16x8(bc[h]), acc[g][h], 0, 0, 0);
      if (slice < 7) {
        a[g] = *reinterpret_cast<const uint4 *>(rd + aoff[slice + 1] + g * 32 * XROW);
      } else if (r >= 60) {
        // the next double step's slice-0 fragments: a[i] after the hand-over and
        // after its last MFMA here (group 56 + i)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((56 + i > 60 ? 56 + i : 60) == r) a[i] = *reinterpret_cast<const uint4 *>(nx + aoff[0] + i * 32 * XROW);
      }
      if (r % 2 == 0 && r <= 30) {
        const int piece = r / 2;   // 0..7 tile 2d+2, 8..15 tile 2d+3
        if (piece < 8)
          issue_x1(rl0, ldp, piece);
        else
          issue_x1(rl1, ldp + XTILE, piece - 8);
      }
      // B words: word slice+1 of both rows for the next slice
      if (slice < 7 && g < 6) {
        const int h = g / 3, ph = g % 3;
        if (ph == 0) select8(word(cc, h, slice + 1), sa[h], sb[h]);
        if (ph == 1) lookup4(sa[h], lut[h], bn[h][0], bn[h][1]);
        if (ph == 2) lookup4(sb[h], lut[h], bn[h][2], bn[h][3]);
      }
      // the next double step's tables (word 7's lookups are done in group 53)
      if (r >= 54 && r <= 57) {
        const int h = (r - 54) >> 1, q0 = 2 * ((r - 54) & 1);
        if (q0 == 0) ahn[h] = ahat_at(d + 1, cn, h);
        make_lut_quarter<FP4>(ahn[h], q0, lut[h]);
        make_lut_quarter<FP4>(ahn[h], q0 + 1, lut[h]);
      }
      // and its word 0
      if (r >= 58) {
        const int q = r - 58, h = q / 3, ph = q % 3;
        if (ph == 0) select8(word(cn, h, 0), sa[h], sb[h]);
        if (ph == 1) lookup4(sa[h], lut[h], bn[h][0], bn[h][1]);
        if (ph == 2) lookup4(sb[h], lut[h], bn[h][2], bn[h][3]);
      }
      sched_cut();
    });
  };
  for (int64_t d = 0; d < nd; d += 2) {
    dstep(d, xp0, xp1, cs0, cs1);
    dstep(d + 1, xp1, xp0, cs1, cs0);
  }
  __builtin_amdgcn_s_waitcnt(0);

  // epilogue: lane l, register r of a 32x32 tile holds row 8(r/4)+4(l/32)+r%4, column l%32
  if (m0 + BM <= M && n0 + BN <= N && N < ((int64_t)1 << 27)) {
    constexpr int ES = Y_BF16 ? 2 : 4;
    const uint32_t voff = (uint32_t)((4 * kg) * (uint32_t)N + bl) * ES;
    uint8_t *ycol = reinterpret_cast<uint8_t *>(Y) + (m0 * N + n0 + 64 * wave) * ES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uint8_t *rowp = ycol + (int64_t)(32 * i + 8 * (r / 4) + (r % 4)) * N * ES + 32 * h * ES;
          if (Y_BF16)
            *reinterpret_cast<uint16_t *>(rowp + voff) = (uint16_t)(pack_bf16x2(acc[i][h][r], 0.f) & 0xffffu);
          else
            *reinterpret_cast<float *>(rowp + voff) = acc[i][h][r];
        }
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (ncol[h] >= N) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + 32 * i + 8 * (r / 4) + 4 * kg + (r % 4);
          if (row < M) {
            const int64_t off = row * N + ncol[h];
            if (Y_BF16)
              reinterpret_cast<uint16_t *>(Y)[off] = (uint16_t)(pack_bf16x2(acc[i][h][r], 0.f) & 0xffffu);
            else
              reinterpret_cast<float *>(Y)[off] = acc[i][h][r];
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                      const AbsmaxSrc &src, const LowRank &lr, void *y, int y_is_bf16, hipStream_t stream) {
  const uint16_t *X = reinterpret_cast<const uint16_t *>(x);
  const int sel = (y_is_bf16 ? 4 : 0) | (src.dq ? 2 : 0) | (lr.r > 0 ? 1 : 0);
  const int64_t row_groups = (N + 15) / 16;
  // the kernel's 32-bit offsets: a workgroup's codes, and Y as a whole
  const int64_t rows_codes = (row_groups / kRowsGrid + 1) * 16 * (K / 2);
  if (M <= 16 && K <= 8192 && K % 64 == 0 && row_groups >= kRowsMinGroups && rows_codes < (int64_t(1) << 31) &&
      M * N * 4 < (int64_t(1) << 31)) {
    // many weight rows: one 16-wave workgroup per CU over a run of row groups, X in registers
    using R_t = void (*)(const uint16_t *, int, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *, int,
                         int, int);
#define NF4_ROWS(XJ, FP4) {{fwd_rows_kernel<XJ, false, false, FP4>, fwd_rows_kernel<XJ, false, true, FP4>}, \
                           {fwd_rows_kernel<XJ, true, false, FP4>, fwd_rows_kernel<XJ, true, true, FP4>}}
    static const R_t rows[2][2][2][2] = {{NF4_ROWS(1, false), NF4_ROWS(1, true)}, {NF4_ROWS(2, false), NF4_ROWS(2, true)}};
#undef NF4_ROWS
    const int grid = kRowsGrid;
    const int base = (int)(row_groups / grid), extra = (int)(row_groups % grid);
    hipLaunchKernelGGL(rows[K <= 4096 ? 0 : 1][src.qt ? 1 : 0][src.dq ? 1 : 0][src.lbs == 5 ? 1 : 0], dim3(grid),
                       dim3(64 * kRowsWaves), 0, stream, X, (int)M, N, K, packed, src, lr, y, y_is_bf16 ? 1 : 0, base,
                       extra);
  } else if (M <= 16) {
    using K_t = void (*)(const uint16_t *, int, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *);
#define NF4_SMALL(BS32, FP4, XL)                                                                              \
    {fwd_small_kernel<false, false, false, BS32, FP4, XL>, fwd_small_kernel<false, false, true, BS32, FP4, XL>, \
     fwd_small_kernel<false, true, false, BS32, FP4, XL>,  fwd_small_kernel<false, true, true, BS32, FP4, XL>,  \
     fwd_small_kernel<true, false, false, BS32, FP4, XL>,  fwd_small_kernel<true, false, true, BS32, FP4, XL>,  \
     fwd_small_kernel<true, true, false, BS32, FP4, XL>,   fwd_small_kernel<true, true, true, BS32, FP4, XL>}
    static const K_t kern[2][2][8] = {{NF4_SMALL(false, false, false), NF4_SMALL(true, false, false)},
                                      {NF4_SMALL(false, true, false), NF4_SMALL(true, true, false)}};
    static const K_t kern_xlds[2][8] = {NF4_SMALL(false, false, true), NF4_SMALL(false, true, true)};
#undef NF4_SMALL
    const dim3 g((unsigned)((N + kSmallCols - 1) / kSmallCols)), b(64 * kSmallWaves);
    // X staged in LDS (M >= 4, block sizes of 64 or more): it must fit, K must be a
    // multiple of 512, and every wave must own at least one superchunk of 256
    const int64_t nsc = (K + 255) / 256, per = (nsc + kSmallWaves - 1) / kSmallWaves;
    const size_t xbytes = (size_t)M * (size_t)(2 * K + 16) + 128;
    const bool xlds = M >= 4 && src.lbs != 5 && K % 512 == 0 && (kSmallWaves - 1) * per < nsc &&
                      xbytes <= kSmallXldsBytes;
    if (xlds)
      hipLaunchKernelGGL(kern_xlds[src.qt ? 1 : 0][sel], g, b, xbytes, stream, X, (int)M, N, K, packed, src, lr, y);
    else
      hipLaunchKernelGGL(kern[src.qt ? 1 : 0][src.lbs == 5][sel], g, b, 0, stream, X, (int)M, N, K, packed, src, lr,
                         y);
  } else if (src.lbs == 6 && lr.r == 0 && K % (4 * BK) == 0) {
    // block size 64, no adapter term, K a multiple of 256: one wave per SIMD, 64 columns per wave
    using W_t = void (*)(const uint16_t *, int64_t, int64_t, int64_t, const uint8_t *, AbsmaxSrc, void *, int, int);
    static const W_t kern[2][2][2] = {{{fwd_wide_kernel<false, false, false>, fwd_wide_kernel<false, false, true>},
                                       {fwd_wide_kernel<false, true, false>, fwd_wide_kernel<false, true, true>}},
                                      {{fwd_wide_kernel<true, false, false>, fwd_wide_kernel<true, false, true>},
                                       {fwd_wide_kernel<true, true, false>, fwd_wide_kernel<true, true, true>}}};
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern[y_is_bf16 ? 1 : 0][src.dq ? 1 : 0][src.qt ? 1 : 0], dim3((unsigned)(tiles_m * tiles_n)),
                       dim3(64 * NWAVE_W), 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
  } else {
    using K_t = void (*)(const uint16_t *, int64_t, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *,
                         int, int);
#define NF4_LARGE(GBS, FP4)                                                                                   \
    {fwd_large_kernel<false, false, false, GBS, FP4>, fwd_large_kernel<false, false, true, GBS, FP4>,          \
     fwd_large_kernel<false, true, false, GBS, FP4>,  fwd_large_kernel<false, true, true, GBS, FP4>,           \
     fwd_large_kernel<true, false, false, GBS, FP4>,  fwd_large_kernel<true, false, true, GBS, FP4>,           \
     fwd_large_kernel<true, true, false, GBS, FP4>,   fwd_large_kernel<true, true, true, GBS, FP4>}
    static const K_t kern[2][2][8] = {{NF4_LARGE(false, false), NF4_LARGE(true, false)},
                                      {NF4_LARGE(false, true), NF4_LARGE(true, true)}};
#undef NF4_LARGE
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 g((unsigned)(tiles_m * tiles_n)), b(64 * NWAVE);
    hipLaunchKernelGGL(kern[src.qt ? 1 : 0][src.lbs != 6][sel], g, b, 0, stream, X, M, N, K, packed, src, lr, y,
                       tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace nf4
