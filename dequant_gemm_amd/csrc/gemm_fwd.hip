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
//   fwd_small_kernel  M <= 16 otherwise, and larger M while its 16-row grid
//                     rows times N stay small, streaming-bound: one workgroup
//                     per 16 weight rows (per grid row), its eight waves split
//                     K; every weight byte is read once per grid row, all of a
//                     lane's loads are issued together.
//   fwd_wide_kernel   otherwise, matrix-core-bound: 256x256 output tiles, four
//                     waves of 64 weight rows (one wave per SIMD), X staged
//                     through LDS by buffer-to-LDS loads; a lane dequantizes
//                     whole 64-element chunks of its weight rows straight into
//                     MFMA operand registers (no LDS round trip, no duplicate
//                     dequantization inside the workgroup).
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
constexpr int kSmallRows = 16;     // X rows per grid row (the MFMA's 16 A rows)
// Above 16 rows the launcher keeps this kernel (one grid row per 16 rows, each
// dequantizing the whole weight again) while (grid rows) x N is at most
// kSmallChunkBudget.  Its time grows with the grid rows (about N K / 3e12 s
// each, the dequantization's VALU rate), while the 256x256 kernel below 256
// rows takes one round of tiles, about K x 20 ns, on a mostly idle chip;
// measured crossovers: 14 grid rows at N = 4096, 4-5 at 11008, 2 at 28672.
constexpr int64_t kSmallChunkBudget = 14 * 4096;
constexpr int kSmallWaves = 8;
constexpr int kNonTemporal = 2;    // buffer-load cache policy: bit 1 = nt (streaming)
constexpr size_t kSmallXldsBytes = 131456;   // X staged in LDS: at most 16 rows of 4096 (+16 bytes), a zero pad
constexpr int kSmallXldsRows = 11;           // X staged in LDS from this many rows on

template <bool Y_BF16, bool DQ, bool LR, bool BS32, bool FP4, bool XLDS>
__global__ __launch_bounds__(64 * kSmallWaves) void fwd_small_kernel(
    const uint16_t *__restrict__ X, int M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ Y) {
  __shared__ f32x4 red[kSmallWaves - 1][64];
  {
    // more than 16 rows: grid row y takes rows 16y .. 16y + 15 of X (and of U and Y)
    const int m0 = kSmallRows * (int)blockIdx.y;
    X += (int64_t)m0 * K;
    lr.u += (int64_t)m0 * lr.r;
    Y = reinterpret_cast<uint8_t *>(Y) + (int64_t)m0 * N * (Y_BF16 ? 2 : 4);
    M = M - m0 < kSmallRows ? M - m0 : kSmallRows;
  }
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
  // from LDS by the lanes whose X row exists.  The loads have landed only
  // after a wait for every vector-memory operation, the weight loads issued
  // after them included (a count that leaves those in flight does not order
  // buffer-to-LDS loads before them), so the first chunk's arithmetic waits
  // for the second chunk's codes.  Against per-lane X loads from L2 (each
  // instruction touching 64 different 128-byte lines) staging is faster from
  // about 11 rows on: 4096x4096 calls, per-lane / staged, 5.92 / 6.48 us at
  // M = 4, 6.59 / 6.72 at 8, 6.86 / 6.82 at 10, 7.33 / 6.93 at 12.  The launcher
  // uses it from M = 11, when every wave owns at least one superchunk (the
  // hand-over barrier is inside the first iteration) and K % 512 == 0.
  extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
  const uint32_t xstride = (uint32_t)(K * 2 + 16);
  const uint32_t xzero = (uint32_t)M * xstride;     // 128 zero bytes after the M rows
  if (XLDS) {
    if (threadIdx.x < 8) *reinterpret_cast<uint4 *>(xs + xzero + 16 * threadIdx.x) = make_uint4(0u, 0u, 0u, 0u);
    // Piece c0 = 64 w + 512 i (while c0 < M cpr) is row c0 / cpr, 16-byte chunk
    // c0 % cpr; both are kept as wave-uniform counters (scalar registers), so a
    // lane's offset is the constant 16 l and the rest is the scalar offset: no
    // per-lane division or 64-bit multiply ahead of the weight loads.
    const int cpr = (int)(K / 8);                   // 16-byte pieces per X row, a multiple of 64
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    int m = 0, ch0 = 64 * wv;
    while (ch0 >= cpr) {
      ch0 -= cpr;
      ++m;
    }
    while (m < M) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void *)(xs + m * xstride + 16 * ch0), 16,
                                               16u * (uint32_t)lane, (uint32_t)(m * (int)K * 2 + 16 * ch0), 0, 0);
      ch0 += 64 * kSmallWaves;
      while (ch0 >= cpr) {
        ch0 -= cpr;
        ++m;
      }
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
        // the X pieces landed: a wait for all vector-memory operations (a count
        // that leaves the later weight loads in flight does not order the
        // buffer-to-LDS loads before them)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
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
// Workgroup tile 256 (M) x 256 (N), four waves, one per SIMD; wave w owns the
// 64 output columns n0 + 64w .. +63 (two halves h of 32: weight rows
// n0 + 64w + 32h + l%32) over all 256 rows: 8 x 2 MFMA 32x32x16 tiles, 256
// fp32 accumulators per lane.  Each wave dequantizes only its own weight rows
// (the weight never passes through LDS, no row is dequantized twice in a
// workgroup); each dequantized B fragment feeds 8 MFMAs and each A fragment
// read from LDS feeds two.
//
// K advances in double steps of 128 in which lane group kg = l/32 owns the
// 64-element chunk 2d + kg of both its weight rows: one table per 64 weights
// and row (two at block size 32, whose blocks split the chunk).  MFMA slice j
// (0..7) takes elements 8j .. 8j+7 of that chunk from both operands (A and B
// only have to agree on the K index of each slot); the A fragment of lane
// group kg comes from the X tile of its chunk, so a double step reads two
// 64-K tiles at once: four LDS stages, one pair read while the other loads.
// A double step is 64 groups of two MFMAs (group g of a slice: M-tile g
// against both halves); the other work:
//   A reads     after its MFMAs, group g refills a[g] for the next slice; the
//               next double step's slice 0 after the hand-over
//   B words     the next slice's fragments (word j+1 of both rows) in groups
//               0-5 of slice j < 7; at block size 32 the tables of the
//               chunk's second block in groups 6-7 of slice 2 (in place,
//               after word 3); the next double step's tables once word 7 is
//               done (slice 6 groups 6-7, slice 7 groups 0-1), then its word 0
//               (slice 7 groups 2-7)
//   X loads     the next double step's two tiles into the other pair of
//               stages: groups 0, 2, ..., 30
//   hand-over   before group 60: all loads and this wave's LDS reads complete,
//               barrier, codes two double steps ahead (into the slot of this
//               double step's own codes)
// Double steps run in pairs (a loop body with a conditional second double step
// spills); chunks past K -- the second half of a last double step when K / 64
// is odd, a padding double step -- get zero weights.
constexpr int BM = 256, BN = 256, BK = 64;
constexpr int XROW = BK * 2;                 // 128-byte LDS rows
constexpr int XTILE = BM * XROW;             // 32 KiB
constexpr int NWAVE_W = 4;

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

__device__ __forceinline__ void sched_cut() { __builtin_amdgcn_sched_barrier(0); }

template <typename T>
__device__ __forceinline__ const uint8_t *uniform_ptr(const T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
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

// A lane's weight state for one double step: the codes of its chunk of both
// rows and the absmax state of the chunk's block (blocks, at size 32).
template <bool BS32>
struct DoubleCodes {
  uint4 w[2][2];             // [row half][16-byte piece]: the 64 codes of each row's chunk
  ChunkAbsmax<BS32> r[2];
};

template <bool Y_BF16, bool DQ, bool FP4, bool BS32, bool LR>
__global__ __launch_bounds__(64 * NWAVE_W) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_wide_kernel(
    const uint16_t *__restrict__ X, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ Y, int tiles_m, int tiles_n) {
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
  const int64_t nb64 = K / BK;                          // 64-element chunks per row (K % 64 == 0)
  const int64_t nd = (nb64 + 1) / 2;                    // double steps
  const int64_t ndp = (nd + 1) & ~(int64_t)1;           // run in pairs

  // B operands: this lane's two weight rows; a column past N loads row N-1
  // (its outputs are never stored)
  const uint8_t *wrow[2];
  int64_t flat0[2], ncol[2], nclamp[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ncol[h] = n0 + 64 * wave + 32 * h + bl;
    nclamp[h] = ncol[h] < N ? ncol[h] : N - 1;
    wrow[h] = packed + nclamp[h] * (K / 2);
    flat0[h] = nclamp[h] * K;   // flat index of the row's first element: blocks may span rows
  }

  // X tile loads: a 64-K tile is 256 rows x 128 bytes; wave w's load i (0..7)
  // fills LDS bytes (8w + i) * 1024 .. +1023, i.e. tile rows 8(8w + i) .. +7;
  // lane l takes row 8(8w + i) + l/8 and physical 16-byte chunk l%8, which
  // holds logical chunk (l%8) ^ ((row/2) & 7).  One buffer descriptor per wave
  // and tile, based at the wave's first row and sized to its rows that exist:
  // lanes of rows past M fall outside it and load zeros.  Offsets and sizes
  // are 32-bit (K < 2^24); the descriptor fields are made explicitly
  // wave-uniform since a descriptor lives in SGPRs.
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
  // A fragments: lane l reads row 32i + l%32 of the tile of its chunk, logical
  // chunk j of slice j, stored at chunk j ^ ((row/2) & 7)
  int aoff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) aoff[j] = bl * XROW + ((j ^ ((bl >> 1) & 7)) << 4);

  auto xrsrc = [&](int64_t t) {   // the 64-K tile t; past K the last tile again (its weights are zero)
    const int64_t tc = t < nb64 ? t : nb64 - 1;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(xwave + tc * (BK * 2)), (short)0, wbytes,
                                             0x00020000);
  };
  auto issue_x1 = [&](__amdgpu_buffer_rsrc_t rs, uint8_t *dst, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (8 * wave + i) * 1024), 16, xvoff[i], 0, 0, 0);
  };
  auto issue_codes = [&](int64_t d, DoubleCodes<BS32> &c) {
    const int64_t j0 = 2 * d + kg;
    const int64_t j = j0 < nb64 ? j0 : nb64 - 1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint4 *p = reinterpret_cast<const uint4 *>(wrow[h] + j * (BK / 2));
      c.w[h][0] = p[0];
      c.w[h][1] = p[1];
      c.r[h].template load<DQ>(src, (flat0[h] + j * BK) >> src.lbs);
    }
  };
  auto ahat_at = [&](int64_t d, const DoubleCodes<BS32> &c, int h, int u) {
    return 2 * d + kg < nb64 ? c.r[h].ahat(u, DQ, mu) : 0.f;
  };
  auto word = [&](const DoubleCodes<BS32> &c, int h, int j) {
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
  DoubleCodes<BS32> cs0, cs1;      // double step d's codes sit in slot d % 2

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
    const float ah = ahat_at(0, cs0, h, 0);
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
  auto dstep = [&](int64_t d, uint8_t *rdp, uint8_t *ldp, DoubleCodes<BS32> &cc, const DoubleCodes<BS32> &cn) {
    Sel4 sa[2], sb[2];
    float ahn[2] = {0.f, 0.f};
    const uint8_t *rd = rdp + kg * XTILE;
    const uint8_t *nx = ldp + kg * XTILE;
    const __amdgpu_buffer_rsrc_t rl0 = xrsrc(2 * d + 2), rl1 = xrsrc(2 * d + 3);
    static_for<64>([&](auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int slice = r / 8, g = r % 8;
      uint32_t(*bc)[4] = (slice & 1) ? B1 : B0;
      uint32_t(*bn)[4] = (slice & 1) ? B0 : B1;
      if constexpr (r == 60) {
        __builtin_amdgcn_s_waitcnt(0);   // the next tiles landed, this wave's LDS reads done
        __builtin_amdgcn_s_barrier();
        sched_cut();
        issue_codes(d + 2, cc);
        sched_cut();
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acc[g][h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[g]), as_bf16x8(bc[h]), acc[g][h], 0, 0, 0);
      if constexpr (slice < 7) {
        a[g] = *reinterpret_cast<const uint4 *>(rd + aoff[slice + 1] + g * 32 * XROW);
      } else if constexpr (r >= 60) {
        // the next double step's slice-0 fragments: a[i] after the hand-over and
        // after its last MFMA here (group 56 + i)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if ((56 + i > 60 ? 56 + i : 60) == r) a[i] = *reinterpret_cast<const uint4 *>(nx + aoff[0] + i * 32 * XROW);
      }
      if constexpr (r % 2 == 0 && r <= 30) {
        constexpr int piece = r / 2;   // 0..7 tile 2d+2, 8..15 tile 2d+3
        if constexpr (piece < 8)
          issue_x1(rl0, ldp, piece);
        else
          issue_x1(rl1, ldp + XTILE, piece - 8);
      }
      // B words: word slice+1 of both rows for the next slice
      if constexpr (slice < 7 && g < 6) {
        constexpr int h = g / 3, ph = g % 3;
        if constexpr (ph == 0) select8(word(cc, h, slice + 1), sa[h], sb[h]);
        if constexpr (ph == 1) lookup4(sa[h], lut[h], bn[h][0], bn[h][1]);
        if constexpr (ph == 2) lookup4(sb[h], lut[h], bn[h][2], bn[h][3]);
      }
      // block size 32: words 4-7 belong to the chunk's second block
      if constexpr (BS32 && slice == 2 && g >= 6) {
        constexpr int h = g - 6;
        const float ab = ahat_at(d, cc, h, 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) make_lut_quarter<FP4>(ab, q, lut[h]);
      }
      // the next double step's tables (word 7's lookups are done in group 53)
      if constexpr (r >= 54 && r <= 57) {
        constexpr int h = (r - 54) >> 1, q0 = 2 * ((r - 54) & 1);
        if constexpr (q0 == 0) ahn[h] = ahat_at(d + 1, cn, h, 0);
        make_lut_quarter<FP4>(ahn[h], q0, lut[h]);
        make_lut_quarter<FP4>(ahn[h], q0 + 1, lut[h]);
      }
      // and its word 0
      if constexpr (r >= 58) {
        constexpr int q = r - 58, h = q / 3, ph = q % 3;
        if constexpr (ph == 0) select8(word(cn, h, 0), sa[h], sb[h]);
        if constexpr (ph == 1) lookup4(sa[h], lut[h], bn[h][0], bn[h][1]);
        if constexpr (ph == 2) lookup4(sb[h], lut[h], bn[h][2], bn[h][3]);
      }
      sched_cut();
    });
  };
  for (int64_t d = 0; d < ndp; d += 2) {
    dstep(d, xp0, xp1, cs0, cs1);
    dstep(d + 1, xp1, xp0, cs1, cs0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  // the adapter term: ranks in chunks of 112 (256 staged rows of 240 bytes in the first pair of stages)
  if (LR) add_lowrank_wide<112>(acc, lr, m0, M, nclamp, bl, kg, xp0);

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
  } else if (M <= 16 || ((M + kSmallRows - 1) / kSmallRows) * N <= kSmallChunkBudget) {
    // a few rows: the streaming kernel, one grid row per 16 rows of X
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
    const dim3 g((unsigned)((N + kSmallCols - 1) / kSmallCols), (unsigned)((M + kSmallRows - 1) / kSmallRows)),
        b(64 * kSmallWaves);
    // X staged in LDS (M >= 11, block sizes of 64 or more): it must fit, K must be a
    // multiple of 512, and every wave must own at least one superchunk of 256
    const int64_t nsc = (K + 255) / 256, per = (nsc + kSmallWaves - 1) / kSmallWaves;
    const int64_t mrows = M < kSmallRows ? M : kSmallRows;   // X rows a workgroup stages
    const size_t xbytes = (size_t)mrows * (size_t)(2 * K + 16) + 128;
    const bool xlds = M >= kSmallXldsRows && src.lbs != 5 && K % 512 == 0 && (kSmallWaves - 1) * per < nsc &&
                      xbytes <= kSmallXldsBytes;
    if (xlds)
      hipLaunchKernelGGL(kern_xlds[src.qt ? 1 : 0][sel], g, b, xbytes, stream, X, (int)M, N, K, packed, src, lr, y);
    else
      hipLaunchKernelGGL(kern[src.qt ? 1 : 0][src.lbs == 5][sel], g, b, 0, stream, X, (int)M, N, K, packed, src, lr,
                         y);
  } else {
    // M > 16: 256x256 tiles, one wave per SIMD
    using W_t = void (*)(const uint16_t *, int64_t, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *, int,
                         int);
#define NF4_WIDE(YB, DQ, FP4) {{fwd_wide_kernel<YB, DQ, FP4, false, false>, fwd_wide_kernel<YB, DQ, FP4, false, true>}, \
                               {fwd_wide_kernel<YB, DQ, FP4, true, false>, fwd_wide_kernel<YB, DQ, FP4, true, true>}}
    static const W_t kern[2][2][2][2][2] = {{{NF4_WIDE(false, false, false), NF4_WIDE(false, false, true)},
                                             {NF4_WIDE(false, true, false), NF4_WIDE(false, true, true)}},
                                            {{NF4_WIDE(true, false, false), NF4_WIDE(true, false, true)},
                                             {NF4_WIDE(true, true, false), NF4_WIDE(true, true, true)}}};
#undef NF4_WIDE
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    hipLaunchKernelGGL(kern[y_is_bf16 ? 1 : 0][src.dq ? 1 : 0][src.qt ? 1 : 0][src.lbs == 5 ? 1 : 0][lr.r > 0 ? 1 : 0],
                       dim3((unsigned)(tiles_m * tiles_n)), dim3(64 * NWAVE_W), 0, stream, X, M, N, K, packed, src, lr,
                       y, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace nf4
