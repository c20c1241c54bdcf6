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
// Two kernels, chosen by M:
//   fwd_small_kernel  M <= 16, streaming-bound: one workgroup per 16 weight
//                     rows, its eight waves split K; every weight byte is read
//                     once, all of a lane's loads are issued together.
//   fwd_large_kernel  M > 16, matrix-core-bound: 256x256 output tiles; X
//                     staged through LDS (double-buffered), each wave
//                     dequantizes its own 64 weight rows straight into MFMA
//                     operand registers (no LDS round trip, no duplicate
//                     dequantization inside the workgroup).
#include "nf4_launch.h"

namespace nf4 {
namespace {

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

template <bool Y_BF16>
__global__ __launch_bounds__(64 * kSmallWaves) void fwd_small_kernel(
    const uint16_t *__restrict__ X, int M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, void *__restrict__ Y) {
  __shared__ f32x4 red[kSmallWaves - 1][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * kSmallCols + col;
  const bool nvalid = n < N;
  const int64_t nc = nvalid ? n : N - 1;       // columns past N compute garbage, never stored
  const int m = col < M ? col : M - 1;         // rows past M likewise
  const float mu = src.dq ? *src.mean : 0.f;
  const int64_t kblocks = K / kBlock;
  const int64_t nsc = (K + 255) / 256;
  const int64_t per = (nsc + kSmallWaves - 1) / kSmallWaves;
  const int64_t s0 = wave * per;
  const int64_t s1 = s0 + per < nsc ? s0 + per : nsc;
  const uint8_t *wrow = packed + nc * (K / 2);
  const uint16_t *xrow = X + (int64_t)m * K;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t sc = s0; sc < s1; sc += 2) {
    uint4 c[2][2];
    AbsmaxRaw r[2];
    uint4 xa[2][8];
    bool ok[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t bi = 4 * (sc + u) + kg;
      ok[u] = (sc + u < s1) && (bi < kblocks);
      const int64_t bic = ok[u] ? bi : 0;
      const uint4 *p = reinterpret_cast<const uint4 *>(wrow + bic * (kBlock / 2));
      c[u][0] = p[0];
      c[u][1] = p[1];
      r[u] = load_absmax_raw(src, nc * kblocks + bic);
      const uint4 *xp = reinterpret_cast<const uint4 *>(xrow + bic * kBlock);
#pragma unroll
      for (int j = 0; j < 8; ++j) xa[u][j] = xp[j];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (sc + u >= s1) break;
      const Lut t = make_lut(ok[u] ? ahat_of(r[u], src.dq, mu) : 0.f);
      const uint32_t words[8] = {c[u][0].x, c[u][0].y, c[u][0].z, c[u][0].w,
                                 c[u][1].x, c[u][1].y, c[u][1].z, c[u][1].w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t b[4];
        dequant8(words[j], t, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[u][j]), as_bf16x8(b), acc, 0, 0, 0);
      }
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

// ----------------------------------------------------------------- large M

// Instruction-scheduling strategy for the K loop (1: the compiler's
// single-wave MFMA interleave, the fastest measured on gfx950).
#ifndef NF4_FWD_SCHED
#define NF4_FWD_SCHED 1
#endif

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int LDS_ROW = BK * 2 + 16;  // bytes; 16 bytes of padding keep ds_read_b128 conflict-free

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// takes a contiguous run of tiles, then walk tiles in groups of 8 M-tiles so
// that workgroups running together share X row panels and weight columns in
// their XCD's L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int total = tiles_m * tiles_n;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + idx;
  constexpr int G = 8;
  const int per_group = G * tiles_n;
  const int group = t / per_group;
  const int first_m = group * G;
  const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
  const int in_group = t % per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <bool Y_BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_large_kernel(const uint16_t *__restrict__ X, int64_t M,
                                                        int64_t N, int64_t K,
                                                        const uint8_t *__restrict__ packed,
                                                        AbsmaxSrc src, void *__restrict__ Y,
                                                        int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2][BM * LDS_ROW];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const float mu = src.dq ? *src.mean : 0.f;

  // B operand: this lane's two weight rows (one per 32-column subtile).
  // Columns past N and rows past M load in-bounds stand-ins; their outputs
  // are never stored, so every load is unconditional.
  const int bl = lane & 31, kg = lane >> 5;
  int64_t ncol[2];
  const uint8_t *wp[2];
  int64_t blk0[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ncol[t] = n0 + 64 * wave + 32 * t + bl;
    const int64_t nn = ncol[t] < N ? ncol[t] : N - 1;
    wp[t] = packed + nn * (K / 2) + kg * 16;
    blk0[t] = nn * (K / kBlock);
  }

  // X staging: eight threads per 128-byte row segment, 32 rows per pass
  const int xr = tid >> 3, xc = tid & 7;
  const uint16_t *xp[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + xr + 32 * i;
    xp[i] = X + (row < M ? row : M - 1) * K + xc * 8;
  }

  const int64_t nk = K / BK;
  const uint4 *xq[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) xq[i] = reinterpret_cast<const uint4 *>(xp[i]);
  const uint4 *wq0 = reinterpret_cast<const uint4 *>(wp[0]);
  const uint4 *wq1 = reinterpret_cast<const uint4 *>(wp[1]);
  uint8_t *xs = &smem[0][(xr * LDS_ROW) + xc * 16];

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  // prologue: tile 0 to LDS, its codes in registers
  uint4 x0 = xq[0][0], x1 = xq[1][0], x2 = xq[2][0], x3 = xq[3][0];
  uint4 x4 = xq[4][0], x5 = xq[5][0], x6 = xq[6][0], x7 = xq[7][0];
  uint4 cn0 = wq0[0], cn1 = wq1[0];
  AbsmaxRaw rn0 = load_absmax_raw(src, blk0[0]), rn1 = load_absmax_raw(src, blk0[1]);
  {
    uint8_t *d = xs;
    *reinterpret_cast<uint4 *>(d + 0 * 32 * LDS_ROW) = x0;
    *reinterpret_cast<uint4 *>(d + 1 * 32 * LDS_ROW) = x1;
    *reinterpret_cast<uint4 *>(d + 2 * 32 * LDS_ROW) = x2;
    *reinterpret_cast<uint4 *>(d + 3 * 32 * LDS_ROW) = x3;
    *reinterpret_cast<uint4 *>(d + 4 * 32 * LDS_ROW) = x4;
    *reinterpret_cast<uint4 *>(d + 5 * 32 * LDS_ROW) = x5;
    *reinterpret_cast<uint4 *>(d + 6 * 32 * LDS_ROW) = x6;
    *reinterpret_cast<uint4 *>(d + 7 * 32 * LDS_ROW) = x7;
  }
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const uint4 cc0 = cn0, cc1 = cn1;
    const AbsmaxRaw r0 = rn0, r1 = rn1;
    // next tile's loads (the last iteration re-reads tile nk-1, harmlessly)
    const int64_t kn = kt + 1 < nk ? kt + 1 : kt;
    const int64_t xo = kn * (BK / 8);
    x0 = xq[0][xo]; x1 = xq[1][xo]; x2 = xq[2][xo]; x3 = xq[3][xo];
    x4 = xq[4][xo]; x5 = xq[5][xo]; x6 = xq[6][xo]; x7 = xq[7][xo];
    cn0 = wq0[kn * 2];
    cn1 = wq1[kn * 2];
    rn0 = load_absmax_raw(src, blk0[0] + kn);
    rn1 = load_absmax_raw(src, blk0[1] + kn);

    const Lut t0 = make_lut(ahat_of(r0, src.dq, mu)), t1 = make_lut(ahat_of(r1, src.dq, mu));
    const uint32_t w0[4] = {cc0.x, cc0.y, cc0.z, cc0.w};
    const uint32_t w1[4] = {cc1.x, cc1.y, cc1.z, cc1.w};
    const uint8_t *abase = &smem[cur][bl * LDS_ROW + kg * 64];
    // Software pipeline over the four 16-wide K slices: the A fragments and
    // the dequantized B fragments of slice j+1 are produced while the 16
    // MFMAs of slice j run.
    uint4 a[8];
    uint32_t b0[4], b1[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4 *>(abase + 32 * i * LDS_ROW);
    dequant8(w0[0], t0, b0);
    dequant8(w1[0], t1, b1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 an[8];
      uint32_t bn0[4], bn1[4];
      if (j < 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          an[i] = *reinterpret_cast<const uint4 *>(abase + 32 * i * LDS_ROW + 16 * (j + 1));
        dequant8(w0[j + 1], t0, bn0);
        dequant8(w1[j + 1], t1, bn1);
      }
      const bf16x8 bv0 = as_bf16x8(b0), bv1 = as_bf16x8(b1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bf16x8 av = as_bf16x8(a[i]);
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv1, acc[i][1], 0, 0, 0);
      }
#if NF4_FWD_SCHED == 3
      if (j < 3) {
#pragma unroll
        for (int g = 0; g < 16; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          if (g < 8) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
#endif
      if (j < 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = an[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          b0[e] = bn0[e];
          b1[e] = bn1[e];
        }
      }
    }
#if NF4_FWD_SCHED == 1
    __builtin_amdgcn_iglp_opt(1);
#elif NF4_FWD_SCHED == 2
    __builtin_amdgcn_iglp_opt(0);
#endif
    {
      uint8_t *d = xs + (cur ^ 1) * (BM * LDS_ROW);
      *reinterpret_cast<uint4 *>(d + 0 * 32 * LDS_ROW) = x0;
      *reinterpret_cast<uint4 *>(d + 1 * 32 * LDS_ROW) = x1;
      *reinterpret_cast<uint4 *>(d + 2 * 32 * LDS_ROW) = x2;
      *reinterpret_cast<uint4 *>(d + 3 * 32 * LDS_ROW) = x3;
      *reinterpret_cast<uint4 *>(d + 4 * 32 * LDS_ROW) = x4;
      *reinterpret_cast<uint4 *>(d + 5 * 32 * LDS_ROW) = x5;
      *reinterpret_cast<uint4 *>(d + 6 * 32 * LDS_ROW) = x6;
      *reinterpret_cast<uint4 *>(d + 7 * 32 * LDS_ROW) = x7;
    }
    __syncthreads();
  }

  // epilogue: lane l, register r of a 32x32 tile holds row 8(r/4)+4(l/32)+r%4, column l%32
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (ncol[t] >= N) continue;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 32 * i + 8 * (r / 4) + 4 * kg + (r % 4);
        if (row < M) {
          const int64_t off = row * N + ncol[t];
          if (Y_BF16)
            reinterpret_cast<uint16_t *>(Y)[off] = (uint16_t)(pack_bf16x2(acc[i][t][r], 0.f) & 0xffffu);
          else
            reinterpret_cast<float *>(Y)[off] = acc[i][t][r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd(const void *x, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                      const AbsmaxSrc &src, void *y, int y_is_bf16, hipStream_t stream) {
  const uint16_t *X = reinterpret_cast<const uint16_t *>(x);
  if (M <= 16) {
    const dim3 g((unsigned)((N + kSmallCols - 1) / kSmallCols)), b(64 * kSmallWaves);
    if (y_is_bf16)
      hipLaunchKernelGGL((fwd_small_kernel<true>), g, b, 0, stream, X, (int)M, N, K, packed, src, y);
    else
      hipLaunchKernelGGL((fwd_small_kernel<false>), g, b, 0, stream, X, (int)M, N, K, packed, src, y);
  } else {
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const dim3 g((unsigned)(tiles_m * tiles_n)), b(256);
    if (y_is_bf16)
      hipLaunchKernelGGL((fwd_large_kernel<true>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((fwd_large_kernel<false>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
  }
  return hipGetLastError();
}

}  // namespace nf4
