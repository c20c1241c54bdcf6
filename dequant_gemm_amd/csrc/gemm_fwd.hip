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
//                     rows, its four waves split K; every weight byte is read
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
// weight row), each with eight K values; lane group kg = l/16 takes 32
// consecutive K of a 128-wide chunk (one 16-byte load of codes), of which
// MFMA j uses elements 8j..8j+7.  A and B lanes of the same kg hold the same
// K indices, which is all the MFMA requires.

constexpr int kSmallCols = 16;
constexpr int kSmallUnroll = 8;

template <bool Y_BF16>
__global__ __launch_bounds__(256) void fwd_small_kernel(const uint16_t *__restrict__ X, int M,
                                                        int64_t N, int64_t K,
                                                        const uint8_t *__restrict__ packed,
                                                        AbsmaxSrc src, void *__restrict__ Y) {
  __shared__ f32x4 red[3][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  const int64_t n = (int64_t)blockIdx.x * kSmallCols + col;
  const bool nvalid = n < N;
  const bool mvalid = col < M;
  const float mu = src.dq ? *src.mean : 0.f;
  const int64_t nchunk = (K + 127) / 128;
  const int64_t per = (nchunk + 3) / 4;
  const int64_t c0 = wave * per;
  const int64_t c1 = c0 + per < nchunk ? c0 + per : nchunk;
  const uint8_t *wrow = packed + (nvalid ? n : 0) * (K / 2);
  const uint16_t *xrow = X + (mvalid ? col : 0) * K;
  const int64_t blk_row = (nvalid ? n : 0) * (K / kBlock);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int64_t c = c0; c < c1; c += kSmallUnroll) {
    uint4 cw[kSmallUnroll];
    float ah[kSmallUnroll];
#pragma unroll
    for (int u = 0; u < kSmallUnroll; ++u) {
      const int64_t k = (c + u) * 128 + kg * 32;
      const bool ok = nvalid && (c + u < c1) && (k < K);
      cw[u] = ok ? *reinterpret_cast<const uint4 *>(wrow + k / 2) : make_uint4(0, 0, 0, 0);
      ah[u] = ok ? block_ahat(src, blk_row + k / kBlock, mu) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kSmallUnroll; ++u) {
      if (c + u >= c1) break;
      const int64_t k = (c + u) * 128 + kg * 32;
      const bool kok = k < K;
      const Lut t = make_lut(ah[u]);
      const uint32_t words[4] = {cw[u].x, cw[u].y, cw[u].z, cw[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 xa = make_uint4(0, 0, 0, 0);
        if (mvalid && kok) xa = *reinterpret_cast<const uint4 *>(xrow + k + 8 * j);
        uint32_t b[4];
        dequant8(words[j], t, b);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa), as_bf16x8(b), acc, 0, 0, 0);
      }
    }
  }
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    const f32x4 o = red[w][lane];
    acc[0] += o[0]; acc[1] += o[1]; acc[2] += o[2]; acc[3] += o[3];
  }
  if (!nvalid) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int m = 4 * kg + r;
    if (m < M) {
      if (Y_BF16)
        reinterpret_cast<uint16_t *>(Y)[(int64_t)m * N + n] = (uint16_t)(pack_bf16x2(acc[r], 0.f) & 0xffffu);
      else
        reinterpret_cast<float *>(Y)[(int64_t)m * N + n] = acc[r];
    }
  }
}

// ----------------------------------------------------------------- large M

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
__global__ __launch_bounds__(256) void fwd_large_kernel(const uint16_t *__restrict__ X, int64_t M,
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

  // B operand: this lane's two weight rows (one per 32-column subtile)
  const int bl = lane & 31, kg = lane >> 5;
  int64_t ncol[2];
  bool nval[2];
  const uint8_t *wp[2];
  int64_t blk0[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ncol[t] = n0 + 64 * wave + 32 * t + bl;
    nval[t] = ncol[t] < N;
    const int64_t nn = nval[t] ? ncol[t] : 0;
    wp[t] = packed + nn * (K / 2) + kg * 16;
    blk0[t] = nn * (K / kBlock);
  }

  // X staging: eight threads per 128-byte row segment, 32 rows per pass
  const int xr = tid >> 3, xc = tid & 7;
  const uint16_t *xp[8];
  bool xval[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + xr + 32 * i;
    xval[i] = row < M;
    xp[i] = X + (xval[i] ? row : 0) * K + xc * 8;
  }

  const int64_t nk = K / BK;
  uint4 xreg[8];
  uint4 creg[2];
  float areg[2];
  auto load_x = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xreg[i] = xval[i] ? *reinterpret_cast<const uint4 *>(xp[i] + kt * BK) : make_uint4(0, 0, 0, 0);
  };
  auto load_b = [&](int64_t kt) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      creg[t] = nval[t] ? *reinterpret_cast<const uint4 *>(wp[t] + kt * (BK / 2)) : make_uint4(0, 0, 0, 0);
      areg[t] = nval[t] ? block_ahat(src, blk0[t] + kt, mu) : 0.f;
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4 *>(&smem[buf][(xr + 32 * i) * LDS_ROW + xc * 16]) = xreg[i];
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  load_x(0);
  load_b(0);
  store_x(0);
  __syncthreads();

  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    const uint4 cc0 = creg[0], cc1 = creg[1];
    const float a0 = areg[0], a1 = areg[1];
    const bool more = kt + 1 < nk;
    if (more) {
      load_x(kt + 1);
      load_b(kt + 1);
    }
    const Lut t0 = make_lut(a0), t1 = make_lut(a1);
    const uint32_t w0[4] = {cc0.x, cc0.y, cc0.z, cc0.w};
    const uint32_t w1[4] = {cc1.x, cc1.y, cc1.z, cc1.w};
    const uint8_t *abase = &smem[cur][bl * LDS_ROW + kg * 64];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t b0[4], b1[4];
      dequant8(w0[j], t0, b0);
      dequant8(w1[j], t1, b1);
      const bf16x8 bv0 = as_bf16x8(b0), bv1 = as_bf16x8(b1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 a = *reinterpret_cast<const uint4 *>(abase + 32 * i * LDS_ROW + 16 * j);
        const bf16x8 av = as_bf16x8(a);
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv1, acc[i][1], 0, 0, 0);
      }
    }
    if (more) store_x(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane l, register r of a 32x32 tile holds row 8(r/4)+4(l/32)+r%4, column l%32
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (!nval[t]) continue;
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
    const dim3 g((unsigned)((N + kSmallCols - 1) / kSmallCols)), b(256);
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
