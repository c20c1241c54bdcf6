// gemm_bwd.hip -- fused NF4-dequant GEMM, backward with respect to the input:
// dX = dY W^ (no gradient for the frozen weight).
//
// "Zenbit" page, section "What's inside", bullet zenbit.pallas_nf4: a fused
// backward pass forms dL/dX without materialising the dequantized weight, and
// dL/dW is not computed for a frozen quantized base weight.
//
// dY is bf16 [M, N]; the weight is NF4 [N, K]; dX is fp32 (or bf16) [M, K].
// Here the reduction runs over N while the weight's 64-blocks run along K, so
// the dequantized tile has to change orientation before it can feed the MFMA
// (whose operands hold eight consecutive reduction indices per lane): each
// thread dequantizes two weight rows over 32 K, pairs the two rows' values
// per K into one 32-bit word and writes it to an LDS tile stored K-major
// ([k][n]); the MFMA then reads B fragments from that tile with 16-byte loads.
//
// Tiles: 256 (M) x 256 (K) outputs per workgroup, reduction steps of 64 N,
// four waves in a 2x2 arrangement of 128x128, MFMA 32x32x16 bf16, dY and the
// weight tile both double-buffered in LDS.
#include "nf4_launch.h"

namespace nf4 {
namespace {

constexpr int TM = 256, TK = 256, TN = 64;
constexpr int ROWB = TN * 2 + 16;  // LDS row stride in bytes (64 bf16 + padding)

__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_k, int &tm, int &tk) {
  const int total = tiles_m * tiles_k;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + idx;
  constexpr int G = 8;
  const int per_group = G * tiles_k;
  const int group = t / per_group;
  const int first_m = group * G;
  const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
  const int in_group = t % per_group;
  tm = first_m + in_group % gsize;
  tk = in_group / gsize;
}

template <bool DX_BF16>
__global__ __launch_bounds__(256) void bwd_dx_kernel(const uint16_t *__restrict__ dY, int64_t M,
                                                     int64_t N, int64_t K,
                                                     const uint8_t *__restrict__ packed,
                                                     AbsmaxSrc src, void *__restrict__ dX,
                                                     int tiles_m, int tiles_k) {
  __shared__ __attribute__((aligned(16))) uint8_t sa[2][TM * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t sb[2][TK * ROWB];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tk;
  tile_of(blockIdx.x, tiles_m, tiles_k, tm, tk);
  const int64_t m0 = (int64_t)tm * TM, k0 = (int64_t)tk * TK;
  const float mu = src.dq ? *src.mean : 0.f;

  // dY staging: eight threads per 128-byte row segment, 32 rows per pass
  const int ar = tid >> 3, ac = tid & 7;
  const uint16_t *ap[8];
  bool aval[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + ar + 32 * i;
    aval[i] = row < M;
    ap[i] = dY + (aval[i] ? row : 0) * N + ac * 8;
  }
  // N may be ragged: the last reduction step masks columns n >= N
  // weight dequant: rows n0 + 2p and n0 + 2p + 1, K range k0 + 32q .. +32
  const int p = tid & 31, q = tid >> 5;
  const int64_t kq = k0 + 32 * q;
  const bool kval = kq < K;  // K % 64 == 0 and the tile start is < K, so kq+32 <= K when kq < K

  const int64_t nsteps = (N + TN - 1) / TN;
  const bool rows16 = (N % 8) == 0;  // dY rows start on 16-byte boundaries
  uint4 areg[8];
  uint4 creg[2];
  float ahreg[2];

  auto load_a = [&](int64_t s) {
    const int64_t n = s * TN + ac * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (aval[i] && rows16 && n + 8 <= N) {
        areg[i] = *reinterpret_cast<const uint4 *>(ap[i] + s * TN);
      } else if (aval[i] && n < N) {
        // ragged or unaligned rows: element-wise
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = (n + e < N) ? ap[i][s * TN + e] : (uint16_t)0;
        areg[i] = make_uint4(tmp[0] | (uint32_t)tmp[1] << 16, tmp[2] | (uint32_t)tmp[3] << 16,
                             tmp[4] | (uint32_t)tmp[5] << 16, tmp[6] | (uint32_t)tmp[7] << 16);
      } else {
        areg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto load_b = [&](int64_t s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t n = s * TN + 2 * p + h;
      const bool ok = kval && n < N;
      creg[h] = ok ? *reinterpret_cast<const uint4 *>(packed + n * (K / 2) + kq / 2) : make_uint4(0, 0, 0, 0);
      ahreg[h] = ok ? block_ahat(src, (n * K + kq) / kBlock, mu) : 0.f;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4 *>(&sa[buf][(ar + 32 * i) * ROWB + ac * 16]) = areg[i];
  };
  // dequantize the two rows and write [k][n] pairs into the weight tile
  auto store_b = [&](int buf) {
    const Lut t0 = make_lut(ahreg[0]), t1 = make_lut(ahreg[1]);
    const uint32_t c0[4] = {creg[0].x, creg[0].y, creg[0].z, creg[0].w};
    const uint32_t c1[4] = {creg[1].x, creg[1].y, creg[1].z, creg[1].w};
    uint8_t *base = &sb[buf][(32 * q) * ROWB + 4 * p];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t r0[4], r1[4];
      dequant8(c0[j], t0, r0);
      dequant8(c1[j], t1, r1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // r0[e] = {row0 k=8j+2e, row0 k=8j+2e+1}; pair rows per k
        const uint32_t lo = perm(r1[e], r0[e], 0x05040100u);  // k = 8j+2e: {row0, row1}
        const uint32_t hi = perm(r1[e], r0[e], 0x07060302u);  // k = 8j+2e+1
        *reinterpret_cast<uint32_t *>(base + (8 * j + 2 * e) * ROWB) = lo;
        *reinterpret_cast<uint32_t *>(base + (8 * j + 2 * e + 1) * ROWB) = hi;
      }
    }
  };

  // MFMA roles: wave (wm, wk) covers rows 128 wm .. +127 and K columns 128 wk .. +127
  const int wm = wave >> 1, wk = wave & 1;
  const int bl = lane & 31, kg = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  load_a(0);
  load_b(0);
  store_a(0);
  store_b(0);
  __syncthreads();

  for (int64_t s = 0; s < nsteps; ++s) {
    const int cur = (int)(s & 1);
    const bool more = s + 1 < nsteps;
    if (more) {
      load_a(s + 1);
      load_b(s + 1);
    }
    const uint8_t *abase = &sa[cur][(128 * wm + bl) * ROWB + kg * 64];
    const uint8_t *bbase = &sb[cur][(128 * wk + bl) * ROWB + kg * 64];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 bv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bv[t] = as_bf16x8(*reinterpret_cast<const uint4 *>(bbase + 32 * t * ROWB + 16 * j));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8 av = as_bf16x8(*reinterpret_cast<const uint4 *>(abase + 32 * i * ROWB + 16 * j));
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv[t], acc[i][t], 0, 0, 0);
      }
    }
    if (more) {
      store_a(cur ^ 1);
      store_b(cur ^ 1);
    }
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t col = k0 + 128 * wk + 32 * t + bl;
    if (col >= K) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + 128 * wm + 32 * i + 8 * (r / 4) + 4 * kg + (r % 4);
        if (row < M) {
          const int64_t off = row * K + col;
          if (DX_BF16)
            reinterpret_cast<uint16_t *>(dX)[off] = (uint16_t)(pack_bf16x2(acc[i][t][r], 0.f) & 0xffffu);
          else
            reinterpret_cast<float *>(dX)[off] = acc[i][t][r];
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_bwd_dx(const void *dy, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                         const AbsmaxSrc &src, void *dx, int dx_is_bf16, hipStream_t stream) {
  const uint16_t *dY = reinterpret_cast<const uint16_t *>(dy);
  const int tiles_m = (int)((M + TM - 1) / TM), tiles_k = (int)((K + TK - 1) / TK);
  const dim3 g((unsigned)(tiles_m * tiles_k)), b(256);
  if (dx_is_bf16)
    hipLaunchKernelGGL((bwd_dx_kernel<true>), g, b, 0, stream, dY, M, N, K, packed, src, dx, tiles_m, tiles_k);
  else
    hipLaunchKernelGGL((bwd_dx_kernel<false>), g, b, 0, stream, dY, M, N, K, packed, src, dx, tiles_m, tiles_k);
  return hipGetLastError();
}

}  // namespace nf4
