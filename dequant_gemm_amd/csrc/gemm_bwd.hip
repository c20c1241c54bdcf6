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
// weight tile both double-buffered in LDS.  The codes are loaded two steps
// ahead and the next step's weight tile is dequantized between the current
// step's MFMAs, so the dequantization overlaps the matrix cores.
#include "nf4_launch.h"

namespace nf4 {
namespace {

#ifndef NF4_BWD_SCHED
#define NF4_BWD_SCHED 0
#endif

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
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dx_kernel(const uint16_t *__restrict__ dY, int64_t M,
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

  // dY staging: eight threads per 128-byte row segment, 32 rows per pass.
  // Rows past M load row M-1 (their outputs are never stored); columns past N
  // meet weight values forced to zero, so whatever is loaded there is
  // multiplied by zero.
  const int ar = tid >> 3, ac = tid & 7;
  const uint16_t *ap[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = m0 + ar + 32 * i;
    ap[i] = dY + (row < M ? row : M - 1) * N;
  }
  // weight dequant: rows n0 + 2p and n0 + 2p + 1, K range k0 + 32q .. +32
  const int p = tid & 31, q = tid >> 5;
  const int64_t kq = k0 + 32 * q;
  const bool kval = kq < K;  // K % 64 == 0: if kq < K then kq + 32 <= K
  const int64_t kqc = kval ? kq : 0;

  const int64_t nsteps = (N + TN - 1) / TN;
  const bool rows16 = (N % 8) == 0;  // dY rows start on 16-byte boundaries
  uint4 areg[8];
  uint4 creg[2];       // codes of the step after next
  AbsmaxRaw rreg[2];
  bool cok[2];

  auto load_a = [&](int64_t s) {
    const int64_t n = s * TN + ac * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (rows16 && n + 8 <= N) {
        areg[i] = *reinterpret_cast<const uint4 *>(ap[i] + n);
      } else {
        uint16_t tmp[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) tmp[e] = ap[i][n + e < N ? n + e : N - 1];
        areg[i] = make_uint4(tmp[0] | (uint32_t)tmp[1] << 16, tmp[2] | (uint32_t)tmp[3] << 16,
                             tmp[4] | (uint32_t)tmp[5] << 16, tmp[6] | (uint32_t)tmp[7] << 16);
      }
    }
  };
  auto load_b = [&](int64_t s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t n = s * TN + 2 * p + h;
      cok[h] = kval && n < N;
      const int64_t nc = n < N ? n : N - 1;
      creg[h] = *reinterpret_cast<const uint4 *>(packed + nc * (K / 2) + kqc / 2);
      rreg[h] = load_absmax_raw(src, (nc * K + kqc) / kBlock);
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4 *>(&sa[buf][(ar + 32 * i) * ROWB + ac * 16]) = areg[i];
  };
  // Dequantize dword j (eight K values) of both rows and write the [k][n]
  // pairs into the weight tile.
  auto store_b_part = [&](int buf, int j, const uint32_t c0[4], const uint32_t c1[4], const Lut &t0,
                          const Lut &t1) {
    uint8_t *base = &sb[buf][(32 * q) * ROWB + 4 * p];
    uint32_t r0[4], r1[4];
    dequant8(c0[j], t0, r0);
    dequant8(c1[j], t1, r1);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // r0[e] = {row0 at k = 8j+2e, row0 at 8j+2e+1}; pair the two rows per k
      *reinterpret_cast<uint32_t *>(base + (8 * j + 2 * e) * ROWB) = perm(r1[e], r0[e], 0x05040100u);
      *reinterpret_cast<uint32_t *>(base + (8 * j + 2 * e + 1) * ROWB) = perm(r1[e], r0[e], 0x07060302u);
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

  // prologue: step 0 fully staged, codes of step 1 in registers
  load_a(0);
  load_b(0);
  store_a(0);
  {
    const uint32_t c0[4] = {creg[0].x, creg[0].y, creg[0].z, creg[0].w};
    const uint32_t c1[4] = {creg[1].x, creg[1].y, creg[1].z, creg[1].w};
    const Lut t0 = make_lut(cok[0] ? ahat_of(rreg[0], src.dq, mu) : 0.f);
    const Lut t1 = make_lut(cok[1] ? ahat_of(rreg[1], src.dq, mu) : 0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) store_b_part(0, j, c0, c1, t0, t1);
  }
  if (nsteps > 1) load_b(1);
  __syncthreads();

  for (int64_t s = 0; s < nsteps; ++s) {
    const int cur = (int)(s & 1);
    const bool more = s + 1 < nsteps;
    // codes for step s+1 (loaded one step ago); start the loads for s+2
    const uint32_t c0[4] = {creg[0].x, creg[0].y, creg[0].z, creg[0].w};
    const uint32_t c1[4] = {creg[1].x, creg[1].y, creg[1].z, creg[1].w};
    const AbsmaxRaw r0 = rreg[0], r1 = rreg[1];
    const bool ok0 = cok[0], ok1 = cok[1];
    if (more) load_a(s + 1);
    if (s + 2 < nsteps) load_b(s + 2);
    Lut t0, t1;
    if (more) {
      t0 = make_lut(ok0 ? ahat_of(r0, src.dq, mu) : 0.f);
      t1 = make_lut(ok1 ? ahat_of(r1, src.dq, mu) : 0.f);
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
      // the next step's weight tile, a quarter at a time, into the other buffer
      if (more) store_b_part(cur ^ 1, j, c0, c1, t0, t1);
    }
    if (more) store_a(cur ^ 1);
#if NF4_BWD_SCHED == 1
    __builtin_amdgcn_iglp_opt(1);
#elif NF4_BWD_SCHED == 2
    __builtin_amdgcn_iglp_opt(0);
#endif
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
