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
//                     staged through LDS (double-buffered, filled by direct
//                     global->LDS loads), each wave
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

constexpr int BM = 256, BN = 256, BK = 128;
constexpr int XTILE = BM * BK * 2;          // 64 KiB: 256 rows of 256 bytes

typedef __attribute__((address_space(3))) void lds_void;

// Workgroups are dealt round-robin to the 8 XCDs; renumber them so each XCD
// takes a contiguous run of tiles, then walk tiles in groups of 4 M-tiles so
// that workgroups running together share X row panels and weight columns in
// their XCD's L2.
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

// A lane's weight state for one K-step: the 64 codes (one whole block) of
// each of its two columns and the blocks' absmax state.
struct Codes {
  uint4 c0a, c0b, c1a, c1b;
  AbsmaxRaw r0, r1;
};

// The 128 MFMAs of one 128-wide K-step for a wave's 256x64 slice.  Lane group
// kg owns K range kg*64 .. +63 of the step -- one whole block per column, one
// LUT per 64 weights; MFMA slice j (0..7) takes elements 8j..8j+7 of it from
// both operands.  Dequantization of slice j+1 and the A-fragment LDS reads of
// slice j+1 are issued while the 16 MFMAs of slice j run.  `xt` is the X tile
// in LDS; row R's 16-byte chunk c sits at chunk c ^ (R & 7).
template <bool DQ>
__device__ __forceinline__ void mma_tile(f32x16 (&acc)[8][2], const uint8_t *xt, int bl, int kg,
                                         const Codes &cd, float mu, bool real) {
  const Lut t0 = make_lut(real ? ahat_of(cd.r0, DQ, mu) : 0.f);
  const Lut t1 = make_lut(real ? ahat_of(cd.r1, DQ, mu) : 0.f);
  const uint32_t w0[8] = {cd.c0a.x, cd.c0a.y, cd.c0a.z, cd.c0a.w, cd.c0b.x, cd.c0b.y, cd.c0b.z, cd.c0b.w};
  const uint32_t w1[8] = {cd.c1a.x, cd.c1a.y, cd.c1a.z, cd.c1a.w, cd.c1b.x, cd.c1b.y, cd.c1b.z, cd.c1b.w};
  const uint8_t *row = xt + bl * 256;
  const int sw = bl & 7;
  uint4 a[8];
  uint32_t b0[4], b1[4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a[i] = *reinterpret_cast<const uint4 *>(row + 32 * i * 256 + (((kg * 8) ^ sw) << 4));
  dequant8(w0[0], t0, b0);
  dequant8(w1[0], t1, b1);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    uint4 an[8];
    uint32_t bn0[4], bn1[4];
    if (j < 7) {
      const int off = ((kg * 8 + j + 1) ^ sw) << 4;
#pragma unroll
      for (int i = 0; i < 8; ++i) an[i] = *reinterpret_cast<const uint4 *>(row + 32 * i * 256 + off);
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
    if (j < 7) {
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
}

// X tiles (256 rows x 128 K) reach LDS by direct global->LDS loads (no
// register staging), double-buffered: the next tile loads during a whole
// K-step of MFMA work.  Wave w's load instruction i fills LDS rows
// 4(16w + i) .. +3; lane l takes row 4(16w + i) + l/16 and physical chunk
// l%16, which holds logical chunk (l%16) ^ (row & 7) -- the swizzle that keeps
// the MFMA-fragment reads (eight rows, one logical chunk) free of LDS bank
// conflicts.  One barrier per K-step, after this wave's loads of the tile
// about to be read have completed.
template <bool Y_BF16, bool DQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void fwd_large_kernel(
    const uint16_t *__restrict__ X, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, void *__restrict__ Y, int tiles_m, int tiles_n) {
  // two separate arrays (not one indexed by stage) so that the compiler can
  // tell the tile being read from the tile being loaded and does not make the
  // reads wait for those loads
  __shared__ __attribute__((aligned(1024))) uint8_t xs0[XTILE];
  __shared__ __attribute__((aligned(1024))) uint8_t xs1[XTILE];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const float mu = DQ ? *src.mean : 0.f;

  // B operand: this lane's two weight rows (one per 32-column subtile).
  // Columns past N and rows past M load in-bounds stand-ins; their outputs
  // are never stored, so every load is unconditional.
  const int bl = lane & 31, kg = lane >> 5;
  int64_t ncol[2];
  const uint4 *wq[2];
  int64_t blk0[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    ncol[t] = n0 + 64 * wave + 32 * t + bl;
    const int64_t nn = ncol[t] < N ? ncol[t] : N - 1;
    wq[t] = reinterpret_cast<const uint4 *>(packed + nn * (K / 2) + kg * 32);
    blk0[t] = nn * (K / kBlock) + kg;
  }

  // direct-to-LDS sources: row 4(16w + i) + lane/16, logical chunk (lane%16) ^ (row & 7)
  const int rsub = lane >> 4;
  const uint16_t *xsrc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * (16 * wave + i) + rsub;
    const int chunk = (lane & 15) ^ (r & 7);
    const int64_t row = m0 + r;
    xsrc[i] = X + (row < M ? row : M - 1) * K + chunk * 8;
  }
  const int64_t nk = (K + BK - 1) / BK;
  const bool half = (K % BK) != 0;
  auto issue_x = [&](int64_t kt, uint8_t *dst) {
    // in a 64-wide last step, logical chunks 8..15 (lane bit 3) lie past the
    // row's end: load the chunk 64 columns back instead (it meets a^ = 0)
    const int64_t koff = kt * BK - ((half && kt == nk - 1 && (lane & 8)) ? 64 : 0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(xsrc[i] + koff),
                                       (lds_void *)(dst + (16 * wave + i) * 1024), 16, 0, 0);
  };
  auto issue_codes = [&](int64_t kt, Codes &cd) {
    cd.c0a = wq[0][kt * 4];
    cd.c0b = wq[0][kt * 4 + 1];
    cd.c1a = wq[1][kt * 4];
    cd.c1b = wq[1][kt * 4 + 1];
    cd.r0 = load_raw<DQ>(src, blk0[0] + 2 * kt);
    cd.r1 = load_raw<DQ>(src, blk0[1] + 2 * kt);
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][t][r] = 0.f;

  // K-steps run in pairs (one per LDS buffer); a step past the last real one
  // re-reads tile nk-1 with a^ forced to 0, so it adds exact zeros.  K % 64 ==
  // 0 but K % 128 may be 64: then the last real step's upper half (lane group
  // kg = 1) also gets a^ = 0.
  const int64_t nk2 = (nk + 1) & ~(int64_t)1;
  Codes cur, nxt;
  auto clampk = [&](int64_t k) { return k < nk ? k : nk - 1; };
  // the upper half of a 64-wide last step points one block past the row: load
  // the lower half's block instead (its values are multiplied by a^ = 0)
  auto real_of = [&](int64_t kt) { return kt < nk && !(half && kt == nk - 1 && kg == 1); };
  auto issue_codes_safe = [&](int64_t kt, Codes &cd) {
    if (half && kt == nk - 1 && kg == 1) {
      // stay inside the row: reuse the lower half's codes and block
      cd.c0a = wq[0][kt * 4 - 4 + 2];
      cd.c0b = wq[0][kt * 4 - 4 + 3];
      cd.c1a = wq[1][kt * 4 - 4 + 2];
      cd.c1b = wq[1][kt * 4 - 4 + 3];
      cd.r0 = load_raw<DQ>(src, blk0[0] + 2 * kt - 1);
      cd.r1 = load_raw<DQ>(src, blk0[1] + 2 * kt - 1);
    } else {
      issue_codes(kt, cd);
    }
  };
  issue_x(0, xs0);
  issue_codes_safe(0, cur);
  auto step = [&](int64_t kt, const uint8_t *rd, uint8_t *wr) {
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    const int64_t kn = clampk(kt + 1);
    issue_x(kn, wr);
    issue_codes_safe(kn, nxt);
    mma_tile<DQ>(acc, rd, bl, kg, cur, mu, real_of(kt));
    cur = nxt;
  };
  for (int64_t kt = 0; kt < nk2; kt += 2) {
    step(kt, xs0, xs1);
    step(kt + 1, xs1, xs0);
  }
  __builtin_amdgcn_s_waitcnt(0);

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
    if (src.dq) {
      if (y_is_bf16)
        hipLaunchKernelGGL((fwd_large_kernel<true, true>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
      else
        hipLaunchKernelGGL((fwd_large_kernel<false, true>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
    } else {
      if (y_is_bf16)
        hipLaunchKernelGGL((fwd_large_kernel<true, false>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
      else
        hipLaunchKernelGGL((fwd_large_kernel<false, false>), g, b, 0, stream, X, M, N, K, packed, src, y, tiles_m, tiles_n);
    }
  }
  return hipGetLastError();
}

}  // namespace nf4
