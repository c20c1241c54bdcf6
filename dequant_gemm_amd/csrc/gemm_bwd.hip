// gemm_bwd.hip -- fused NF4-dequant GEMM, backward with respect to the input:
// dX = dY W^ (no gradient for the frozen weight).
//
// "Zenbit" page, section "What's inside", bullet zenbit.pallas_nf4: a fused
// backward pass forms dL/dX without materialising the dequantized weight, and
// dL/dW is not computed for a frozen quantized base weight.
//
// dY is bf16 [M, N]; the weight is NF4 [N, K]; dX is fp32 (or bf16) [M, K].
// The reduction runs over N while the weight's 64-blocks run along K, so the
// dequantized weight has to change orientation before it can feed the MFMA
// (whose operands hold eight consecutive reduction indices per lane).
//
// Three kernels:
//   bwd_dx_small_kernel    up to 16 rows of dY (more as grid rows of 16 while
//                          cheaper), N % 8 == 0 and N < 2^24: one workgroup per
//                          32 or 64 output columns streams the whole weight
//                          band, 16 waves taking 64-row steps in turn.
//   bwd_dx_wide_kernel     otherwise, N % 8 == 0 (16-byte dY rows) and N < 2^24: dY
//                          through buffer-to-LDS loads, each wave dequantizes
//                          its own 64 weight columns row by row into a private
//                          LDS tile and reads MFMA operands back with
//                          transposing LDS reads; one wave per SIMD.
//   bwd_dx_generic_kernel  any shape: dY staged through registers, the
//                          weight tile written to LDS already transposed.
#include "nf4_launch.h"

namespace nf4 {
namespace {

// ------------------------------------------------------------ generic kernel
//
// Each thread dequantizes two weight rows over 32 K, pairs the two rows'
// values per K into one 32-bit word and writes it to an LDS tile stored
// K-major ([k][n]); the MFMA then reads B fragments from that tile with
// 16-byte loads.  Tiles: 256 (M) x 256 (K) outputs per workgroup, reduction
// steps of 64 N, four waves in a 2x2 arrangement of 128x128, dY and the
// weight tile both double-buffered in LDS.  The codes are loaded two steps
// ahead and the next step's weight tile is dequantized between the current
// step's MFMAs.
namespace generic {

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

template <bool DX_BF16, bool LR, bool FP4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dx_generic_kernel(const uint16_t *__restrict__ dY, int64_t M,
                                                     int64_t N, int64_t K,
                                                     const uint8_t *__restrict__ packed,
                                                     AbsmaxSrc src, LowRank lr, void *__restrict__ dX,
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
      rreg[h] = load_absmax_raw(src, (nc * K + kqc) >> src.lbs);
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
    const Lut t0 = make_lut<FP4>(cok[0] ? ahat_of(rreg[0], src.dq, mu) : 0.f);
    const Lut t1 = make_lut<FP4>(cok[1] ? ahat_of(rreg[1], src.dq, mu) : 0.f);
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
      t0 = make_lut<FP4>(ok0 ? ahat_of(r0, src.dq, mu) : 0.f);
      t1 = make_lut<FP4>(ok1 ? ahat_of(r1, src.dq, mu) : 0.f);
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
    __syncthreads();
  }

  if (LR) {
    // adapter term, rank slices of 16: lane group kg takes ranks 16s + 8kg .. +7
    // (rows past M and columns past K read existing ones; never stored)
    const uint16_t *vrow[4], *urow[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t col = k0 + 128 * wk + 32 * t + bl;
      vrow[t] = lr.v + (col < K ? col : K - 1) * lr.r + 8 * kg;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + 128 * wm + 32 * i + bl;
      urow[i] = lr.u + (row < M ? row : M - 1) * lr.r + 8 * kg;
    }
    // two slices in flight: slice s + 1 loads while slice s multiplies
    auto load = [&](int s, uint4 (&bv)[4], uint4 (&av)[4]) {
#pragma unroll
      for (int t = 0; t < 4; ++t) bv[t] = *reinterpret_cast<const uint4 *>(vrow[t] + 16 * s);
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const uint4 *>(urow[i] + 16 * s);
    };
    auto mma = [&](const uint4 (&bv)[4], const uint4 (&av)[4]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[i]), as_bf16x8(bv[t]), acc[i][t], 0, 0, 0);
    };
    const int ns = lr.r / 16;
    uint4 b0[4], b1[4], a0[4], a1[4];
    load(0, b0, a0);
    int s = 0;
    for (; s + 2 <= ns; s += 2) {
      load(s + 1, b1, a1);
      mma(b0, a0);
      if (s + 2 < ns) load(s + 2, b0, a0);
      mma(b1, a1);
    }
    if (s < ns) mma(b0, a0);
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

}  // namespace generic

namespace tr_kernel {
// ------------------------------------------------------------ main kernel
//
// Workgroup tile 256 (M) x 256 (K), four waves, one per SIMD; wave w owns the
// 64 output columns k0 + 64w .. +63 (two halves c of 32) over all 256 rows:
// 8 x 2 MFMA 32x32x16 tiles, 256 fp32 accumulators per lane.  The reduction
// runs over N in steps of 64.
//
// A operand (dY): 256 x 64 tiles reach LDS by buffer-to-LDS loads through
// three stages, laid out and read exactly like the X tiles of the forward
// kernel; each A fragment feeds two MFMAs (the two column halves).
//
// B operand (W^, 64 rows n x the wave's 64 columns k): lane l dequantizes row
// n = 64s + l of the wave's columns -- 64 consecutive codes: one block and one
// table at block sizes of 64 and more, two at 32 -- and writes the 64 bf16
// values as one row of a per-wave LDS tile.  The MFMA wants eight consecutive
// n of one column per lane; the transposing LDS read ds_read_b64_tr_b16
// delivers exactly that: within a 16-lane group, output lane i element e is
// element i%4 of the 8 bytes addressed by source lane 4e + i/4, so source lane
// j of group G addresses row r0 + 4h + j/4 and columns
// 32c + 16(G%2) + 4(j%4) .. +3 (kg = G/2, h = which half of the 8 n, c = the
// column half), and output lane i receives rows r0 + 4h .. +3 of column
// 32c + 16(G%2) + i; r0 = 32kg + 8sl is the first of the eight n that lane
// group kg's A fragment holds in slice sl.
//
// Against two waves of 32 columns per SIMD this halves the A-fragment reads
// and the per-block tables per flop; the price is that one wave must hide its
// own latencies.
constexpr int TM = 256, TK = 256, TN = 64;
constexpr int NWAVE_W = 4;
constexpr int AROW = TN * 2;             // 128-byte dY rows in LDS
constexpr int ATILE = TM * AROW;         // 32 KiB
constexpr int BROW_W = 144;              // weight-tile row: 128 bytes of bf16 + 16 of padding
constexpr int BTILE_W = TN * BROW_W;     // per-wave weight tile: 64 rows x 64 bf16

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void tile_of_main(int bid, int tiles_m, int tiles_k, int &tm, int &tk) {
  const int total = tiles_m * tiles_k;
  const int q = total / 8, r = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  const int t = xcd * q + (xcd < r ? xcd : r) + idx;
  constexpr int G = 4;
  const int per_group = G * tiles_k;
  const int group = t / per_group;
  const int first_m = group * G;
  const int gsize = tiles_m - first_m < G ? tiles_m - first_m : G;
  const int in_group = t % per_group;
  tm = first_m + in_group % gsize;
  tk = in_group / gsize;
}

__device__ __forceinline__ void sched_cut() { __builtin_amdgcn_sched_barrier(0); }

template <typename T>
__device__ __forceinline__ const uint8_t *uniform_ptr(const T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t *>(((uint64_t)hi << 32) | lo);
}

template <bool FP4>
__device__ __forceinline__ void lut_quarter(float ahat, int q, Lut &t) {
  const uint32_t p0 = pack_bf16x2(__fmul_rn(lvl<FP4>(4 * q), ahat), __fmul_rn(lvl<FP4>(4 * q + 1), ahat));
  const uint32_t p1 = pack_bf16x2(__fmul_rn(lvl<FP4>(4 * q + 2), ahat), __fmul_rn(lvl<FP4>(4 * q + 3), ahat));
  t.lo[q] = perm(p1, p0, 0x06040200u);
  t.hi[q] = perm(p1, p0, 0x07050301u);
}

// A lane's weight state for one N-step: 64 codes of its weight row and the
// absmax state of their block (blocks, at block size 32).
template <bool BS32>
struct RowCodesW {
  uint4 w0, w1;
  ChunkAbsmax<BS32> r;
};

template <bool DX_BF16, bool DQ, bool FP4, bool BS32, bool LR>
__global__ __launch_bounds__(64 * NWAVE_W) __attribute__((amdgpu_waves_per_eu(1, 1))) void bwd_dx_wide_kernel(
    const uint16_t *__restrict__ dY, int64_t M, int64_t N, int64_t K, const uint8_t *__restrict__ packed,
    AbsmaxSrc src, LowRank lr, void *__restrict__ dX, int tiles_m, int tiles_k) {
  // the dY stages first (larger alignment places them at the lowest LDS
  // addresses), so that their fragment reads fold the tile offsets into the
  // 16-bit immediate of the LDS read instead of forming each address
  __shared__ __attribute__((aligned(4096))) uint8_t as0[ATILE];
  __shared__ __attribute__((aligned(4096))) uint8_t as1[ATILE];
  __shared__ __attribute__((aligned(4096))) uint8_t as2[ATILE];
  __shared__ __attribute__((aligned(1024))) uint8_t bs[NWAVE_W * BTILE_W];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  int tm, tk;
  tile_of_main(blockIdx.x, tiles_m, tiles_k, tm, tk);
  const int64_t m0 = (int64_t)tm * TM, k0 = (int64_t)tk * TK;
  const float mu = DQ ? *src.mean : 0.f;
  const int bl = lane & 31, kg = lane >> 5;

  // this wave's 64 output columns (K % 64 == 0: all valid or all past K; past K
  // they read columns K-64 .. K-1 and are never stored)
  const int64_t kcol = k0 + 64 * wave;
  const int64_t kc = kcol < K ? kcol : K - 64;
  // The weight rows are dequantized with the even/odd selectors (two byte
  // permutes fewer per eight codes): the eight values of each code word go to
  // the tile in the column order 0, 2, 4, 6, 1, 3, 5, 7, so tile column q holds
  // weight column 8 (q / 8) + 2 (q % 4) + (q % 8) / 4, and lane l's results
  // (tile column l % 32 of each half) belong to that column.
  const int bcol = (bl & ~7) | ((bl & 3) << 1) | ((bl >> 2) & 1);
  // weight row of this lane in step s: n = 64s + lane; the flat index of its
  // first column, n K + kc, shifted by log2(block size) gives its block (64
  // columns never straddle a block of 64 or more; at 32 they are two blocks)
  const uint8_t *wq = packed + (int64_t)lane * (K / 2) + kc / 2;
  const int64_t flat0 = (int64_t)lane * K + kc;

  // dY tile loads, as the forward kernel's X tiles: wave w's load i (0..7)
  // covers tile rows 8(8w + i) .. +7; one descriptor per wave and step sized
  // to its existing rows; a 16-byte chunk past N gets an offset beyond the
  // descriptor and loads zeros.  (Requires N % 8 == 0 and N < 2^24.)
  const int64_t wrow0 = m0 + 64 * wave;
  const int64_t wrows = M - wrow0 < 0 ? 0 : (M - wrow0 > 64 ? 64 : M - wrow0);
  const int wbytes = __builtin_amdgcn_readfirstlane((int)(uint32_t)(wrows * N * 2));
  const uint8_t *ywave = uniform_ptr(dY + (wrows > 0 ? wrow0 : 0) * N);
  uint32_t yvoff[8];
  int ylast = 0;   // bit i: load i's chunk exists in the last step (N need not be a multiple of 64)
  {
    const int64_t lastn = N - (((N + TN - 1) / TN) - 1) * TN;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int ch = (lane & 7) ^ ((r >> 1) & 7);
      yvoff[i] = (uint32_t)(r * N * 2) + ((uint32_t)ch << 4);
      ylast |= (8 * ch < lastn) << i;
    }
  }
  int aoff[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) aoff[j] = bl * AROW + (((4 * kg + j) ^ ((bl >> 1) & 7)) << 4);

  // per-wave weight tile: row n at n * 144 bytes (the padding keeps both the
  // row writes and the transposing reads clear of most bank conflicts)
  uint8_t *bw = bs + wave * BTILE_W;
  // transposing reads for slice sl, half h, column half c: source lane j of
  // group G reads row 32kg + 8sl + 4h + j/4, columns 32c + 16(G%2) + 4(j%4):
  // 16-byte chunk 4c + 2(G%2) + (j%4)/2, byte 8 * ((j%4) & 1); the slice, half
  // and column-half parts of the address are an immediate
  uint32_t btr;
  {
    const int G = lane >> 4, j = lane & 15;
    const int rbase = 32 * (G >> 1) + (j >> 2);
    const int chunk = 2 * (G & 1) + ((j & 3) >> 1);
    btr = (uint32_t)(uintptr_t)bw + (uint32_t)(rbase * BROW_W + (chunk << 4) + 8 * (j & 1));
  }
  const int64_t ns = (N + TN - 1) / TN;
  auto clamps = [&](int64_t s) { return s < ns ? s : ns - 1; };
  auto yrsrc = [&](int64_t s) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(ywave + clamps(s) * (TN * 2)), (short)0,
                                             wbytes, 0x00020000);
  };
  auto issue_y1 = [&](__amdgpu_buffer_rsrc_t rs, int64_t s, uint8_t *dst, int i) {
    const bool in = clamps(s) < ns - 1 || ((ylast >> i) & 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(dst + (8 * wave + i) * 1024), 16,
                                             in ? yvoff[i] : 0x80000000u, 0, 0, 0);
  };
  // a row past N loads row N-1's codes (in bounds) and gets a^ = 0
  auto issue_codes = [&](int64_t s, RowCodesW<BS32> &c) {
    const int64_t sc = clamps(s);
    const int64_t n = sc * TN + lane;
    const int64_t dn = n < N ? sc * TN : N - 1 - lane;     // row offset from this lane's base row
    const uint4 *wp = reinterpret_cast<const uint4 *>(wq + dn * (K / 2));
    c.w0 = wp[0];
    c.w1 = wp[1];
    c.r.template load<DQ>(src, (flat0 + dn * K) >> src.lbs);
  };
  auto ahat_at = [&](int64_t s, const RowCodesW<BS32> &c, int u) {
    const float v = c.r.ahat(u, DQ, mu);
    return (s < ns && s * TN + lane < N) ? v : 0.f;
  };
  // The transposing read is issued as inline assembly: the compiler's wait
  // insertion cannot tell the intrinsic's LDS address from the dY tiles that
  // buffer-to-LDS loads are filling and would wait for all of those loads
  // before every such read.  Its results are waited for explicitly (an
  // lgkmcnt wait) before the MFMA that consumes them.
  auto tr_read = [&](int sl, int h, int c) {
    v4s v;
    switch ((8 * sl + 4 * h) * BROW_W + 64 * c) {
#define NF4_TR(B) case B: asm volatile("ds_read_b64_tr_b16 %0, %1 offset:" #B : "=v"(v) : "v"(btr) : "memory"); break;
      NF4_TR(0) NF4_TR(576) NF4_TR(1152) NF4_TR(1728) NF4_TR(2304) NF4_TR(2880) NF4_TR(3456) NF4_TR(4032)
      NF4_TR(64) NF4_TR(640) NF4_TR(1216) NF4_TR(1792) NF4_TR(2368) NF4_TR(2944) NF4_TR(3520) NF4_TR(4096)
#undef NF4_TR
    }
    return v;
  };
  auto write_row = [&](const uint32_t st[32]) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      *reinterpret_cast<uint4 *>(bw + lane * BROW_W + (c << 4)) =
          make_uint4(st[4 * c], st[4 * c + 1], st[4 * c + 2], st[4 * c + 3]);
  };
  auto dequant_word = [&](uint32_t wd, const Lut &t, uint32_t *out, int phase, Sel4 &sa, Sel4 &sb) {
    if (phase == 0) select8_even_odd(wd, sa, sb);
    if (phase == 1) lookup4(sa, t, out[0], out[1]);
    if (phase == 2) lookup4(sb, t, out[2], out[3]);
  };

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][c][r] = 0.f;

  uint4 a[8];
  v4s b0[2][2], b1[2][2];   // B fragments [column half][n half] of the current and the next slice
  uint32_t st[32];          // the next step's dequantized weight row, staged for the LDS write
  RowCodesW<BS32> cs0, cs1, cs2;

  // prologue: codes of steps 0-2 and dY tiles 0 and 1 in flight; step 0's row
  // dequantized and written, its slice-0 B fragments read
  {
    RowCodesW<BS32> c0;
    issue_codes(0, c0);
    const __amdgpu_buffer_rsrc_t r0 = yrsrc(0), r1 = yrsrc(1);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_y1(r0, 0, as0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) issue_y1(r1, 1, as1, i);
    issue_codes(1, cs1);
    issue_codes(2, cs2);
    Lut t;
    const float ah = ahat_at(0, c0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) lut_quarter<FP4>(ah, q, t);
    const uint32_t wd[8] = {c0.w0.x, c0.w0.y, c0.w0.z, c0.w0.w, c0.w1.x, c0.w1.y, c0.w1.z, c0.w1.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (BS32 && c == 4) {
        const float ah1 = ahat_at(0, c0, 1);
#pragma unroll
        for (int q = 0; q < 4; ++q) lut_quarter<FP4>(ah1, q, t);
      }
      Sel4 sa, sb;
      select8_even_odd(wd[c], sa, sb);
      lookup4(sa, t, st[4 * c], st[4 * c + 1]);
      lookup4(sb, t, st[4 * c + 2], st[4 * c + 3]);
    }
    write_row(st);
    // the row has landed before it is read back (the transposing reads are not
    // ordered behind this wave's earlier LDS writes by anything else here)
    __builtin_amdgcn_s_waitcnt(lgkm_imm(0));
    b0[0][0] = tr_read(0, 0, 0);
    b0[0][1] = tr_read(0, 1, 0);
    b0[1][0] = tr_read(0, 0, 1);
    b0[1][1] = tr_read(0, 1, 1);
  }
  // every load landed, dY tiles 0 and 1 included; the slice-0 B fragments read
  // (lgkmcnt(0)).  The wait is for all vector-memory operations: a count that
  // leaves later loads in flight does not order the buffer-to-LDS loads before
  // them (measured: a wait that let the last eight loads run on let tiles be read
  // before they had landed)
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~(0xF << 8));
  __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = *reinterpret_cast<const uint4 *>(as0 + aoff[0] + i * 32 * AROW);

  // One N-step as 32 groups of two MFMAs (slice j = groups 8j .. 8j+7; group g
  // of a slice: M-tile g against both column halves):
  //   A reads     after its MFMAs, group g refills a[g] for the next slice;
  //               the next step's slice 0 after the hand-over, from `nx`
  //   B reads     the next slice's four transposing reads in groups 0-3
  //   dY loads    the tile two steps ahead into `ld`: groups 0, 2, ..., 14
  //   dequant     the next step's table (groups 0, 1) and its eight code
  //               words (groups 2-25), staged in registers; at block size 32
  //               words 0-3 in groups 2-13, the second block's table in
  //               groups 14-15 (in place) and words 4-7 in groups 16-27;
  //               written to the weight tile two 16-byte chunks per group in
  //               groups 24-27 (the step's last B reads completed at group 24)
  //   hand-over   before group 28: this wave's LDS traffic is complete and all
  //               its loads have landed (the next dY tile among them; the tile
  //               two steps ahead was issued in groups 0-14), barrier, codes
  //               three steps ahead, the next step's slice-0 B reads
  auto step = [&](int64_t s, uint8_t *rd, uint8_t *nx, uint8_t *ld, const RowCodesW<BS32> &cn, RowCodesW<BS32> &cfill) {
    Sel4 sa, sb;
    Lut t;
    float ahn = 0.f;
    const __amdgpu_buffer_rsrc_t rsl = yrsrc(s + 2);
    const uint32_t wd[8] = {cn.w0.x, cn.w0.y, cn.w0.z, cn.w0.w, cn.w1.x, cn.w1.y, cn.w1.z, cn.w1.w};
    static_for<32>([&](auto rcst) {
      constexpr int r = decltype(rcst)::value;
      constexpr int slice = r / 8, g = r % 8;
      v4s(*bc)[2] = (slice & 1) ? b1 : b0;
      v4s(*bn)[2] = (slice & 1) ? b0 : b1;
      if constexpr (r == 28) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & ~(0xF << 8));   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        sched_cut();
        issue_codes(s + 3, cfill);
        // the next step's slice-0 fragments, only if there is a next step: the
        // compiler takes an inline-asm load's result as written at once, so a
        // result nothing consumes would leave its registers free for reuse while
        // the load is still in flight
        if (s + 1 < ns) {
          b0[0][0] = tr_read(0, 0, 0);
          b0[0][1] = tr_read(0, 1, 0);
          b0[1][0] = tr_read(0, 0, 1);
          b0[1][1] = tr_read(0, 1, 1);
        }
        sched_cut();
      }
      if constexpr (g == 0) {
        // this slice's B fragments: read in groups 0-3 of the previous slice
        // (then four A reads) or after the hand-over (then eight A reads)
        if constexpr (slice == 0)
          __builtin_amdgcn_s_waitcnt(lgkm_imm(8));
        else
          __builtin_amdgcn_s_waitcnt(lgkm_imm(4));
        sched_cut();
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, (uint4){(uint32_t)__builtin_bit_cast(uint64_t, bc[c][0]),
                                                             (uint32_t)(__builtin_bit_cast(uint64_t, bc[c][0]) >> 32),
                                                             (uint32_t)__builtin_bit_cast(uint64_t, bc[c][1]),
                                                             (uint32_t)(__builtin_bit_cast(uint64_t, bc[c][1]) >> 32)});
        acc[g][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[g]), bv, acc[g][c], 0, 0, 0);
      }
      if constexpr (slice < 3) {
        a[g] = *reinterpret_cast<const uint4 *>(rd + aoff[slice + 1] + g * 32 * AROW);
        if constexpr (g < 4) bn[g >> 1][g & 1] = tr_read(slice + 1, g & 1, g >> 1);
      } else if constexpr (r >= 28) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = 2 * (r - 28) + u;
          a[i] = *reinterpret_cast<const uint4 *>(nx + aoff[0] + i * 32 * AROW);
        }
      }
      if constexpr (r % 2 == 0 && r <= 14) issue_y1(rsl, s + 2, ld, r / 2);
      if constexpr (r == 0) {
        ahn = ahat_at(s + 1, cn, 0);
        lut_quarter<FP4>(ahn, 0, t);
        lut_quarter<FP4>(ahn, 1, t);
      }
      if constexpr (r == 1) {
        lut_quarter<FP4>(ahn, 2, t);
        lut_quarter<FP4>(ahn, 3, t);
      }
      if constexpr (!BS32 && r >= 2 && r <= 25) {
        const int c = (r - 2) / 3, ph = (r - 2) % 3;
        dequant_word(wd[c], t, st + 4 * c, ph, sa, sb);
      }
      if constexpr (BS32 && r >= 2 && r <= 13) {
        const int c = (r - 2) / 3, ph = (r - 2) % 3;
        dequant_word(wd[c], t, st + 4 * c, ph, sa, sb);
      }
      if constexpr (BS32 && (r == 14 || r == 15)) {
        if constexpr (r == 14) ahn = ahat_at(s + 1, cn, 1);
        lut_quarter<FP4>(ahn, 2 * (r - 14), t);
        lut_quarter<FP4>(ahn, 2 * (r - 14) + 1, t);
      }
      if constexpr (BS32 && r >= 16 && r <= 27) {
        const int c = 4 + (r - 16) / 3, ph = (r - 16) % 3;
        dequant_word(wd[c], t, st + 4 * c, ph, sa, sb);
      }
      if constexpr (r >= 24 && r < 28) {
        // the row two 16-byte chunks per group, after the step's last B reads
#pragma unroll
        for (int c = 2 * (r - 24); c < 2 * (r - 24) + 2; ++c)
          *reinterpret_cast<uint4 *>(bw + lane * BROW_W + (c << 4)) =
              make_uint4(st[4 * c], st[4 * c + 1], st[4 * c + 2], st[4 * c + 3]);
      }
      sched_cut();
    });
  };
  int64_t s = 0;
  for (; s + 3 <= ns; s += 3) {
    step(s, as0, as1, as2, cs1, cs0);
    step(s + 1, as1, as2, as0, cs2, cs1);
    step(s + 2, as2, as0, as1, cs0, cs2);
  }
  if (s < ns) step(s, as0, as1, as2, cs1, cs0);
  if (s + 1 < ns) step(s + 1, as1, as2, as0, cs2, cs1);
  __builtin_amdgcn_s_waitcnt(0);
  if (LR) {
    const int64_t col[2] = {kc + bcol, kc + 32 + bcol};
    // ranks in chunks of 48 (256 staged rows of 112 bytes in the first dY stage)
    add_lowrank_wide<48>(acc, lr, m0, M, col, bl, kg, as0);
  }

  // epilogue: lane l, register r of a 32x32 tile holds row 8(r/4)+4(l/32)+r%4, column l%32
  if (m0 + TM <= M && k0 + TK <= K && K < ((int64_t)1 << 27)) {
    constexpr int ES = DX_BF16 ? 2 : 4;
    const uint32_t voff = (uint32_t)((4 * kg) * (uint32_t)K + bcol) * ES;
    uint8_t *xcol = reinterpret_cast<uint8_t *>(dX) + (m0 * K + kcol) * ES;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          uint8_t *rowp = xcol + (int64_t)(32 * i + 8 * (r / 4) + (r % 4)) * K * ES + 32 * c * ES;
          if (DX_BF16)
            *reinterpret_cast<uint16_t *>(rowp + voff) = (uint16_t)(pack_bf16x2(acc[i][c][r], 0.f) & 0xffffu);
          else
            *reinterpret_cast<float *>(rowp + voff) = acc[i][c][r];
        }
      }
    }
  } else if (kcol < K) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + 32 * i + 8 * (r / 4) + 4 * kg + (r % 4);
          if (row < M) {
            const int64_t off = row * K + kcol + 32 * c + bcol;
            if (DX_BF16)
              reinterpret_cast<uint16_t *>(dX)[off] = (uint16_t)(pack_bf16x2(acc[i][c][r], 0.f) & 0xffffu);
            else
              reinterpret_cast<float *>(dX)[off] = acc[i][c][r];
          }
        }
      }
    }
  }
}
}  // namespace tr_kernel

// ------------------------------------------------------------ small-M kernel
//
// For at most 16 rows of dY the 256x256 kernels above would leave 15/16 of
// every MFMA idle and launch one workgroup per 256 output columns; here the
// work is the weight stream.  Workgroup b owns a band of CW output columns
// (CW = 32, or 64 when there are enough bands to fill the chip) over all N
// rows of the reduction, and grid row y the dY rows 16y .. 16y + 15 (more
// rows than 16: the weight is streamed once per grid row); bands that share a
// 128-byte line of codes run on one XCD.  The 16 waves (four per SIMD) take
// steps of 64 weight rows in turn (wave w: steps w, w + 16, ...).  In a step
// lane l dequantizes row 64s + l of the band -- one table per row (two at
// block size 32 with CW = 64) -- and writes the CW bf16 values as one row of
// the wave's own LDS tile; the transposing read ds_read_b64_tr_b16 then hands
// each lane eight consecutive rows of one column (within a 16-lane group,
// output lane i element e is element i%4 of the 8 bytes addressed by lane
// 4e + i/4), the B operand of MFMA 16x16x32 whose A operand is dY (lane l:
// row l%16, the same eight reduction indices 8(l/16) .. +7 of a 32-row half).
// Rows of dY past M and reduction indices past N load zeros (buffer
// descriptor), so the weight rows past N (read clamped to the last row) add
// exact zeros.  The next step's codes, absmax state and dY fragments are
// loaded before the current step is dequantized.  At the end the 16 waves'
// partial sums meet in LDS and each thread adds one output element's 16 parts
// in wave order (deterministic, and no workspace).
namespace small {

constexpr int SW = 16;                  // waves per workgroup, four per SIMD
constexpr int SR = 64;                  // weight rows per wave step, one per lane
constexpr int kMaxRows = 16;            // rows of dY per grid row (the MFMA's 16 A rows)
constexpr int kMaxGridRows = 16;        // grid rows considered (M up to 256, one M tile of the 256x256 kernel)
// Measured time of one round of up to 256 workgroups per 4096 weight rows, in
// tenths of a microsecond, for a band width (64 or 32 columns), or for the
// 256x256 kernel (0: one round of its K/256 tiles).  16-column bands took 15 us
// a round, more than 32-column bands at every shape, and are not used.
constexpr int64_t band_cost(int cw) { return cw == 64 ? 165 : cw == 32 ? 140 : 950; }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// CW output columns per workgroup (32 or 64): a lane's CW codes of one weight
// row lie in one block, or in two at block size 32 with CW = 64 (BS32).
template <int CW, bool BS32>
struct StepIn {
  uint4 c[CW / 32];        // the lane's CW codes
  ChunkAbsmax<BS32> ab;    // their block's absmax state
  uint4 a[2];              // dY fragments of the two 32-row halves
};

template <int CW, bool DQ, bool BS32, bool FP4, bool LR>
__global__ __launch_bounds__(64 * SW) void bwd_dx_small_kernel(const uint16_t *__restrict__ dY, int M, int64_t N,
                                                               int64_t K, const uint8_t *__restrict__ packed,
                                                               AbsmaxSrc src, LowRank lr, void *__restrict__ dX,
                                                               int dx_bf16) {
  static_assert(CW == 32 || CW == 64, "32 or 64 columns per workgroup");
  static_assert(!BS32 || CW == 64, "a 32-column chunk lies in one block at every block size");
  constexpr int NJ = CW / 16;           // MFMA column groups
  constexpr int SROW = 2 * CW + 16;     // LDS tile row: CW bf16 + 16 bytes of padding
  constexpr int STILE = SR * SROW;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[SW * STILE > SW * NJ * 64 * 16 ? SW * STILE : SW * NJ * 64 * 16];
  {
    // more than 16 rows: grid row y takes rows 16y .. 16y + 15 of dY (and of V and dX)
    const int m0 = kMaxRows * (int)blockIdx.y;
    dY += (int64_t)m0 * N;
    lr.u += (int64_t)m0 * lr.r;
    dX = reinterpret_cast<uint8_t *>(dX) + (int64_t)m0 * K * (dx_bf16 ? 2 : 4);
    M = M - m0 < kMaxRows ? M - m0 : kMaxRows;
  }
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;
  // bands sharing a 128-byte line of codes go to workgroups of one XCD
  // (consecutive workgroups are dealt to the eight XCDs in turn)
  int band = blockIdx.x;
  {
    const int nb = gridDim.x, q = nb / 8, r = nb % 8, x = band % 8, i = band / 8;
    band = x * q + (x < r ? x : r) + i;
  }
  const uint32_t k0 = (uint32_t)band * CW;
  const float mu = DQ ? *src.mean : 0.f;
  uint8_t *tile = tiles + wave * STILE;
  // 32-bit offsets throughout (the launcher keeps N K below 2^32 and K below
  // 2^24, so row offsets are 24-bit products).  Codes from the workgroup's
  // column band on; dY [M, N] (at most 16 x 2^24 elements): lanes whose row
  // lies past M, and reduction indices past N, get offsets beyond the
  // descriptor (zeros).
  const uint32_t rowb = (uint32_t)(K / 2), Nu = (uint32_t)N, Ku = (uint32_t)K;
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(packed + k0 / 2), (short)0, (int)(Nu * rowb - k0 / 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(dY), (short)0,
                                                                       (int)((uint32_t)M * Nu * 2u), 0x00020000);
  const uint32_t yrow = col < M ? (uint32_t)col * Nu * 2u : 0x80000000u;
  const int nsteps = (int)((N + SR - 1) / SR);

  auto load_step = [&](int s, StepIn<CW, BS32> &in) {
    s = s < nsteps ? s : nsteps - 1;   // past the last step: a repeat, never used
    const uint32_t n = (uint32_t)s * SR + (uint32_t)lane;
    const uint32_t nc = n < Nu ? n : Nu - 1;
    const uint32_t co = __umul24(nc, rowb);
#pragma unroll
    for (int u = 0; u < CW / 32; ++u)
      in.c[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(crs, co + 16u * u, 0, 0));
    in.ab.template load<DQ>(src, (int64_t)((__umul24(nc, Ku) + k0) >> src.lbs));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t na = (uint32_t)s * SR + 32u * h + 8u * kg;   // N % 8 == 0: all eight indices in or out
      const uint32_t off = na < Nu ? yrow + na * 2u : 0x80000000u;
      in.a[h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(yrs, off, 0, 0));
    }
  };

  f32x4 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const StepIn<CW, BS32> &in) {
    const Lut t0 = make_lut<FP4>(in.ab.ahat(0, DQ, mu));
    Lut t1;
    if (BS32) t1 = make_lut<FP4>(in.ab.ahat(1, DQ, mu));
    uint4 row[CW / 8];
#pragma unroll
    for (int j = 0; j < CW / 8; ++j) {
      const uint4 &cw = in.c[j / 4];
      const uint32_t word = (j % 4 == 0) ? cw.x : (j % 4 == 1) ? cw.y : (j % 4 == 2) ? cw.z : cw.w;
      const Lut &tj = (BS32 && j >= 4) ? t1 : t0;
      Sel4 sa, sb;
      select8(word, sa, sb);
      lookup4(sa, tj, row[j].x, row[j].y);
      lookup4(sb, tj, row[j].z, row[j].w);
    }
    // the previous step's reads of the tile have returned before it is rewritten,
    // and the new row is in place before any lane reads it transposed
    __builtin_amdgcn_s_waitcnt(lgkm_imm(0));
#pragma unroll
    for (int j = 0; j < CW / 8; ++j) *reinterpret_cast<uint4 *>(tile + lane * SROW + 16 * j) = row[j];
    __builtin_amdgcn_s_waitcnt(lgkm_imm(0));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        // lane 4e + q of the group addresses row 32h + 8kg + e (+4) and columns 16j + 4q .. +3
        const uint8_t *a = tile + (32 * h + 8 * kg + (col >> 2)) * SROW + (16 * j + 4 * (col & 3)) * 2;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)a);
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(a + 4 * SROW));
        const v4s b8[2] = {lo, hi};
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(in.a[h]), __builtin_bit_cast(bf16x8, b8),
                                                         acc[j], 0, 0, 0);
      }
    }
  };

  StepIn<CW, BS32> A, B;
  load_step(wave, A);
  for (int s = wave; s < nsteps; s += 2 * SW) {
    load_step(s + SW, B);
    process(A);
    load_step(s + 2 * SW, A);
    if (s + SW < nsteps) process(B);
  }

  if (LR) {
    // adapter term V A^T (lr.u = V [M, r], lr.v = A^T [K, r]): rank slices of 32
    // dealt to the waves; lane group kg takes ranks 32s + 8kg .. +7 (zeros past r)
    for (int s = wave; 32 * s < lr.r; s += SW) {
      const int rk = 32 * s + 8 * kg;
      uint4 av = make_uint4(0u, 0u, 0u, 0u);
      if (rk < lr.r && col < M) av = *reinterpret_cast<const uint4 *>(lr.u + (int64_t)col * lr.r + rk);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        uint4 bv = make_uint4(0u, 0u, 0u, 0u);
        if (rk < lr.r) bv = *reinterpret_cast<const uint4 *>(lr.v + (int64_t)(k0 + 16 * j + col) * lr.r + rk);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(bv), acc[j], 0, 0, 0);
      }
    }
  }

  // the waves' parts through LDS (the tiles are free once every wave is here):
  // part (w, j) of lane l at f32x4 index (NJ w + j) * 64 + l
  __syncthreads();
  f32x4 *red = reinterpret_cast<f32x4 *>(tiles);
#pragma unroll
  for (int j = 0; j < NJ; ++j) red[(NJ * wave + j) * 64 + lane] = acc[j];
  __syncthreads();
  // thread t < 256 NJ: lane l = t % 64, column group j = (t / 64) % NJ, register
  // i = t / (64 NJ); element (row 4(l/16) + i, column k0 + 16j + l%16)
  if (threadIdx.x < 256 * NJ) {
    const int l = threadIdx.x & 63, j = (threadIdx.x >> 6) % NJ, i = (threadIdx.x >> 6) / NJ;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < SW; ++w) sum += red[(NJ * w + j) * 64 + l][i];
    const int m = 4 * (l >> 4) + i;
    if (m < M) {
      const int64_t off = (int64_t)m * K + (int64_t)(k0 + 16 * j + (l & 15));
      if (dx_bf16)
        reinterpret_cast<uint16_t *>(dX)[off] = (uint16_t)(pack_bf16x2(sum, 0.f) & 0xffffu);
      else
        reinterpret_cast<float *>(dX)[off] = sum;
    }
  }
}

}  // namespace small

}  // namespace

hipError_t launch_bwd_dx(const void *dy, int64_t M, int64_t N, int64_t K, const uint8_t *packed,
                         const AbsmaxSrc &src, const LowRank &lr, void *dx, int dx_is_bf16,
                         hipStream_t stream) {
  const uint16_t *dY = reinterpret_cast<const uint16_t *>(dy);
  const bool has_lr = lr.r > 0;
  const bool small_fits = M >= 1 && M <= small::kMaxGridRows * small::kMaxRows && N > 0 && N % 8 == 0 &&
                          N < ((int64_t)1 << 24) && K < ((int64_t)1 << 24) && N * K < ((int64_t)1 << 32);
  // Band width: the one with the least estimated time, rounds of 256 workgroups
  // times the per-round cost (a partly filled round costs about a full one).
  const int64_t grid_rows = (M + small::kMaxRows - 1) / small::kMaxRows;
  int cw = 64;
  int64_t est = 0;
  for (const int c : {64, 32}) {
    const int64_t e = ((K / c) * grid_rows + 255) / 256 * small::band_cost(c);
    if (c == 64 || e < est) {
      cw = c;
      est = e;
    }
  }
  bool use_small = small_fits && M <= small::kMaxRows;
  if (small_fits && !use_small) {
    // more rows: each grid row of 16 re-streams the weight
    const int64_t rounds_wide = ((K + 255) / 256 + 255) / 256;
    use_small = est <= rounds_wide * small::band_cost(0);
  }
  if (use_small) {
    // the weight stream, one workgroup per band of 32 or 64 output columns and grid row
    using namespace small;
    using K_t = void (*)(const uint16_t *, int, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *, int);
#define NF4_BWDS(CW, DQ, BS32, FP4) {bwd_dx_small_kernel<CW, DQ, BS32, FP4, false>, bwd_dx_small_kernel<CW, DQ, BS32, FP4, true>}
    static const K_t kern64[2][2][2][2] = {{{NF4_BWDS(64, false, false, false), NF4_BWDS(64, false, false, true)},
                                            {NF4_BWDS(64, false, true, false), NF4_BWDS(64, false, true, true)}},
                                           {{NF4_BWDS(64, true, false, false), NF4_BWDS(64, true, false, true)},
                                            {NF4_BWDS(64, true, true, false), NF4_BWDS(64, true, true, true)}}};
    static const K_t kern32[2][2][2] = {{NF4_BWDS(32, false, false, false), NF4_BWDS(32, false, false, true)},
                                        {NF4_BWDS(32, true, false, false), NF4_BWDS(32, true, false, true)}};
#undef NF4_BWDS
    const K_t f = cw == 64 ? kern64[src.dq ? 1 : 0][src.lbs == 5 ? 1 : 0][src.qt ? 1 : 0][has_lr ? 1 : 0]
                           : kern32[src.dq ? 1 : 0][src.qt ? 1 : 0][has_lr ? 1 : 0];
    hipLaunchKernelGGL(f, dim3((unsigned)(K / cw), (unsigned)((M + kMaxRows - 1) / kMaxRows)), dim3(64 * SW), 0,
                       stream, dY, (int)M, N, K, packed, src, lr, dx, dx_is_bf16);
  } else if (N % 8 == 0 && N < ((int64_t)1 << 24)) {
    // 16-byte dY rows: buffer-to-LDS dY tiles, transposing weight reads, one wave per SIMD
    using namespace tr_kernel;
    using K_t = void (*)(const uint16_t *, int64_t, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *,
                         int, int);
#define NF4_BWD(XB, DQ, FP4) {{bwd_dx_wide_kernel<XB, DQ, FP4, false, false>, bwd_dx_wide_kernel<XB, DQ, FP4, false, true>}, \
                              {bwd_dx_wide_kernel<XB, DQ, FP4, true, false>, bwd_dx_wide_kernel<XB, DQ, FP4, true, true>}}
    static const K_t kern[2][2][2][2][2] = {{{NF4_BWD(false, false, false), NF4_BWD(false, false, true)},
                                             {NF4_BWD(false, true, false), NF4_BWD(false, true, true)}},
                                            {{NF4_BWD(true, false, false), NF4_BWD(true, false, true)},
                                             {NF4_BWD(true, true, false), NF4_BWD(true, true, true)}}};
#undef NF4_BWD
    const int tiles_m = (int)((M + TM - 1) / TM), tiles_k = (int)((K + TK - 1) / TK);
    hipLaunchKernelGGL(kern[dx_is_bf16 ? 1 : 0][src.dq ? 1 : 0][src.qt ? 1 : 0][src.lbs == 5 ? 1 : 0][has_lr ? 1 : 0],
                       dim3((unsigned)(tiles_m * tiles_k)), dim3(64 * NWAVE_W), 0, stream, dY, M, N, K, packed, src,
                       lr, dx, tiles_m, tiles_k);
  } else {
    using namespace generic;
    using K_t = void (*)(const uint16_t *, int64_t, int64_t, int64_t, const uint8_t *, AbsmaxSrc, LowRank, void *,
                         int, int);
    static const K_t kern[2][4] = {
        {bwd_dx_generic_kernel<false, false, false>, bwd_dx_generic_kernel<false, true, false>,
         bwd_dx_generic_kernel<true, false, false>, bwd_dx_generic_kernel<true, true, false>},
        {bwd_dx_generic_kernel<false, false, true>, bwd_dx_generic_kernel<false, true, true>,
         bwd_dx_generic_kernel<true, false, true>, bwd_dx_generic_kernel<true, true, true>}};
    const int sel = (dx_is_bf16 ? 2 : 0) | (has_lr ? 1 : 0);
    const int tiles_m = (int)((M + TM - 1) / TM), tiles_k = (int)((K + TK - 1) / TK);
    const dim3 g((unsigned)(tiles_m * tiles_k)), b(256);
    hipLaunchKernelGGL(kern[src.qt ? 1 : 0][sel], g, b, 0, stream, dY, M, N, K, packed, src, lr, dx, tiles_m, tiles_k);
  }
  return hipGetLastError();
}

}  // namespace nf4
