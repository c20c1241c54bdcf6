// adapter.hip -- the dense bf16 products of a low-rank adapter on a frozen
// 4-bit weight ("bitsandbytes" page, 4-bit/LoRA paragraph: a frozen 4-bit
// base weight with small trainable adapters).  For an adapter with down
// projection A [r, K] and up projection B [N, r] on input X [M, K] and output
// gradient dY [M, N] (scale s):
//   U  = s X A^T      [M, r]   (the forward's adapter activation)
//   V  = s dY B       [M, r]   (the input gradient's adapter activation)
//   dA = V^T X        [r, K]   (gradient of A)
//   dB = dY^T U       [N, r]   (gradient of B)
// All four are C = alpha op(A) op(B) with op the identity or the transpose:
// bf16 operands, fp32 accumulation on the bf16 matrix cores, fp32 output or
// one round-to-nearest-even bf16 rounding of it.
//
// Workgroup tile 64 x 64 outputs, four waves (2 x 2), each 32 x 32 with MFMA
// 32x32x16; reduction steps of 64.  Each operand tile reaches LDS in the
// layout it has in memory (double buffered, 16-byte loads where the rows
// allow); a fragment whose reduction index runs along an LDS row is one
// 16-byte read, one whose reduction index runs down the rows comes from two
// gfx950 transposing reads (ds_read_b64_tr_b16).  Reads outside the matrices
// return zeros through buffer descriptors.
#include "nf4_launch.h"

namespace nf4 {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int AT = 64;          // output tile rows and columns
constexpr int KT = 64;          // reduction step
constexpr int ROW_K = KT * 2 + 16;   // LDS row of 64 reduction elements (+16 bytes against bank conflicts)
constexpr int ROW_T = AT * 2 + 32;   // LDS row of 64 output-index elements (+32 bytes)
constexpr int STAGE = (ROW_K * AT > ROW_T * KT ? ROW_K * AT : ROW_T * KT);

// One operand's 64 x 64 tile: `T` false -- stored [idx][k] (k contiguous),
// true -- stored [k][idx].  `VEC`: rows are 16-byte aligned and the
// contiguous extent is a multiple of 8, so 16-byte loads are whole or absent.
struct OperandArgs {
  const void *p;
  int64_t ld;       // elements between rows
  int64_t nidx;     // extent of the output index (M for A, N for B)
  int64_t nk;       // extent of the reduction index
};

template <bool T, bool VEC>
struct Operand {
  __amdgpu_buffer_rsrc_t rs;
  int64_t ld, nidx, nk;

  __device__ __forceinline__ explicit Operand(const OperandArgs &a) : ld(a.ld), nidx(a.nidx), nk(a.nk) {
    const int64_t rows = T ? nk : nidx;   // rows of the stored matrix; its bytes are below 2^31 (checked by the caller)
    rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(a.p), (short)0, (int)(rows * ld * 2), 0x00020000);
  }

  // thread t's two 16-byte pieces of the tile at (idx0, k0)
  __device__ __forceinline__ void load(int64_t idx0, int64_t k0, uint4 v[2]) const {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = threadIdx.x + 256 * p;                    // 512 pieces of 8 elements
      const int row = c >> 3, ch = c & 7;
      // T: row = k offset, 8 elements along idx; else row = idx offset, 8 along k
      const int64_t r = T ? k0 + row : idx0 + row;
      const int64_t e0 = T ? idx0 + 8 * ch : k0 + 8 * ch;
      const int64_t rows = T ? nk : nidx, cols = T ? nidx : nk;
      if (VEC) {
        const bool ok = r < rows && e0 < cols;
        const uint32_t off = ok ? (uint32_t)((r * ld + e0) * 2) : 0x80000000u;
        v[p] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
      } else {
        uint32_t w[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          uint32_t lo = 0, hi = 0;
          const int64_t ea = e0 + 2 * h, eb = ea + 1;
          if (r < rows && ea < cols) lo = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)((r * ld + ea) * 2), 0, 0);
          if (r < rows && eb < cols) hi = __builtin_amdgcn_raw_buffer_load_b16(rs, (uint32_t)((r * ld + eb) * 2), 0, 0);
          w[h] = lo | (hi << 16);
        }
        v[p] = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
  }

  __device__ __forceinline__ void store(uint8_t *lds, const uint4 v[2]) const {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = threadIdx.x + 256 * p;
      const int row = c >> 3, ch = c & 7;
      *reinterpret_cast<uint4 *>(lds + row * (T ? ROW_T : ROW_K) + 16 * ch) = v[p];
    }
  }

  // the MFMA fragment of this lane for output index base ib (0 or 32 in the
  // tile) and reduction half h (elements 16h .. 16h+15 of the step): index
  // ib + l%32, reduction elements 16h + 8(l/32) .. +7
  __device__ __forceinline__ bf16x8 frag(const uint8_t *lds, int ib, int h) const {
    const int l = threadIdx.x & 63;
    if (!T) {
      return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(
                                            lds + (ib + (l & 31)) * ROW_K + (16 * h + 8 * (l >> 5)) * 2));
    }
    // transposing reads: in a 16-lane group G, lane j addresses row kb + j/4,
    // columns ib + 16(G%2) + 4(j%4); lane j then holds rows kb .. kb+3 of
    // column ib + 16(G%2) + j
    const int G = l >> 4, j = l & 15;
    const int col = ib + 16 * (G & 1) + 4 * (j & 3);
    v4s part[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int kb = 16 * h + 8 * (G >> 1) + 4 * q;
      part[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4s *)(lds + (kb + (j >> 2)) * ROW_T + col * 2));
    }
    const uint2 a = __builtin_bit_cast(uint2, part[0]), b = __builtin_bit_cast(uint2, part[1]);
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
  }
};

// LA: A stored [K, M] (op(A) = A^T); LB: B stored [K, N] (op(B) = B).
template <bool LA, bool LB, bool VA, bool VB, bool C_BF16>
__global__ __launch_bounds__(256) void adapter_gemm_kernel(OperandArgs aa, OperandArgs ba, int64_t M, int64_t N,
                                                           int64_t K, float alpha, void *__restrict__ C, int64_t ldc,
                                                           int tiles_n) {
  const Operand<LA, VA> A(aa);
  const Operand<LB, VB> B(ba);
  __shared__ __attribute__((aligned(16))) uint8_t as[2][STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t bs[2][STAGE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)(blockIdx.x / tiles_n) * AT, n0 = (int64_t)(blockIdx.x % tiles_n) * AT;
  const int64_t steps = (K + KT - 1) / KT;

  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  uint4 ra[2], rb[2];
  A.load(m0, 0, ra);
  B.load(n0, 0, rb);
  A.store(as[0], ra);
  B.store(bs[0], rb);
  __syncthreads();
  for (int64_t s = 0; s < steps; ++s) {
    const int cur = (int)(s & 1);
    const bool more = s + 1 < steps;
    if (more) {
      A.load(m0, (s + 1) * KT, ra);
      B.load(n0, (s + 1) * KT, rb);
    }
#pragma unroll
    for (int h = 0; h < KT / 16; ++h)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A.frag(as[cur], 32 * wm, h), B.frag(bs[cur], 32 * wn, h), acc,
                                                    0, 0, 0);
    if (more) {
      A.store(as[cur ^ 1], ra);
      B.store(bs[cur ^ 1], rb);
    }
    __syncthreads();
  }
  // lane l, register r: row 8(r/4) + 4(l/32) + r%4, column l%32 of the wave's 32 x 32
  const int64_t col = n0 + 32 * wn + (lane & 31);
  if (col >= N) return;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = m0 + 32 * wm + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
    if (row < M) {
      const float v = __fmul_rn(alpha, acc[r]);
      if (C_BF16)
        reinterpret_cast<uint16_t *>(C)[row * ldc + col] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xffffu);
      else
        reinterpret_cast<float *>(C)[row * ldc + col] = v;
    }
  }
}

template <bool LA, bool LB, bool VA, bool VB>
void launch4(const void *a, int64_t lda, const void *b, int64_t ldb, int64_t M, int64_t N, int64_t K, float alpha,
             void *c, int64_t ldc, bool c_bf16, hipStream_t stream) {
  const int tiles_m = (int)((M + AT - 1) / AT), tiles_n = (int)((N + AT - 1) / AT);
  const dim3 g((unsigned)(tiles_m * tiles_n)), blk(256);
  const OperandArgs A = {a, lda, M, K}, B = {b, ldb, N, K};
  if (c_bf16)
    hipLaunchKernelGGL((adapter_gemm_kernel<LA, LB, VA, VB, true>), g, blk, 0, stream, A, B, M, N, K, alpha, c, ldc, tiles_n);
  else
    hipLaunchKernelGGL((adapter_gemm_kernel<LA, LB, VA, VB, false>), g, blk, 0, stream, A, B, M, N, K, alpha, c, ldc, tiles_n);
}

template <bool LA, bool LB>
void launch2(const void *a, int64_t lda, bool va, const void *b, int64_t ldb, bool vb, int64_t M, int64_t N, int64_t K,
             float alpha, void *c, int64_t ldc, bool c_bf16, hipStream_t stream) {
  if (va && vb) launch4<LA, LB, true, true>(a, lda, b, ldb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else if (va) launch4<LA, LB, true, false>(a, lda, b, ldb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else if (vb) launch4<LA, LB, false, true>(a, lda, b, ldb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else launch4<LA, LB, false, false>(a, lda, b, ldb, M, N, K, alpha, c, ldc, c_bf16, stream);
}

}  // namespace

// C = alpha op(A) op(B); `ta`: A is stored [K, M]; `tb`: B is stored [N, K];
// `va` / `vb`: the operand allows 16-byte loads (checked by the caller).
hipError_t launch_adapter_gemm(int ta, int tb, int64_t M, int64_t N, int64_t K, float alpha, const void *a,
                               int64_t lda, bool va, const void *b, int64_t ldb, bool vb, void *c, int64_t ldc,
                               bool c_bf16, hipStream_t stream) {
  if (!ta && !tb) launch2<false, true>(a, lda, va, b, ldb, vb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else if (!ta && tb) launch2<false, false>(a, lda, va, b, ldb, vb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else if (ta && !tb) launch2<true, true>(a, lda, va, b, ldb, vb, M, N, K, alpha, c, ldc, c_bf16, stream);
  else launch2<true, false>(a, lda, va, b, ldb, vb, M, N, K, alpha, c, ldc, c_bf16, stream);
  return hipGetLastError();
}

}  // namespace nf4
