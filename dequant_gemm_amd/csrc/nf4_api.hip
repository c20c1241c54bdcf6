// nf4_api.hip -- the C ABI declared in include/nf4.h: argument validation,
// buffer-size arithmetic and kernel dispatch.  Validation touches no HIP API,
// so every error path can be exercised on a machine without a GPU.
#include <mutex>

#include "nf4.h"
#include "nf4_launch.h"

namespace {

constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_dtype(int d) { return d == NF4_F32 || d == NF4_BF16; }

int check_shape(int64_t rows, int64_t cols) {
  if (rows < 1 || cols < 1 || rows > kMaxDim || cols > kMaxDim) return NF4_ERR_SHAPE;
  if (rows > NF4_MAX_NUMEL / cols) return NF4_ERR_SHAPE;
  return NF4_OK;
}

bool valid_blocksize(int bs) {
  return bs >= NF4_BLOCKSIZE_MIN && bs <= NF4_BLOCKSIZE_MAX && (bs & (bs - 1)) == 0;
}
int log2_of(int bs) { return 31 - __builtin_clz((unsigned)bs); }
int64_t nblocks_of(int64_t numel, int bs) { return (numel + bs - 1) / bs; }
int64_t ngroups_of(int64_t nblocks) { return (nblocks + NF4_DQ_GROUP - 1) / NF4_DQ_GROUP; }

// Checks a quantized tensor descriptor and its buffers.
int check_qtensor(const nf4_qtensor *q) {
  if (!q) return NF4_ERR_NULL;
  if (!valid_blocksize(q->blocksize)) return NF4_ERR_BLOCKSIZE;
  int st = check_shape(q->rows, q->cols);
  if (st) return st;
  if (q->double_quant != 0 && q->double_quant != 1) return NF4_ERR_UNSUPPORTED;
  if (q->quant_type != NF4_QT_NF4 && q->quant_type != NF4_QT_FP4) return NF4_ERR_QUANT_TYPE;
  if (!q->packed) return NF4_ERR_NULL;
  if (!aligned16(q->packed)) return NF4_ERR_ALIGN;
  if (q->double_quant) {
    if (!q->absmax_q || !q->absmax_scale || !q->absmax_mean) return NF4_ERR_NULL;
    if (!aligned16(q->absmax_q) || !aligned16(q->absmax_scale) || !aligned16(q->absmax_mean))
      return NF4_ERR_ALIGN;
  } else {
    if (!q->absmax) return NF4_ERR_NULL;
    if (!aligned16(q->absmax)) return NF4_ERR_ALIGN;
  }
  return NF4_OK;
}

nf4::AbsmaxSrc absmax_src(const nf4_qtensor *q) {
  nf4::AbsmaxSrc s;
  s.absmax = q->absmax;
  s.q = q->absmax_q;
  s.scale = q->absmax_scale;
  s.mean = q->absmax_mean;
  s.dq = q->double_quant;
  s.lbs = log2_of(q->blocksize);
  s.qt = q->quant_type == NF4_QT_FP4 ? 1 : 0;
  return s;
}

int hip_status(hipError_t e) { return e == hipSuccess ? NF4_OK : NF4_ERR_HIP; }

// Argument checks shared by both quantize entry points (no HIP call).
int check_quantize(const void *W, int w_dtype, int64_t rows, int64_t cols, int blocksize, int double_quant,
                   const nf4_qtensor *out, const uint32_t *d_status) {
  if (!valid_blocksize(blocksize)) return NF4_ERR_BLOCKSIZE;
  if (!W || !out) return NF4_ERR_NULL;
  if (!valid_dtype(w_dtype)) return NF4_ERR_DTYPE;
  int st = check_shape(rows, cols);
  if (st) return st;
  if (double_quant != 0 && double_quant != 1) return NF4_ERR_UNSUPPORTED;
  if (!aligned16(W)) return NF4_ERR_ALIGN;
  st = check_qtensor(out);
  if (st) return st;
  if (out->rows != rows || out->cols != cols || out->double_quant != double_quant ||
      out->blocksize != blocksize)
    return NF4_ERR_SHAPE;
  if (d_status && !aligned16(d_status)) return NF4_ERR_ALIGN;
  return NF4_OK;
}

// Queues the quantization of checked arguments; `ws` holds at least
// quant_workspace_bytes(nblocks) bytes when double_quant is set.
int launch_quantize_into(const void *W, int w_dtype, int64_t rows, int64_t cols, int blocksize, int double_quant,
                         const nf4_qtensor *out, void *ws, uint32_t *d_status, void *stream) {
  unsigned long long *partials = nullptr;
  float *absmax = out->absmax;
  if (double_quant) {
    partials = reinterpret_cast<unsigned long long *>(ws);
    absmax = reinterpret_cast<float *>(reinterpret_cast<uint8_t *>(ws) + nf4::absmax_ws_offset());
  }
  return hip_status(nf4::launch_quantize(W, w_dtype == NF4_BF16, rows * cols, log2_of(blocksize),
                                         out->quant_type == NF4_QT_FP4, out->packed, absmax,
                                         partials, d_status, double_quant, out->absmax_q,
                                         out->absmax_scale, out->absmax_mean,
                                         reinterpret_cast<hipStream_t>(stream)));
}

// ---------------------------------------------------------------- fixed scratch
//
// nf4_quantize_noalloc's scratch: the same layout as nf4_quantize's workspace
// (exact-mean rows, then the fp32 absmax of every block), sized for
// NF4_NOALLOC_MAX_BLOCKS blocks.  One copy per GPU, kept for the life of the
// process and shared by every call on that GPU.  In host code `scratch` names
// a host-side stand-in, never the device memory: the device address is taken
// once per device with hipGetSymbolAddress and only that address is passed on.
constexpr size_t kScratchBytes = nf4::quant_workspace_bytes(NF4_NOALLOC_MAX_BLOCKS);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once taken

// The current device's address of `scratch`, looked up on the first call on
// that device (with that device current) and cached.
hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char *nf4_status_string(int status) {
  switch (status) {
    case NF4_OK: return "ok";
    case NF4_ERR_NULL: return "a required pointer is NULL";
    case NF4_ERR_SHAPE: return "a size is out of range or does not match";
    case NF4_ERR_BLOCKSIZE: return "blocksize must be 32, 64, 128 or 256";
    case NF4_ERR_DTYPE: return "unknown dtype";
    case NF4_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case NF4_ERR_WORKSPACE: return "workspace too small";
    case NF4_ERR_UNSUPPORTED: return "unsupported (e.g. GEMM needs cols % 64 == 0)";
    case NF4_ERR_HIP: return "HIP launch failed";
    case NF4_ERR_QUANT_TYPE: return "quant_type must be NF4_QT_NF4 or NF4_QT_FP4";
    case NF4_ERR_SCRATCH: return "more blocks than nf4_quantize_noalloc's fixed scratch holds (NF4_NOALLOC_MAX_BLOCKS)";
    default: return "unknown status";
  }
}

int nf4_codebook(float *levels16) {
  if (!levels16) return NF4_ERR_NULL;
  for (int i = 0; i < 16; ++i) levels16[i] = nf4::level(i);
  return NF4_OK;
}

int nf4_levels(int quant_type, float *levels16) {
  if (!levels16) return NF4_ERR_NULL;
  if (quant_type != NF4_QT_NF4 && quant_type != NF4_QT_FP4) return NF4_ERR_QUANT_TYPE;
  for (int i = 0; i < 16; ++i) levels16[i] = quant_type == NF4_QT_FP4 ? nf4::fp4_level(i) : nf4::level(i);
  return NF4_OK;
}

int nf4_thresholds(float *thresholds15) {
  if (!thresholds15) return NF4_ERR_NULL;
  for (int i = 0; i < 15; ++i) thresholds15[i] = nf4::threshold(i);
  return NF4_OK;
}

int nf4_sizes(int64_t rows, int64_t cols, int blocksize, int double_quant, int64_t *packed_bytes,
              int64_t *nblocks, int64_t *ngroups, size_t *workspace_bytes) {
  if (!valid_blocksize(blocksize)) return NF4_ERR_BLOCKSIZE;
  int st = check_shape(rows, cols);
  if (st) return st;
  if (double_quant != 0 && double_quant != 1) return NF4_ERR_UNSUPPORTED;
  const int64_t numel = rows * cols;
  const int64_t nb = nblocks_of(numel, blocksize);
  if (packed_bytes) *packed_bytes = (numel + 1) / 2;
  if (nblocks) *nblocks = nb;
  if (ngroups) *ngroups = ngroups_of(nb);
  if (workspace_bytes) *workspace_bytes = double_quant ? nf4::quant_workspace_bytes(nb) : 0;
  return NF4_OK;
}

int nf4_quantize(const void *W, int w_dtype, int64_t rows, int64_t cols, int blocksize,
                 int double_quant, const nf4_qtensor *out, void *workspace, size_t workspace_bytes,
                 uint32_t *d_status, void *stream) {
  int st = check_quantize(W, w_dtype, rows, cols, blocksize, double_quant, out, d_status);
  if (st) return st;
  const int64_t nb = nblocks_of(rows * cols, blocksize);
  if (double_quant) {
    if (workspace_bytes < nf4::quant_workspace_bytes(nb)) return NF4_ERR_WORKSPACE;
    if (!workspace) return NF4_ERR_NULL;
    if (!aligned16(workspace)) return NF4_ERR_ALIGN;
  }
  return launch_quantize_into(W, w_dtype, rows, cols, blocksize, double_quant, out, workspace, d_status, stream);
}

int nf4_quantize_noalloc(const void *W, int w_dtype, int64_t rows, int64_t cols, int blocksize,
                         int double_quant, const nf4_qtensor *out, uint32_t *d_status, void *stream) {
  int st = check_quantize(W, w_dtype, rows, cols, blocksize, double_quant, out, d_status);
  if (st) return st;
  if (!double_quant)   // without double quantization the kernels use no scratch at all
    return launch_quantize_into(W, w_dtype, rows, cols, blocksize, 0, out, nullptr, d_status, stream);
  if (nblocks_of(rows * cols, blocksize) > NF4_NOALLOC_MAX_BLOCKS) return NF4_ERR_SCRATCH;
  void *ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return NF4_ERR_HIP;
  return launch_quantize_into(W, w_dtype, rows, cols, blocksize, 1, out, ws, d_status, stream);
}

int nf4_dequantize(const nf4_qtensor *q, void *out, int out_dtype, void *stream) {
  int st = check_qtensor(q);
  if (st) return st;
  if (!out) return NF4_ERR_NULL;
  if (!valid_dtype(out_dtype)) return NF4_ERR_DTYPE;
  if (!aligned16(out)) return NF4_ERR_ALIGN;
  return hip_status(nf4::launch_dequantize(q->packed, absmax_src(q), q->rows * q->cols, out,
                                           out_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

static int check_gemm(const void *A, int64_t M, const nf4_qtensor *q, void *C, int c_dtype) {
  int st = check_qtensor(q);
  if (st) return st;
  if (M < 0 || M > kMaxDim) return NF4_ERR_SHAPE;
  if (!valid_dtype(c_dtype)) return NF4_ERR_DTYPE;
  if (q->cols % NF4_BLOCKSIZE != 0 || q->cols >= NF4_GEMM_COLS_LIMIT) return NF4_ERR_UNSUPPORTED;
  if (M == 0) return NF4_OK;
  if (!A || !C) return NF4_ERR_NULL;
  if (!aligned16(A) || !aligned16(C)) return NF4_ERR_ALIGN;
  return NF4_OK;
}

static int check_lowrank(int64_t M, const void *U, const void *V, int64_t r) {
  if (r < NF4_LORA_RANK_STEP || r > NF4_LORA_MAX_RANK || r % NF4_LORA_RANK_STEP != 0) return NF4_ERR_UNSUPPORTED;
  if (M == 0) return NF4_OK;
  if (!U || !V) return NF4_ERR_NULL;
  if (!aligned16(U) || !aligned16(V)) return NF4_ERR_ALIGN;
  return NF4_OK;
}

static const nf4::LowRank kNoLowRank = {nullptr, nullptr, 0};

int nf4_matmul_fwd(const void *X, int64_t M, const nf4_qtensor *q, void *Y, int y_dtype, void *stream) {
  int st = check_gemm(X, M, q, Y, y_dtype);
  if (st || M == 0) return st;
  return hip_status(nf4::launch_fwd(X, M, q->rows, q->cols, q->packed, absmax_src(q), kNoLowRank, Y,
                                    y_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

int nf4_matmul_bwd_dx(const void *dY, int64_t M, const nf4_qtensor *q, void *dX, int dx_dtype,
                      void *stream) {
  int st = check_gemm(dY, M, q, dX, dx_dtype);
  if (st || M == 0) return st;
  return hip_status(nf4::launch_bwd_dx(dY, M, q->rows, q->cols, q->packed, absmax_src(q), kNoLowRank, dX,
                                       dx_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

int nf4_matmul_fwd_lora(const void *X, int64_t M, const nf4_qtensor *q, const void *U, const void *B,
                        int64_t r, void *Y, int y_dtype, void *stream) {
  int st = check_gemm(X, M, q, Y, y_dtype);
  if (st) return st;
  st = check_lowrank(M, U, B, r);
  if (st || M == 0) return st;
  const nf4::LowRank lr = {reinterpret_cast<const uint16_t *>(U), reinterpret_cast<const uint16_t *>(B), (int)r};
  return hip_status(nf4::launch_fwd(X, M, q->rows, q->cols, q->packed, absmax_src(q), lr, Y,
                                    y_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

int nf4_matmul_bwd_dx_lora(const void *dY, int64_t M, const nf4_qtensor *q, const void *V, const void *At,
                           int64_t r, void *dX, int dx_dtype, void *stream) {
  int st = check_gemm(dY, M, q, dX, dx_dtype);
  if (st) return st;
  st = check_lowrank(M, V, At, r);
  if (st || M == 0) return st;
  const nf4::LowRank lr = {reinterpret_cast<const uint16_t *>(V), reinterpret_cast<const uint16_t *>(At), (int)r};
  return hip_status(nf4::launch_bwd_dx(dY, M, q->rows, q->cols, q->packed, absmax_src(q), lr, dX,
                                       dx_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

int nf4_adapter_matmul(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K, float alpha, const void *A,
                       int64_t lda, const void *B, int64_t ldb, void *C, int c_dtype, int64_t ldc, void *stream) {
  if ((trans_a != 0 && trans_a != 1) || (trans_b != 0 && trans_b != 1)) return NF4_ERR_UNSUPPORTED;
  if (M < 0 || N < 0 || K < 1 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return NF4_ERR_SHAPE;
  if (!valid_dtype(c_dtype)) return NF4_ERR_DTYPE;
  // stored shapes: A [M, K] or [K, M]; B [K, N] or [N, K]; rows of `ld` elements
  const int64_t a_rows = trans_a ? K : M, a_cols = trans_a ? M : K;
  const int64_t b_rows = trans_b ? N : K, b_cols = trans_b ? K : N;
  if (lda < a_cols || ldb < b_cols || ldc < N || lda < 1 || ldb < 1 || ldc < 1) return NF4_ERR_SHAPE;
  if (M == 0 || N == 0) return NF4_OK;
  if (!A || !B || !C) return NF4_ERR_NULL;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return NF4_ERR_ALIGN;
  const int64_t lim = ((int64_t)1 << 31) / 2;   // 32-bit byte offsets into each stored operand
  if (a_rows > lim / lda || b_rows > lim / ldb) return NF4_ERR_UNSUPPORTED;
  if (((M + 63) / 64) * ((N + 63) / 64) > kMaxDim) return NF4_ERR_UNSUPPORTED;
  const bool va = a_cols % 8 == 0 && lda % 8 == 0;   // 16-byte loads of whole rows
  const bool vb = b_cols % 8 == 0 && ldb % 8 == 0;
  return hip_status(nf4::launch_adapter_gemm(trans_a, trans_b, M, N, K, alpha, A, lda, va, B, ldb, vb, C, ldc,
                                             c_dtype == NF4_BF16, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
