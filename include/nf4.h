/*
 * nf4.h -- C ABI of libnf4 (package dequant_gemm_amd): NF4 blockwise weight
 * quantization with double quantization, and the fused NF4-dequant GEMMs,
 * for AMD Instinct MI355X (gfx950).
 *
 * What the calls compute (sources cited by page title and passage):
 *
 *  - "Zenbit" (PyPI project page), section "What's inside", bullet zenbit.nf4:
 *    NF4 blockwise quantization with double quantization of the scale
 *    factors, QLoRA-style.  Bullet zenbit.pallas_nf4: a fused NF4
 *    dequant+matmul whose weight streams compressed and is dequantized on
 *    chip, never materialised at full precision in device memory; a fused
 *    backward that forms dL/dX without materialising the weight, and no dL/dW
 *    (the quantized base weight is frozen).
 *  - "bitsandbytes" (unfragile.ai artifact page), NF4 data-type paragraph:
 *    16 levels from the inverse normal CDF, more of them near zero; weights
 *    map to levels through lookup tables after per-block scaling.
 *    Double-quantization paragraph: one absmax per 64-weight block, the absmax
 *    values themselves quantized to 8 bits with their own meta-scales; the
 *    scales are dequantized first, then used to dequantize the weights.
 *    Quantized-GEMM paragraph: weights dequantized on the fly, float32
 *    multiply, float32 outputs.  QuantState paragraph: the quantized data,
 *    absmax, data type and shape travel together (here: nf4_qtensor).
 *    4-bit training paragraph: the 4-bit data type is NF4 or FP4, standard
 *    floating-point 4-bit (quant_type NF4_QT_FP4 here).
 *
 * Exact semantics (the readings where the pages are silent):
 *  - weight W is logical [rows, cols] row-major, flattened e = r*cols + c;
 *    with B weights per block (64 by default; 32, 128 or 256), block b holds
 *    elements Bb .. Bb+B-1 (the last block may be partial);
 *  - a_b = max|x| over the block (fp32); n = fp32(x / a_b) (IEEE division);
 *    code = index of the nearest level, ties to the lower index; an all-zero
 *    block codes every element as the +0 level (NF4 code 7, FP4 code 0);
 *  - NF4 levels ascend with the code (nf4_codebook).  FP4 codes are the bit
 *    patterns of the E2M1 4-bit float (bit 3 the sign, bits 2-1 the exponent
 *    with bias 1, bit 0 the mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6)
 *    and a level is the value over 6, rounded once to fp32; ties to the lower
 *    code then go toward zero, and zero takes code 0;
 *  - packed byte j = code[2j] | code[2j+1] << 4 (odd count: high nibble 0);
 *  - double quantization: mu = exact mean of all a_b rounded once to fp32;
 *    a'_b = fp32(a_b - mu); per group of 256 consecutive blocks
 *    s_g = fp32(max|a'| / 127); q_b = clamp(rint_even(fp32(a'_b / s_g)),
 *    -127, 127) as int8; an all-zero group has s_g = 0 and q = 0;
 *  - dequantized absmax a^_b = fp32(fp32(q_b * s_g) + mu) with double
 *    quantization (two roundings, no fused multiply-add), else a^_b = a_b;
 *  - W^_e = bf16_rne(fp32(level[code_e] * a^_b)); the fp32 variant returns
 *    fp32(level * a^) unrounded;
 *  - GEMMs: Y = X W^T and dX = dY W^ with bf16 operands, fp32 accumulation
 *    and fp32 (or, on request, bf16-rounded) outputs; W^ is formed on chip.
 *
 * Conventions for every call:
 *  - Device pointers point to memory of the current HIP device; every device
 *    pointer must be 16-byte aligned (NF4_ERR_ALIGN otherwise).
 *  - The caller owns and frees every buffer.  The library never allocates or
 *    frees device memory and never synchronises; work is queued on `stream`
 *    (a hipStream_t; NULL means the default stream) and outputs are valid once
 *    the stream has reached that point.  No global mutable state.
 *  - Every problem the host can see (NULL pointer, bad size, bad blocksize,
 *    bad dtype enum, misalignment, short workspace, unsupported shape) is
 *    returned before anything is launched, and outputs are left untouched.
 *    A failed launch returns NF4_ERR_HIP.
 *  - Non-finite weights are outside the method's domain (precondition); if
 *    `d_status` is given, the quantizer ORs bit 0 into it when it sees a
 *    non-finite block absmax.
 *  - Dense tensors are row-major and contiguous: X [M,K], Y [M,N],
 *    dY [M,N], dX [M,K], where the weight is [N,K] (nn.Linear's [out,in]).
 */
#ifndef NF4_H_
#define NF4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nf4_status {
  NF4_OK = 0,
  NF4_ERR_NULL = 1,         /* a required pointer is NULL */
  NF4_ERR_SHAPE = 2,        /* a size is negative, zero where it may not be, or too large */
  NF4_ERR_BLOCKSIZE = 3,    /* blocksize is not 32, 64, 128 or 256 */
  NF4_ERR_DTYPE = 4,        /* unknown nf4_dtype value */
  NF4_ERR_ALIGN = 5,        /* a device pointer is not 16-byte aligned */
  NF4_ERR_WORKSPACE = 6,    /* workspace smaller than nf4_sizes reports */
  NF4_ERR_UNSUPPORTED = 7,  /* valid but not supported, e.g. a GEMM with cols % 64 != 0 */
  NF4_ERR_HIP = 8,          /* a HIP launch failed */
  NF4_ERR_QUANT_TYPE = 9,   /* unknown nf4_quant_type value */
  NF4_ERR_SCRATCH = 10      /* the tensor needs more than the fixed scratch of nf4_quantize_noalloc */
};

enum nf4_dtype {
  NF4_F32 = 0,
  NF4_BF16 = 1
};

/* The 4-bit data type of a quantized weight: its level table. */
enum nf4_quant_type {
  NF4_QT_NF4 = 0,   /* the NF4 levels (default) */
  NF4_QT_FP4 = 1    /* E2M1 values over 6 */
};

/* Largest element count a quantized tensor may hold (2^36; a weight that size
 * is 128 GiB in bf16, and its block count fits 32 bits at every block size). */
#define NF4_MAX_NUMEL ((int64_t)1 << 36)
/* The GEMMs take weights with fewer columns than this (32-bit tile offsets). */
#define NF4_GEMM_COLS_LIMIT ((int64_t)1 << 24)
/* Weights per absmax block: the default (and the workloads' size) is 64;
 * 32, 128 and 256 are accepted as well (any power of two in that range). */
#define NF4_BLOCKSIZE 64
#define NF4_BLOCKSIZE_MIN 32
#define NF4_BLOCKSIZE_MAX 256
/* Absmax values per double-quantization group. */
#define NF4_DQ_GROUP 256
/* Low-rank adapter ranks: a multiple of this step, at most the maximum. */
#define NF4_LORA_RANK_STEP 16
#define NF4_LORA_MAX_RANK 1024

/*
 * A quantized weight: host struct, device buffers (the QuantState analogue).
 * Blocks run over the row-major flattening: block b holds elements
 * b*blocksize .. b*blocksize + blocksize - 1 (it may span rows when blocksize
 * does not divide cols; the last one may be partial).  Sizes for rows x cols
 * (numel = rows*cols, nblocks = ceil(numel/blocksize), ngroups =
 * ceil(nblocks/256)):
 *   packed        ceil(numel/2) bytes
 *   absmax        nblocks fp32     (double_quant == 0; NULL otherwise)
 *   absmax_q      nblocks int8     (double_quant == 1)
 *   absmax_scale  ngroups fp32     (double_quant == 1)
 *   absmax_mean   1 fp32           (double_quant == 1)
 * quant_type (an nf4_quant_type) names the level table; every call that
 * reads the struct rejects other values with NF4_ERR_QUANT_TYPE.  It is the
 * last field so that a zero-initialised tail means NF4.
 * The struct is read during a call only; the library keeps no pointer to it.
 */
typedef struct nf4_qtensor {
  int64_t rows;
  int64_t cols;
  int32_t blocksize;
  int32_t double_quant;
  uint8_t *packed;
  float *absmax;
  int8_t *absmax_q;
  float *absmax_scale;
  float *absmax_mean;
  int32_t quant_type;
} nf4_qtensor;

/* A short English description of a status code (static storage). */
const char *nf4_status_string(int status);

/*
 * Copies the 16 NF4 levels, ascending (level 0 = -1, level 7 = 0,
 * level 15 = +1), into host memory `levels16`.  Source: "bitsandbytes" page,
 * NF4 data-type paragraph (levels from the inverse normal CDF); construction:
 * QLoRA's 8 positive / 7 negative normal quantiles with offset 0.9677083,
 * normalised by the largest, rounded once to fp32.
 */
int nf4_codebook(float *levels16);

/*
 * Copies the 16 levels of `quant_type` (an nf4_quant_type), indexed by code,
 * into host memory `levels16`: NF4 as nf4_codebook; FP4 c[0] = +0 .. c[7] = 1
 * and c[8 + i] = -c[i].  Errors: NF4_ERR_NULL, NF4_ERR_QUANT_TYPE.
 */
int nf4_levels(int quant_type, float *levels16);

/*
 * Copies into host memory `thresholds15` the 15 decision thresholds the
 * quantizer uses: t_i is the smallest fp32 n that codes to i+1, so that
 * code(n) = #{i : n >= t_i} equals the nearest level with ties to the lower
 * index.  Exposed so the derivation can be checked against an independent
 * nearest-level search.
 */
int nf4_thresholds(float *thresholds15);

/*
 * Buffer sizes for a rows x cols weight.  Any output pointer may be NULL.
 * workspace_bytes is the device workspace nf4_quantize needs (0 without
 * double quantization).  Errors: NF4_ERR_SHAPE (rows or cols < 1, or
 * numel > NF4_MAX_NUMEL), NF4_ERR_BLOCKSIZE.
 */
int nf4_sizes(int64_t rows, int64_t cols, int blocksize, int double_quant,
              int64_t *packed_bytes, int64_t *nblocks, int64_t *ngroups,
              size_t *workspace_bytes);

/*
 * Quantizes W (device, [rows, cols] row-major, dtype w_dtype = NF4_F32 or
 * NF4_BF16) into `out`, whose rows/cols/blocksize/double_quant must match the
 * arguments and whose buffers are sized per nf4_sizes; out->quant_type picks
 * the level table (NF4 or FP4).  "Zenbit" page,
 * zenbit.nf4 bullet; "bitsandbytes" page, NF4 and double-quantization
 * paragraphs.  `workspace` (device, >= workspace_bytes from nf4_sizes, may be
 * NULL when that is 0) is scratch for the fp32 absmax and the exact-mean
 * accumulators; its contents on entry do not matter.  `d_status` (device
 * uint32, may be NULL): bit 0 is ORed in if a block absmax is non-finite.
 * Bit-exact and deterministic: the mean is formed from integer sums, so the
 * result does not depend on launch order.
 */
int nf4_quantize(const void *W, int w_dtype, int64_t rows, int64_t cols,
                 int blocksize, int double_quant, const nf4_qtensor *out,
                 void *workspace, size_t workspace_bytes, uint32_t *d_status,
                 void *stream);

/*
 * nf4_quantize without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * nf4_quantize; the double-quantization scratch (exact-mean rows and the fp32
 * absmax of every block) lives in a fixed buffer inside the library, one per
 * GPU, sized for NF4_NOALLOC_MAX_BLOCKS blocks (about 16.3 MiB), held until
 * the process ends.  A tensor with more blocks, with double_quant set, is
 * refused with NF4_ERR_SCRATCH before anything is launched; without double
 * quantization no scratch is used and every size nf4_quantize takes is
 * accepted.  Calls no allocating routine.  The buffer is shared by every call
 * on a GPU and keeps the last call's contents (the kernels overwrite every
 * byte they later read, so nothing needs clearing between calls); calls whose
 * execution overlaps on one GPU (different streams, different threads) race
 * on it and must be serialised by the caller.  The first call on each device
 * looks the buffer's device address up (thread-safe); NF4_ERR_HIP if that
 * fails.
 */
#define NF4_NOALLOC_MAX_BLOCKS ((int64_t)1 << 22)
int nf4_quantize_noalloc(const void *W, int w_dtype, int64_t rows, int64_t cols,
                         int blocksize, int double_quant, const nf4_qtensor *out,
                         uint32_t *d_status, void *stream);

/*
 * Writes the dequantized weight W^ (device, [rows, cols] row-major) in
 * out_dtype: NF4_BF16 gives bf16_rne(level * a^) (the operand the GEMMs
 * use), NF4_F32 gives fp32(level * a^).  "bitsandbytes" page,
 * double-quantization paragraph: absmax first, then the weights.
 */
int nf4_dequantize(const nf4_qtensor *q, void *out, int out_dtype, void *stream);

/*
 * Y = X W^T.  X: device bf16 [M, K] with K = q->cols; Y: device [M, N] with
 * N = q->rows, in y_dtype (NF4_F32, or NF4_BF16 = one rounding of the fp32
 * accumulator).  W^ is dequantized on chip to bf16 and never written to
 * memory.  Requires K % 64 == 0 and K < NF4_GEMM_COLS_LIMIT
 * (NF4_ERR_UNSUPPORTED otherwise).  M == 0 is a successful no-op.  "Zenbit" page, zenbit.pallas_nf4 bullet (fused
 * forward); "bitsandbytes" page, quantized-GEMM paragraph (fp32 output).
 */
int nf4_matmul_fwd(const void *X, int64_t M, const nf4_qtensor *q, void *Y,
                   int y_dtype, void *stream);

/*
 * dX = dY W^ (the backward pass with respect to the input of Y = X W^T; no
 * gradient for the frozen weight).  dY: device bf16 [M, N] with N = q->rows;
 * dX: device [M, K] with K = q->cols, in dx_dtype (NF4_F32 or NF4_BF16).
 * Requires K % 64 == 0 and K < NF4_GEMM_COLS_LIMIT (NF4_ERR_UNSUPPORTED
 * otherwise).  M == 0 is a successful no-op.  "Zenbit" page,
 * zenbit.pallas_nf4 bullet (fused backward, dL/dX only).
 */
int nf4_matmul_bwd_dx(const void *dY, int64_t M, const nf4_qtensor *q, void *dX,
                      int dx_dtype, void *stream);

/*
 * Y = X W^T + U B^T: the fused forward with a low-rank adapter term added in
 * the same fp32 accumulators before the single store.  "bitsandbytes" page,
 * 4-bit/LoRA paragraph (frozen 4-bit base weight plus small trainable
 * adapters); "Zenbit" page, NF4DenseFused.  For an adapter with down
 * projection A [r, K] and up projection B [N, r] (nn.Linear layouts), U is the
 * down-projected activation X A^T.  U: device bf16 [M, r]; B: device bf16
 * [N, r] with N = q->rows (any adapter scaling folded in); both row-major.
 * X, Y, y_dtype and the shape rules as nf4_matmul_fwd.  r must be a multiple
 * of NF4_LORA_RANK_STEP in [NF4_LORA_RANK_STEP, NF4_LORA_MAX_RANK]
 * (NF4_ERR_UNSUPPORTED otherwise); U and B must be 16-byte aligned.  The
 * adapter product runs on the same bf16 matrix cores with fp32 accumulation.
 */
int nf4_matmul_fwd_lora(const void *X, int64_t M, const nf4_qtensor *q,
                        const void *U, const void *B, int64_t r, void *Y,
                        int y_dtype, void *stream);

/*
 * dX = dY W^ + V A: the fused backward with respect to the input, with the
 * adapter's contribution added in the same accumulators.  For the adapter of
 * nf4_matmul_fwd_lora, V = dY B (device bf16 [M, r]) and At = A^T (device
 * bf16 [K, r] with K = q->cols), both row-major.  dY, dX, dx_dtype and the
 * shape rules as nf4_matmul_bwd_dx; r as nf4_matmul_fwd_lora.  The
 * adapter's own products (U, V and its gradients) are nf4_adapter_matmul.
 */
int nf4_matmul_bwd_dx_lora(const void *dY, int64_t M, const nf4_qtensor *q,
                           const void *V, const void *At, int64_t r, void *dX,
                           int dx_dtype, void *stream);

/*
 * C = alpha op(A) op(B): the dense products of a low-rank adapter on the
 * frozen 4-bit weight ("bitsandbytes" page, 4-bit/LoRA paragraph: a frozen
 * 4-bit base weight with small trainable adapters).  For an adapter with down
 * projection Ad [r, K] and up projection Bu [N, r] (scale s) on input X [M, K]
 * and output gradient dY [M, N]:
 *   U  = s X Ad^T  (trans_a 0, trans_b 1)   the activation nf4_matmul_fwd_lora adds
 *   V  = s dY Bu   (trans_a 0, trans_b 0)   the activation nf4_matmul_bwd_dx_lora adds
 *   dAd = V^T X    (trans_a 1, trans_b 0)   gradient of the down projection
 *   dBu = dY^T U   (trans_a 1, trans_b 0)   gradient of the up projection
 * op(A) is [M, K]: A (trans_a = 0, stored [M, K]) or A^T (trans_a = 1, stored
 * [K, M]); op(B) is [K, N]: B (trans_b = 0, stored [K, N]) or B^T (trans_b =
 * 1, stored [N, K]).  A and B are device bf16, row-major with row strides lda
 * and ldb elements (at least the stored row length); C is device [M, N] with
 * row stride ldc >= N in c_dtype: NF4_F32, or NF4_BF16 = one round-to-nearest-
 * even rounding of the fp32 value.  Products accumulate in fp32 on the bf16
 * matrix cores; alpha multiplies the fp32 sum once.  M or N == 0 is a
 * successful no-op; K >= 1.  Errors: NF4_ERR_UNSUPPORTED (trans flag not 0 or
 * 1, a stored operand of 2^31 bytes or more), NF4_ERR_SHAPE (negative size,
 * K < 1, a stride shorter than its row), NF4_ERR_DTYPE, NF4_ERR_NULL,
 * NF4_ERR_ALIGN (A, B and C 16-byte aligned).
 */
int nf4_adapter_matmul(int trans_a, int trans_b, int64_t M, int64_t N, int64_t K,
                       float alpha, const void *A, int64_t lda, const void *B,
                       int64_t ldb, void *C, int c_dtype, int64_t ldc, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_H_ */
