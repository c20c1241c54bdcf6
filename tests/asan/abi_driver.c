/* Host-side checks of the C ABI under AddressSanitizer and UndefinedBehavior-
 * Sanitizer: every validation path of include/nf4.h and the host-only calls.
 * None of them reaches a HIP call, so this runs without a GPU.  Exit status 0
 * when every call returns the documented status. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "nf4.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    int got_ = (call);                                                                  \
    if (got_ != (want)) {                                                               \
      fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
              got_, (want));                                                            \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

/* fake, 16-byte aligned device addresses: never dereferenced on these paths */
#define P ((void *)(uintptr_t)(1u << 20))
#define P2 ((void *)(uintptr_t)((1u << 20) + 4))

static nf4_qtensor qt(int64_t rows, int64_t cols, int bs, int dq, int type) {
  nf4_qtensor q;
  memset(&q, 0, sizeof q);
  q.rows = rows;
  q.cols = cols;
  q.blocksize = bs;
  q.double_quant = dq;
  q.packed = (uint8_t *)P;
  q.absmax = dq ? NULL : (float *)P;
  q.absmax_q = dq ? (int8_t *)P : NULL;
  q.absmax_scale = dq ? (float *)P : NULL;
  q.absmax_mean = dq ? (float *)P : NULL;
  q.quant_type = type;
  return q;
}

int main(void) {
  float levels[16], thr[15];
  int64_t pb, nb, ng;
  size_t ws;
  for (int s = -1; s < 12; ++s) {
    const char *str = nf4_status_string(s);
    if (!str || !str[0]) ++failures;
  }
  EXPECT(nf4_codebook(levels), NF4_OK);
  EXPECT(nf4_codebook(NULL), NF4_ERR_NULL);
  EXPECT(nf4_levels(NF4_QT_NF4, levels), NF4_OK);
  EXPECT(nf4_levels(NF4_QT_FP4, levels), NF4_OK);
  EXPECT(nf4_levels(2, levels), NF4_ERR_QUANT_TYPE);
  EXPECT(nf4_levels(NF4_QT_FP4, NULL), NF4_ERR_NULL);
  EXPECT(nf4_thresholds(thr), NF4_OK);
  EXPECT(nf4_thresholds(NULL), NF4_ERR_NULL);

  /* sizes: every block size, odd counts, the element limit, NULL outputs */
  const int sizes[4] = {32, 64, 128, 256};
  for (int i = 0; i < 4; ++i) {
    EXPECT(nf4_sizes(3, 37, sizes[i], 1, &pb, &nb, &ng, &ws), NF4_OK);
    EXPECT(nf4_sizes((int64_t)1 << 18, (int64_t)1 << 18, sizes[i], 1, NULL, &nb, NULL, NULL), NF4_OK);
    EXPECT(nf4_sizes(((int64_t)1 << 18) + 1, (int64_t)1 << 18, sizes[i], 0, NULL, NULL, NULL, NULL), NF4_ERR_SHAPE);
  }
  EXPECT(nf4_sizes(0, 64, 64, 1, &pb, &nb, &ng, &ws), NF4_ERR_SHAPE);
  EXPECT(nf4_sizes(64, -5, 64, 1, &pb, &nb, &ng, &ws), NF4_ERR_SHAPE);
  EXPECT(nf4_sizes(INT64_MAX, INT64_MAX, 64, 1, &pb, &nb, &ng, &ws), NF4_ERR_SHAPE);
  EXPECT(nf4_sizes(64, 64, 48, 1, &pb, &nb, &ng, &ws), NF4_ERR_BLOCKSIZE);
  EXPECT(nf4_sizes(64, 64, 64, 2, &pb, &nb, &ng, &ws), NF4_ERR_UNSUPPORTED);

  /* quantize */
  nf4_sizes(64, 64, 64, 1, NULL, NULL, NULL, &ws);
  nf4_qtensor q = qt(64, 64, 64, 1, NF4_QT_NF4), bad;
  EXPECT(nf4_quantize(NULL, NF4_BF16, 64, 64, 64, 1, &q, P, ws, NULL, NULL), NF4_ERR_NULL);
  EXPECT(nf4_quantize(P, 7, 64, 64, 64, 1, &q, P, ws, NULL, NULL), NF4_ERR_DTYPE);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 16, 1, &q, P, ws, NULL, NULL), NF4_ERR_BLOCKSIZE);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 128, 1, &q, P, ws, NULL, NULL), NF4_ERR_SHAPE);
  EXPECT(nf4_quantize(P2, NF4_BF16, 64, 64, 64, 1, &q, P, ws, NULL, NULL), NF4_ERR_ALIGN);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, &q, P, ws - 1, NULL, NULL), NF4_ERR_WORKSPACE);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, &q, NULL, ws, NULL, NULL), NF4_ERR_NULL);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, &q, P, ws, (uint32_t *)P2, NULL), NF4_ERR_ALIGN);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, NULL, P, ws, NULL, NULL), NF4_ERR_NULL);
  bad = qt(64, 64, 64, 1, 5);
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, &bad, P, ws, NULL, NULL), NF4_ERR_QUANT_TYPE);
  bad = qt(64, 64, 64, 1, NF4_QT_NF4);
  bad.absmax_mean = NULL;
  EXPECT(nf4_quantize(P, NF4_BF16, 64, 64, 64, 1, &bad, P, ws, NULL, NULL), NF4_ERR_NULL);

  /* dequantize and the GEMMs */
  nf4_qtensor g = qt(128, 256, 64, 1, NF4_QT_FP4);
  EXPECT(nf4_dequantize(NULL, P, NF4_BF16, NULL), NF4_ERR_NULL);
  EXPECT(nf4_dequantize(&g, NULL, NF4_BF16, NULL), NF4_ERR_NULL);
  EXPECT(nf4_dequantize(&g, P, 9, NULL), NF4_ERR_DTYPE);
  EXPECT(nf4_dequantize(&g, P2, NF4_BF16, NULL), NF4_ERR_ALIGN);
  EXPECT(nf4_matmul_fwd(P, 0, &g, NULL, NF4_F32, NULL), NF4_OK);              /* M == 0: no-op */
  EXPECT(nf4_matmul_bwd_dx(P, 0, &g, NULL, NF4_F32, NULL), NF4_OK);
  EXPECT(nf4_matmul_fwd(P, -1, &g, P, NF4_F32, NULL), NF4_ERR_SHAPE);
  EXPECT(nf4_matmul_fwd(NULL, 4, &g, P, NF4_F32, NULL), NF4_ERR_NULL);
  EXPECT(nf4_matmul_bwd_dx(P, 4, &g, P2, NF4_F32, NULL), NF4_ERR_ALIGN);
  nf4_qtensor k96 = qt(128, 96, 64, 1, NF4_QT_NF4);
  EXPECT(nf4_matmul_fwd(P, 4, &k96, P, NF4_F32, NULL), NF4_ERR_UNSUPPORTED);
  EXPECT(nf4_matmul_fwd_lora(P, 4, &g, P, P, 8, P, NF4_F32, NULL), NF4_ERR_UNSUPPORTED);
  EXPECT(nf4_matmul_bwd_dx_lora(P, 4, &g, NULL, P, 16, P, NF4_F32, NULL), NF4_ERR_NULL);
  bad = qt(128, 256, 64, 1, -1);
  EXPECT(nf4_matmul_bwd_dx(P, 4, &bad, P, NF4_F32, NULL), NF4_ERR_QUANT_TYPE);

  if (failures) fprintf(stderr, "%d failures\n", failures);
  return failures ? 1 : 0;
}
