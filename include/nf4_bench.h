/*
 * nf4_bench.h -- C ABI of libnf4_bench (package dequant_gemm_amd): a plain
 * HBM read stream, the achievable-bandwidth reference that the benchmark
 * reports beside the NF4 kernels' GB/s.  Not part of the quantization method.
 */
#ifndef NF4_BENCH_H_
#define NF4_BENCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` bytes at device pointer `src` once (16-byte loads, a
 * grid-stride loop over `grid` workgroups of `block` threads) and writes one
 * 32-bit XOR of each thread's data to `sink` (device, grid * block uint32),
 * so that no load can be dropped.  `bytes` must be a positive multiple of 16,
 * `src` and `sink` 16-byte aligned, `block` one of 64, 128, 256, 512, 1024,
 * `grid` in [1, 65536].  Returns 0, 1 for a bad argument (nothing launched),
 * or 2 for a failed launch.  Queued on `stream` (a hipStream_t, NULL = default).
 */
int nf4bench_read_stream(const void *src, size_t bytes, uint32_t *sink, int grid, int block, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* NF4_BENCH_H_ */
