/*
 * pkv_bench.h -- a measurement helper exported by libpkv.so beside the
 * entry points of pkv.h.  It is not a step of the method: the benchmark
 * calls it to measure, on the same GPU and in the same run, the bandwidth a
 * plain streaming copy reaches, as context for the kernels' figures.
 */
#ifndef PKV_BENCH_H
#define PKV_BENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * pkv_stream_copy -- copy `bytes` bytes from src to dst (both device
 * pointers, 16-byte aligned, not overlapping) with one kernel: 16-byte
 * non-temporal loads and stores, grid-stride over `blocks` blocks of 256
 * threads, enqueued on `stream` (a hipStream_t, NULL for the default
 * stream).  Returns 0 (PKV_OK) when enqueued; PKV_ERR_NULL (1) for a NULL
 * pointer, PKV_ERR_SHAPE (2) for blocks == 0, PKV_ERR_ALIGN (4) when a
 * pointer or `bytes` is not a multiple of 16, PKV_ERR_LAUNCH (7) when the
 * launch is refused.  bytes == 0 enqueues nothing.  Allocates nothing.
 */
int pkv_stream_copy(const void* src, void* dst, uint64_t bytes, uint32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BENCH_H */
