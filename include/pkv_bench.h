/*
 * pkv_bench.h -- measurement helpers exported by libpkv.so beside the
 * entry points of pkv.h.  They are not steps of the method: the benchmark
 * calls them to measure, on the same GPU and in the same run, the bandwidth
 * a plain streaming copy reaches, and the time a plain stream of each
 * kernel's own read and write traffic takes, as context for the kernels'
 * figures.
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

/*
 * pkv_stream_mix -- read `read_bytes` bytes from src and write `write_bytes`
 * bytes to dst (device pointers, 16-byte aligned) with one kernel of
 * `blocks` blocks of 256 threads, enqueued on `stream`: 16-byte
 * non-temporal loads and stores, grid-stride, the reads and the writes
 * interleaved evenly at the ratio read_bytes : write_bytes throughout the
 * launch (the longer stream sets the iterations; the shorter one moves on
 * at the matching fraction of them), each lane with four 16-byte loads in
 * flight and every wave instruction covering 1 KiB contiguous.
 * It stands for a kernel that moves those bytes in that mix, so that a
 * kernel's time can be set beside a plain stream of its own traffic.
 * src == dst is the in-place form (read_bytes must equal write_bytes): every
 * 16-byte piece is read and written back at its own address, unchanged.
 * With read_bytes == write_bytes and distinct buffers dst receives a copy of
 * src; at other ratios a written piece is the XOR of the pieces its thread
 * read since its previous write (contents are not part of the contract).
 * write_bytes == 0 is a read-only stream (dst is then not written).
 * Returns 0 (PKV_OK) when enqueued; PKV_ERR_NULL (1) for a NULL pointer;
 * PKV_ERR_SHAPE (2) for blocks == 0, or src == dst with read_bytes !=
 * write_bytes; PKV_ERR_ALIGN (4) when a pointer or a byte count is not a
 * multiple of 16; PKV_ERR_RANGE (6) when a byte count is 32 GiB or more, or
 * the two ranges overlap without being the same; PKV_ERR_LAUNCH (7) when the
 * launch is refused.  Nothing is enqueued when both counts are 0.  Allocates
 * nothing.
 */
int pkv_stream_mix(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                   uint32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BENCH_H */
