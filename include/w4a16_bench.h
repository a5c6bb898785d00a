/*
 * w4a16_bench.h -- measurement kernels shipped with the W4A16 library.
 *
 * Not part of the method: these give the achievable HBM read bandwidth of
 * the device (the ceiling the verify linear is measured against) and a plain
 * copy of known size whose hardware byte counters calibrate the FETCH_SIZE
 * and WRITE_SIZE readings of the verify kernels.  The pages ask that
 * throughput be profiled before it is trusted (ordoresearch.ai review,
 * "Design Implications for Practitioners").
 */
#ifndef W4A16_BENCH_H
#define W4A16_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (multiple of 16, device pointer 16-byte aligned) once with
 * 128-bit loads; each workgroup writes one XOR digest to sink[blockIdx]
 * (device, at least w4_bench_read_blocks() uint32 entries).  Async on
 * `stream`.  Returns a W4_* status. */
int w4_bench_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);
int w4_bench_read_blocks(void);

/* Copy `bytes` (multiple of 16, both 16-byte aligned, non-overlapping). */
int w4_bench_copy(void* dst, const void* src, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* W4A16_BENCH_H */
