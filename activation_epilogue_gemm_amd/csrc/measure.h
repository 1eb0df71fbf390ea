/*
 * libgemmepi_measure: measurement helpers used by the benchmark beside
 * libgemmepi (not part of the GEMM library's ABI).
 *
 * gemmepi_measure_stream_read: read `bytes` bytes at `p` once with 128-bit
 * loads spread over the whole GPU and write at most one word per workgroup
 * into `sink`, so that the loads cannot be dropped.  It is the practical HBM
 * read rate that the thin-M decode kernel is compared with.
 *   p            device memory, 16-byte aligned; bytes a positive multiple of 16
 *   sink         device memory of at least 4096 bytes (contents unspecified)
 *   threads      workgroup size: 256, 512 or 1024
 *   loads        16-byte loads per thread, all in flight at once: 4, 8, 16 or 32
 *                (each workgroup reads threads * loads * 16 contiguous bytes)
 *   nontemporal  1: non-temporal loads (streaming, evict-first), 0: normal loads
 *   stream       hipStream_t or NULL; the call only enqueues
 * Returns 0, 1 for an invalid argument (nothing launched), 2 for a launch error.
 */
#ifndef GEMMEPI_MEASURE_H
#define GEMMEPI_MEASURE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int gemmepi_measure_stream_read(const void* p, size_t bytes, void* sink, int threads, int loads,
                                int nontemporal, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMMEPI_MEASURE_H */
