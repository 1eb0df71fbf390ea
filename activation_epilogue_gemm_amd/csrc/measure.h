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
 *
 * gemmepi_measure_mfma_loop: the matrix cores alone at the chip's power
 * limit, with no memory traffic.  Each of `blocks` workgroups has 8 waves of
 * 64 threads (2 per SIMD, as the 256 x 256 GEMM tile); wave w loads 12
 * operand fragments of 16 bytes per lane from src (fragment slot f of wave
 * w, lane l at byte ((12 w + f) 64 + l) 16; slots 0-7 are the A fragments,
 * 8-11 the B fragments), then issues `rounds` times the 32
 * v_mfma_f32_16x16x32 (fp16, or bf16 with bf16 = 1) of one k step of the
 * tile's 128 x 64 accumulators, in the GEMM's order.  Lane 0 of wave 0
 * stores the fp32 sum of its 128 accumulators into float sink[block % 1024].
 * Work per call: blocks x 8 x rounds x 32 x 16384 flop.
 *   src      device memory, 16-byte aligned, src_bytes >= 98304
 *            (every workgroup reads the same 96 KiB)
 *   sink     device memory of at least 4096 bytes, 4-byte aligned
 *   blocks   1 .. 65535;  rounds 1 .. 2^24;  bf16 0 or 1
 *   stream   hipStream_t or NULL; the call only enqueues
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
int gemmepi_measure_mfma_loop(const void* src, size_t src_bytes, void* sink, int blocks, int rounds,
                              int bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMMEPI_MEASURE_H */
