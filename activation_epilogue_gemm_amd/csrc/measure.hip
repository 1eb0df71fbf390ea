// libgemmepi_measure: measurement helpers beside the fused GEMM library, used
// by the benchmark only (not part of libgemmepi's ABI).
//
// gemmepi_measure_stream_read reads a device buffer once with 128-bit loads
// spread over the whole GPU: the practical HBM read rate that the thin-M
// decode kernel, which must stream its whole weight matrix on every call, is
// compared with (ops-nn MatMul fusion article, section "Why MatMul is the
// core bottleneck of LLM inference").  Its launch shape is a parameter, so
// that the best rate over block sizes, loads in flight and cache policy is
// the one reported.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "measure.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads the contiguous block [b * THREADS * LOADS, ...) of 16-byte
// chunks, LOADS chunks per thread, all in flight before any is consumed.
template <int THREADS, int LOADS, bool NT>
__global__ void __launch_bounds__(THREADS) stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                              uint32_t* sink) {
  const size_t base = (size_t)blockIdx.x * THREADS * LOADS + threadIdx.x;
  u32x4 v[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) {
    const size_t i = base + (size_t)u * THREADS;
    if (i < n16)
      v[u] = NT ? __builtin_nontemporal_load(p + i) : p[i];
    else
      v[u] = u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t acc = 0;
#pragma unroll
  for (int u = 0; u < LOADS; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  // never true for the benchmark's data in practice; keeps the loads alive
  if (acc == 0x9E3779B9u) sink[blockIdx.x & 1023] = acc;
}

template <int THREADS, int LOADS>
hipError_t launch(const void* p, size_t n16, uint32_t* sink, int nt, hipStream_t s) {
  const size_t per_block = (size_t)THREADS * LOADS;
  const size_t blocks = (n16 + per_block - 1) / per_block;
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<THREADS, LOADS, true>), dim3((unsigned)blocks),
                       dim3(THREADS), 0, s, (const u32x4*)p, n16, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<THREADS, LOADS, false>), dim3((unsigned)blocks),
                       dim3(THREADS), 0, s, (const u32x4*)p, n16, sink);
  return hipGetLastError();
}

template <int THREADS>
hipError_t by_loads(int loads, const void* p, size_t n16, uint32_t* sink, int nt, hipStream_t s) {
  switch (loads) {
    case 4: return launch<THREADS, 4>(p, n16, sink, nt, s);
    case 8: return launch<THREADS, 8>(p, n16, sink, nt, s);
    case 16: return launch<THREADS, 16>(p, n16, sink, nt, s);
    case 32: return launch<THREADS, 32>(p, n16, sink, nt, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

extern "C" int gemmepi_measure_stream_read(const void* p, size_t bytes, void* sink, int threads,
                                           int loads, int nontemporal, void* stream) {
  if (!p || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)p % 16) != 0) return 1;
  const size_t n16 = bytes / 16;
  if (threads != 256 && threads != 512 && threads != 1024) return 1;
  if (loads != 4 && loads != 8 && loads != 16 && loads != 32) return 1;
  if (n16 / ((size_t)threads * loads) >= 0x7FFFFFFFull) return 1;
  (void)hipGetLastError();
  hipError_t e;
  hipStream_t s = (hipStream_t)stream;
  if (threads == 256) e = by_loads<256>(loads, p, n16, (uint32_t*)sink, nontemporal, s);
  else if (threads == 512) e = by_loads<512>(loads, p, n16, (uint32_t*)sink, nontemporal, s);
  else e = by_loads<1024>(loads, p, n16, (uint32_t*)sink, nontemporal, s);
  return e == hipSuccess ? 0 : 2;
}
