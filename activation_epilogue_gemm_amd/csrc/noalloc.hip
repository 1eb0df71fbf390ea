// Library-owned device scratch for gemmepi_execute_noalloc, the entry point
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The split-K partial tiles and arrival counters of a plan normally live in
// a caller-owned workspace (gemmepi_execute_ws).  Here they live in a
// file-scope device array of kScratchBytes instead, which the code object
// loader allocates once per device when the library's kernels are first
// loaded there, and which stays allocated until the process ends.
//
// Host code never uses the array's name as a device address (on the host
// it is only a stand-in for the symbol): the address is looked up once per
// device with hipGetSymbolAddress, with that device current, and cached.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace gemmepi {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

hipError_t scratch_pointer(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    ptrs[dev] = p;
  }
  *ptr = ptrs[dev];
  return hipSuccess;
}

}  // namespace gemmepi
