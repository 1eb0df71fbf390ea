// Tiled MFMA GEMM instantiations: bf16 inputs, B stored [K,N] (N contiguous).
// One file per (dtype, B layout) so the tile variants compile in parallel.
#include "gemm_mfma.hpp"

namespace gemmepi {

hipError_t launch_gemm_bf16_bn(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_by_tile<__bf16, false>(tile, a, s);
}

hipError_t blocks_per_cu_bf16_bn(int tile, int* n) {
  return blocks_per_cu_by_tile<__bf16, false>(tile, n);
}

}  // namespace gemmepi
