// Tiled MFMA GEMM instantiations: bf16 inputs, B stored [N,K] (K contiguous).
// One file per (dtype, B layout) so the tile variants compile in parallel.
#include "gemm_mfma.hpp"

namespace gemmepi {

hipError_t launch_gemm_bf16_bt(int tile, const GemmArgs& a, hipStream_t s) {
  return launch_by_tile<__bf16, true>(tile, a, s);
}

hipError_t blocks_per_cu_bf16_bt(int tile, int* n) {
  return blocks_per_cu_by_tile<__bf16, true>(tile, n);
}

}  // namespace gemmepi
