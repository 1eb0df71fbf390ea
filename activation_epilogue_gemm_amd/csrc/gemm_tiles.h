// The tile configurations of the tiled MFMA GEMM, shared by the kernel
// instantiations and the host-side planner:
//   X(id, BM, BN, BK, waves along M, waves along N, LDS stages)
// BM x BN is the output tile of one workgroup, BK the K depth of one slab,
// and the LDS holds a ring of `stages` slabs ((BM + BN) * BK * 2 bytes each).
#pragma once

#define GEMMEPI_TILES(X)      \
  X(0, 256, 256, 64, 2, 4, 2) \
  X(1, 256, 256, 32, 2, 4, 4) \
  X(2, 256, 256, 32, 2, 2, 4) \
  X(3, 256, 128, 64, 2, 2, 3) \
  X(4, 128, 128, 64, 2, 2, 3) \
  X(5, 128, 64, 64, 2, 2, 3)  \
  X(6, 64, 64, 64, 2, 2, 3)
