// The tile configurations of the tiled MFMA GEMM, shared by the kernel
// instantiations and the host-side planner:
//   X(id, BM, BN, BK, waves along M, waves along N, LDS stages, schedule)
// BM x BN is the output tile of one workgroup, BK the K depth of one slab,
// and the LDS holds a ring of `stages` slabs ((BM + BN) * BK * 2 bytes each).
// schedule 0: every wave loads its fragments and multiplies in lockstep;
// schedule 1: ping-pong -- the two wave rows alternate between a phase that
// only loads (LDS -> registers, next slabs -> LDS) and a phase that only
// issues MFMAs, so each SIMD always has one wave feeding its matrix core
// (eight waves);
// schedule 2: ping-pong with A (K-contiguous) fetched in double-wide slabs,
// so every A load instruction reads whole 128-byte lines: A in a ring of 3
// double slabs, B in a ring of `stages` slabs (160 KiB for 256 x 256 x 32);
// B stored [N,K] (K-contiguous as well) in a ring of 2 double slabs.
#pragma once

#define GEMMEPI_TILES(X)         \
  X(0, 256, 256, 64, 2, 4, 2, 0) \
  X(1, 256, 256, 32, 2, 4, 4, 0) \
  X(2, 256, 128, 64, 2, 2, 3, 0) \
  X(3, 128, 128, 64, 2, 2, 3, 0) \
  X(4, 128, 64, 64, 2, 2, 3, 0)  \
  X(5, 64, 64, 64, 2, 2, 3, 0)   \
  X(6, 256, 256, 32, 2, 4, 4, 1) \
  X(7, 256, 128, 64, 4, 2, 3, 1) \
  X(8, 256, 256, 32, 2, 4, 4, 2)
