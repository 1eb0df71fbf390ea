// The tile configurations of the tiled MFMA GEMM, shared by the kernel
// instantiations and the host-side planner:
//   X(id, BM, BN, BK, waves along M, waves along N, LDS stages, schedule, MFMA)
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
// MFMA: 16 = v_mfma_f32_16x16x32, 32 = v_mfma_f32_32x32x16.
// Tile 9 is the 64 x 64 tile with 128-wide slabs (3 in flight, 96 KiB): for
// shapes whose workgroups walk a short K range on their own, where the bytes
// in flight per CU, not the MFMAs, set the pace (measured on the
// 1024 x 512 x 2048 GEMM split in 2: 7 % faster than tile 5; a ring of 8
// 64-wide slabs was no faster than tile 5).
#pragma once

#define GEMMEPI_TILES(X)              \
  X(0, 256, 256, 64, 2, 4, 2, 0, 16)  \
  X(1, 256, 256, 32, 2, 4, 4, 0, 16)  \
  X(2, 256, 128, 64, 2, 2, 3, 0, 16)  \
  X(3, 128, 128, 64, 2, 2, 3, 0, 32)  \
  X(4, 128, 64, 64, 2, 2, 3, 0, 32)   \
  X(5, 64, 64, 64, 2, 2, 3, 0, 32)    \
  X(6, 256, 256, 32, 2, 4, 4, 1, 16)  \
  X(7, 256, 128, 64, 4, 2, 3, 1, 16)  \
  X(8, 256, 256, 32, 2, 4, 4, 2, 16)  \
  X(9, 64, 64, 128, 2, 2, 4, 0, 32)
