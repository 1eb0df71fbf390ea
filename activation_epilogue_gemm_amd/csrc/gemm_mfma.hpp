// Tiled MFMA GEMM with an in-register epilogue, for gfx950 (MI355X).
//
//   out[M,N] = epilogue(A[M,K] . B + bias)
//
// The GEMM result never leaves the chip before the epilogue: bias add,
// activation, mask packing and bias-gradient reduction are applied to the
// fp32 accumulators, then each output element is rounded and written once.
// This is the fused sequence of the pages (the GEMM result stays in
// registers / on-chip memory and is combined with the bias there before a
// single write-back: "Fusing bias addition with matrix multiplication using
// nvmath-python", paragraph 2; ops-nn MatMul fusion article, section
// "Level 1: basic fusion"), designed here for CDNA4 rather than taken from
// those pages' hardware.
//
// Structure of one workgroup (WM x WN wavefronts of 64 lanes):
//   * the workgroup owns a BM x BN output tile; wave (wm, wn) owns a
//     (BM/WM) x (BN/WN) sub-tile made of 32x32 MFMA tiles;
//   * K is walked in slabs of BK.  Each slab of A [BM x BK] and of B is
//     fetched with 128-bit buffer loads that write straight into LDS (no
//     register staging) into a ring of NS stage buffers: while the MFMAs
//     consume slab kt, the loads of slabs kt+1 .. kt+NS-1 are in flight, so
//     the prefetch distance covers HBM latency even with one workgroup per
//     CU.  One barrier per slab.  Out-of-range rows, columns and k read as
//     zero through the buffer descriptor's range check;
//   * LDS rows are XOR-swizzled in 16-byte units so that the 128-bit
//     fragment reads (and the 64-bit transposing reads of a row-major [K,N]
//     B) hit distinct banks of the 64-bank LDS;
//   * v_mfma_f32_16x16x32_{f16,bf16} or v_mfma_f32_32x32x16_{f16,bf16}
//     (the tile's MFMA shape MT, MfmaShape below): exact products, fp32
//     accumulation.  The B fragment is passed as the instruction's first
//     operand and the A fragment as its second, so the accumulator holds the
//     transposed block: with MT = 16 lane l, element r of a 16x16 block is
//         row m = l % 16,   column n = 4*(l/16) + r,
//     with MT = 32 lane l, element r of a 32x32 block is
//         row m = l % 32,   column n = 8*(r/4) + 4*(l/32) + (r%4),
//     i.e. each lane owns one output row and runs of 4 consecutive columns,
//     which become 8-byte stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_tiles.h"

#include "kernels.h"

namespace gemmepi {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x4_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define GEMMEPI_LDS __attribute__((address_space(3)))

// Out-of-range voffset: larger than the descriptor's record count, so the
// buffer load returns zeros.
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kNumRecords = 0x7FFFFFFF;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  // gfx9 family descriptor word 3 (no swizzle, 32-bit data format).
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, kNumRecords, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Debug build (GEMMEPI_LDS_POISON=1), a race detector for the LDS rings:
// before a wave issues a global->LDS load, it fills the 1 KiB block that
// load will write with NaN bits (0xFFFF in fp16 and in bf16) and waits for
// those writes.  A wave that reads a block before the load into it has
// landed (a missing vmcnt wait or barrier) then reads NaN rather than the
// block's previous, plausible contents, and a refill that overtakes a
// reader of the previous contents hands it NaN as well; after the main loop
// the whole ring is poisoned again before the epilogue reuses it.  On
// integer inputs every such read turns the result wrong, where the release
// build would often compute the right result from stale data.
#ifndef GEMMEPI_LDS_POISON
#define GEMMEPI_LDS_POISON 0
#endif

__device__ __forceinline__ void poison_lds_blocks(uint32_t lds_addr, int blocks) {
  if constexpr (GEMMEPI_LDS_POISON != 0) {
    const u32x4 nan4 = {~0u, ~0u, ~0u, ~0u};
    for (int b = 0; b < blocks; ++b)
      *(GEMMEPI_LDS u32x4*)(GEMMEPI_LDS uint8_t*)(uintptr_t)(lds_addr + 1024u * b +
                                                             16u * (threadIdx.x & 63u)) = nan4;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
}

// 16 bytes per lane from a buffer straight into LDS: lane L's data lands at
// LDS byte address lds_addr + 16 L (lds_addr must be wave-uniform; it goes
// to M0).  Written as inline assembly on purpose: the compiler then does not
// see an LDS write in flight, and does not make every later LDS read wait
// for it (it cannot prove that the transposing reads of the other stage do
// not alias it).  The caller orders these writes with wait_loads() and a
// barrier before any wave reads the stage.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr,
                                                  uint32_t off) {
  poison_lds_blocks(lds_addr, 1);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(off), "s"(r), "s"(lds_addr)
               : "memory");
}

// Wait until at most N vector memory operations of this wave are still in
// flight (loads complete in issue order, so every older buffer->LDS load,
// LDS write included, has then landed).
// f(integral_constant<int, i>) for i = 0 .. N-1: compile-time indices for
// the accumulator array whatever the unroller decides about a large body
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// G (1..4) loads of 16 bytes per lane from one buffer into G consecutive
// 1 KiB LDS blocks starting at lds_addr, with a single write of M0: load g
// carries the immediate offset 1024 g, which the hardware adds to both the
// LDS and the global address, so voff[g] must be the global offset of block
// g minus 1024 g (or an out-of-range offset, which reads zero).
// The output tile's 16-byte row stores carry the non-temporal hint (1) or
// are ordinary stores (0).  The output is written once and not read again
// by the kernel; with the hint it displaces less of the operands' cached
// panels.  Measured inside the benchmark suite (cold operands, one box,
// runs alternated): the FFN GEMMs 1.5-4 % faster, C3 bf16 1 %, C4 0.2 %,
// C3 fp16 0.3 % slower (within its run-to-run spread).
#ifndef GEMMEPI_NT_OUT
#define GEMMEPI_NT_OUT 1
#endif

#ifndef GEMMEPI_M0_GROUPS
#define GEMMEPI_M0_GROUPS 0
#endif
template <int G>
__device__ __forceinline__ void buffer_load16_lds_group(__amdgpu_buffer_rsrc_t r, uint32_t lds_addr,
                                                        const uint32_t* voff) {
  static_assert(G >= 1 && G <= 4, "one M0 covers at most 4 KiB of immediate offsets");
  poison_lds_blocks(lds_addr, G);
  if constexpr (G == 1) {
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff[0]), "s"(r), "s"(lds_addr)
                 : "memory");
  } else if constexpr (G == 2) {
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %0, %2, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen offset:1024 lds"
        :
        : "v"(voff[0]), "v"(voff[1]), "s"(r), "s"(lds_addr)
        : "memory");
  } else if constexpr (G == 3) {
    asm volatile(
        "s_mov_b32 m0, %4\n\t"
        "buffer_load_dwordx4 %0, %3, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %3, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen offset:2048 lds"
        :
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "s"(r), "s"(lds_addr)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 m0, %5\n\t"
        "buffer_load_dwordx4 %0, %4, 0 offen lds\n\t"
        "buffer_load_dwordx4 %1, %4, 0 offen offset:1024 lds\n\t"
        "buffer_load_dwordx4 %2, %4, 0 offen offset:2048 lds\n\t"
        "buffer_load_dwordx4 %3, %4, 0 offen offset:3072 lds"
        :
        : "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(r), "s"(lds_addr)
        : "memory");
  }
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)(uintptr_t)(const GEMMEPI_LDS void*)p;
}

template <typename T> struct Frag;
template <> struct Frag<_Float16> { using type = f16x8; };
template <> struct Frag<__bf16> { using type = bf16x8; };

__device__ __forceinline__ f32x16 mfma_op(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_op(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_op(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_op(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The MFMA shape of a tile: MT x MT output blocks, v_mfma_f32_32x32x16
// (MT = 32) or v_mfma_f32_16x16x32 (MT = 16); every part of the kernel is
// written for both, and the tile table picks one per tile.  The 16x16x32
// form spends less energy per FLOP (in a bare MFMA loop shaped like the
// 256 x 256 tile it holds a ~14 % higher clock at the power limit); measured
// interleaved on one box against 32x32x16 it ran the large tiles 1-11 %
// faster and the 64 x 64 tile of the 1024 x 512 x 2048 GEMM 6 % slower.
template <int MT> struct AccOf;
template <> struct AccOf<32> { using type = f32x16; };
template <> struct AccOf<16> { using type = f32x4; };
template <int MT>
struct MfmaShape {
  static_assert(MT == 16 || MT == 32, "MFMA shape");
  static constexpr int kAccN = MT * MT / 64;       // accumulator floats per lane per block
  static constexpr int kLaneGroups = 64 / MT;      // lane groups l / MT
  static constexpr int kKStep = 8 * kLaneGroups;   // k depth of one MFMA
  static constexpr int kColStride = 4 * kLaneGroups;  // columns between a lane's 4-column groups
  using AccBlock = typename AccOf<MT>::type;
};

// 4 consecutive-k values of one column from a row-major [K,N] LDS tile:
// within each group of 16 lanes, lane (4*h + q) points at row h, columns
// 4q..4q+3 of a 4 x 16 block; after the transposing read lane i holds
// column i of the block (rows 0..3).
__device__ __forceinline__ u32x2 lds_read_tr(const uint8_t* p, _Float16) {
  fp16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((GEMMEPI_LDS fp16x4_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}
__device__ __forceinline__ u32x2 lds_read_tr(const uint8_t* p, __bf16) {
  bf16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((GEMMEPI_LDS bf16x4_t*)(p));
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ float to_f32(_Float16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ _Float16 from_f32<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// Two fp32 values -> one 32-bit word of two 16-bit values (round to nearest
// even; the low half is `a`).
__device__ __forceinline__ uint32_t pack2(float a, float b, _Float16) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint32_t pack2(float a, float b, __bf16) {
  bf16x2 h = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Exact (erf) GELU: gelu(z) = z Phi(z) = 0.5 z (1 + erf(z / sqrt 2)).
// erf is evaluated with Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (|error| <= 1.5e-7 for x >= 0):
//   erf(x) = 1 - q,  q = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
//   t = 1 / (1 + p x),
// taken at x = |z| / sqrt 2.  Both functions below use
//   h = Phi(-|z|) = erfc(|z| / sqrt 2) / 2 = q / 2,
// computed directly (not as 1 - something), so the negative branch keeps
// full relative accuracy.  The halving is folded into the coefficients,
// and with u = |z| sqrt(log2(e) / 2) the exponential exp(-z^2 / 2) is
// 2^(-u^2) and p x = (p / sqrt(log2 e)) u.
struct ErfcHalf {
  float h;  // Phi(-|z|)
  float e;  // exp(-z^2 / 2)
};
__device__ __forceinline__ ErfcHalf erfc_half(float z) {
  const float u = fabsf(z) * 0.8493218002880191f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2727374808792225f, u, 1.0f));
  float poly = fmaf(0.5307027145f, t, -0.7265760135f);
  poly = fmaf(poly, t, 0.7107068705f);
  poly = fmaf(poly, t, -0.142248368f);
  poly = fmaf(poly, t, 0.127414796f);
  const float e = __builtin_amdgcn_exp2f(-(u * u));
  return {poly * t * e, e};
}
// z >= 0: z Phi(z) = z - z h,   z < 0: z Phi(z) = z h = -|z| h,
// so gelu(z) = max(z, 0) - |z| h: 11 VALU operations and two
// transcendentals per element.
__device__ __forceinline__ float gelu_erf(float z) {
  return fmaf(-fabsf(z), erfc_half(z).h, fmaxf(z, 0.0f));
}
// gelu'(z) = Phi(z) + z phi(z), phi(z) = exp(-z^2 / 2) / sqrt(2 pi): the
// exponential of phi is the one the erf evaluation already computed.
__device__ __forceinline__ float gelu_grad(float z) {
  const ErfcHalf r = erfc_half(z);
  const float Phi = z >= 0.0f ? 1.0f - r.h : r.h;
  return fmaf(z * 0.3989422804014327f, r.e, Phi);
}

// blockIdx -> output tile.  The hardware hands consecutive workgroup ids
// to the 8 XCDs round-robin (id % 8), and each XCD has its own L2.
//  * Chip-block raster (sb_m > 0): the tiles run in rounds of sb_m x sb_n
//    (one per CU), rounds ordered along N; inside a round XCD x takes a
//    (sb_m / xcd_m) x (sb_n / xcd_n) sub-block.  Concurrent tiles of one XCD
//    share their A and B panels in its L2, and the whole chip's concurrent
//    tiles touch only sb_m + sb_n panels, which the XCDs share through the
//    Infinity Cache instead of each reading them from HBM.
//  * Otherwise (shapes that do not divide): with xcd_remap each XCD walks a
//    contiguous run of the tile order, grouped by `group_m` tile rows.
//  Tile id `bid` of `nb` (the workgroup id, or its tile under split-K).
__device__ __forceinline__ void tile_coords(const GemmArgs& p, int bid, int nb, int& tm, int& tn) {
  if (p.sb_m > 0) {
    const int x = bid & 7;                 // XCD of this workgroup
    const int j = bid >> 3;                // its index on that XCD
    const int per_xcd = (p.sb_m * p.sb_n) >> 3;
    const int round = j / per_xcd, slot = j - round * per_xcd;
    const int sub_n = p.sb_n / p.xcd_n;
    const int rounds_n = p.tiles_n / p.sb_n;
    const int rm = round / rounds_n, rn = round - rm * rounds_n;
    const int xm = x / p.xcd_n, xn = x - xm * p.xcd_n;
    tm = rm * p.sb_m + xm * (p.sb_m / p.xcd_m) + slot / sub_n;
    tn = rn * p.sb_n + xn * sub_n + slot % sub_n;
    return;
  }
  if (p.xcd_remap) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int per_group = p.group_m * p.tiles_n;
  const int g = bid / per_group;
  const int first_m = g * p.group_m;
  const int gsz = min(p.tiles_m - first_m, p.group_m);
  const int r = bid - g * per_group;
  tm = first_m + r % gsz;
  tn = r / gsz;
}

template <int BM, int BN, int BK, int WM, int WN, int NS, int MT>
struct GemmTile {
  static constexpr int kMfma = MT;
  static constexpr int NT = WM * WN * 64;
  static constexpr int NW = WM * WN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int FM = WTM / kMfma, FN = WTN / kMfma;
  static constexpr int KCH = BK / 8;                 // 16 B chunks per K-contiguous row
  static constexpr int NCH = BN / 8;                 // 16 B chunks per N-contiguous row
  static constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_CH = A_BYTES / (NT * 16);   // 1 KiB load blocks per wave (A)
  static constexpr int B_CH = B_BYTES / (NT * 16);   // 1 KiB load blocks per wave (B)
  static constexpr int A_RPB = 1024 / (BK * 2);      // K-contiguous rows per 1 KiB block
  static constexpr int B_RPB = 1024 / (BN * 2);      // N-contiguous rows per 1 KiB block
  // rows sharing one 256-byte bank line
  static constexpr int RPK = (BK * 2 >= 256) ? 1 : 256 / (BK * 2);
  static constexpr int RPN = (BN * 2 >= 256) ? 1 : 256 / (BN * 2);
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32-row/32-column blocks");
  static_assert(BK % 16 == 0 && BK >= 32, "BK");
  static_assert(A_BYTES % (NT * 16) == 0 && B_BYTES % (NT * 16) == 0, "load split");
  static_assert(64 % KCH == 0 && 64 % NCH == 0 && BN * 2 <= 1024, "load split");
  static constexpr int LPS = A_CH + B_CH;            // load instructions per slab per wave
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS");
  static_assert((NS - 1) * LPS < 64, "vmcnt range");
  // epilogue: the output tile [BM][BN] and the per-wave-row column sums of
  // the bias gradient, [WM][BN] fp32, reuse the staging ring
  // ([WN][BM][2] fp64 partial row sums for the norm epilogue)
  static constexpr int OUT_BYTES = BM * BN * 2;
  static constexpr int RED_BYTES = WM * BN * 4 > BM * WN * 16 ? WM * BN * 4 : BM * WN * 16;
  // the tile's bias slice (BM or BN fp32), or for the single-pass norm its
  // bias, gamma and beta slices (3 BN fp32), and a flag word
  static constexpr int BIAS_BYTES = (BM > 3 * BN ? BM : 3 * BN) * 4 + 16;
  static constexpr int EPI_BYTES = OUT_BYTES + RED_BYTES + BIAS_BYTES;
  static constexpr int SMEM = NS * STAGE > EPI_BYTES ? NS * STAGE : EPI_BYTES;
  static_assert(SMEM <= 160 * 1024, "LDS");
  static_assert(NT % (BN / 8) == 0 && BM % (NT / (BN / 8)) == 0, "epilogue copy split");

  // 16 B-chunk swizzle of a K-contiguous row r (A, or B stored [N,K])
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPK) % KCH; }
  // 16 B-chunk swizzle of row r of the staged output tile
  static __device__ __forceinline__ int swz_o(int r) { return r % (BN / 8); }
  // 16 B-chunk swizzle of an N-contiguous row kr (B stored [K,N]).  With
  // 16x16x32 MFMAs, one transposing read of 32 lanes covers k rows h and
  // h + 8 (h = 0..3) at the same columns; the swizzle gives those 8 rows 8
  // distinct even chunk offsets within a 256-byte bank line (4 per line and
  // two lines when 2 rows share one), so the 32 lanes hit 64 distinct banks.
  // It repeats every 16 rows.
  static __device__ __forceinline__ int swz_n(int kr) {
    if constexpr (kMfma == 32) return (4 * (kr / RPN)) % NCH;
    else return 2 * ((kr / RPN) % (4 / RPN)) + (8 / RPN) * ((kr / 8) % 2);
  }
};

// A workgroup barrier that the instruction scheduler may not move any
// instruction across (the ping-pong phases must stay separated).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int NS, bool BT, int SCHED, int MT>
__global__ void __launch_bounds__(WM * WN * 64, 1) gemm_kernel(const GemmArgs p) {
  using G = GemmTile<BM, BN, BK, WM, WN, NS, MT>;
  using Shape = MfmaShape<MT>;
  constexpr int kMfma = MT;
  constexpr int kAccN = Shape::kAccN, kKStep = Shape::kKStep, kColStride = Shape::kColStride;
  using AccBlock = typename Shape::AccBlock;
  using V8 = typename Frag<T>::type;
  constexpr int NT = G::NT, NW = G::NW, WTM = G::WTM, WTN = G::WTN, FM = G::FM, FN = G::FN;
  constexpr int KCH = G::KCH, NCH = G::NCH, A_CH = G::A_CH, B_CH = G::B_CH;

  // schedule 2 keeps A in a ring of 3 double-wide slabs and B in a ring of
  // NS slabs
  constexpr int RING2 = 3 * BM * (2 * BK) * 2 + NS * G::B_BYTES;
  constexpr int SMEM_BYTES = (SCHED == 2 && RING2 > G::SMEM) ? RING2 : G::SMEM;
  static_assert(SMEM_BYTES <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SMEM_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int ntiles = p.tiles_m * p.tiles_n;
  const int split = p.splits > 1 ? (int)blockIdx.x / ntiles : 0;
  const int tile_id = (int)blockIdx.x - split * ntiles;
  int tm, tn;
  tile_coords(p, tile_id, ntiles, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- slab loads: 128-bit buffer loads straight into LDS ----------------
  // Each load instruction of a wave fills one contiguous 1 KiB block of an
  // LDS stage (lane L -> bytes 16L..16L+15).  The swizzled layout is made by
  // choosing which global chunk each lane fetches: the lane that owns LDS
  // chunk slot `phys` of row r fetches logical chunk phys ^ swizzle(r).
  // Offsets are relative to the slab's first k; an offset with bit 31 set
  // is past the 2^31 - 1 byte buffer range and reads zero.  tail_bits has
  // bit j set when load j lies beyond K in the last slab.
  const int KT = (K + BK - 1) / BK;
  const int k_last = (KT - 1) * BK;
  // this workgroup's slabs [kt_begin, kt_end): all of K, or one split of it
  const int kt_begin = p.splits > 1 ? split * p.kt_split : 0;
  const int kt_end = p.splits > 1 ? min(KT, kt_begin + p.kt_split) : KT;
  uint32_t tail_bits = 0;
  uint32_t a_off[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int blk = i * NW + wave;
    const int r = blk * G::A_RPB + lane / KCH;
    const int kc = (lane % KCH) ^ G::swz_k(r);
    a_off[i] = (m0 + r < M) ? (uint32_t)((r * p.lda + kc * 8) * 2) : kOOB;
    if (k_last + kc * 8 >= K) tail_bits |= 1u << i;
  }
  uint32_t b_off[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int blk = i * NW + wave;
    if constexpr (BT) {  // B stored [N,K]: rows are n
      const int r = blk * G::A_RPB + lane / KCH;
      const int kc = (lane % KCH) ^ G::swz_k(r);
      b_off[i] = (n0 + r < N) ? (uint32_t)((r * p.ldb + kc * 8) * 2) : kOOB;
      if (k_last + kc * 8 >= K) tail_bits |= 1u << (A_CH + i);
    } else {             // B stored [K,N]: rows are k
      const int kr = blk * G::B_RPB + lane / NCH;
      const int nc = (lane % NCH) ^ G::swz_n(kr);
      b_off[i] = (n0 + nc * 8 < N) ? (uint32_t)((kr * p.ldb + nc * 8) * 2) : kOOB;
      if (k_last + kr >= K) tail_bits |= 1u << (A_CH + i);
    }
  }

  const uint8_t* Abase = (const uint8_t*)p.A + (size_t)m0 * p.lda * 2;
  const uint8_t* Bbase = BT ? (const uint8_t*)p.B + (size_t)n0 * p.ldb * 2
                            : (const uint8_t*)p.B + (size_t)n0 * 2;

  // load j (0 <= j < LPS) of this wave's share of slab kt into stage st:
  // j < A_CH are A blocks, the rest B blocks.  A slab kt >= kt_end is a
  // placeholder: its loads read nothing and write zeros into a stage that
  // no later slab uses, which keeps the count of loads per slab uniform.
  auto issue_one = [&](int kt, uint8_t* st, int j) {
    const uint32_t st_addr = __builtin_amdgcn_readfirstlane(lds_addr_of(st));
    const bool none = kt >= kt_end;
    const int k0 = none ? 0 : kt * BK;
    // branch-free: bit 31 from "placeholder" (uniform) or "beyond K" (lane)
    const uint32_t kill = (none ? kOOB : 0u) | ((kt == KT - 1 ? (tail_bits >> j) & 1u : 0u) << 31);
    if (j < A_CH) {
      const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase + (size_t)k0 * 2);
      buffer_load16_lds(rA, st_addr + (j * NW + wave) * 1024, a_off[j] | kill);
    } else {
      const int i = j - A_CH;
      const __amdgpu_buffer_rsrc_t rB =
          BT ? make_rsrc(Bbase + (size_t)k0 * 2) : make_rsrc(Bbase + (size_t)k0 * p.ldb * 2);
      buffer_load16_lds(rB, st_addr + G::A_BYTES + (i * NW + wave) * 1024, b_off[i] | kill);
    }
  };
  auto issue = [&](int kt, uint8_t* st) {
#pragma unroll
    for (int j = 0; j < G::LPS; ++j) issue_one(kt, st, j);
  };

  AccBlock acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < kAccN; ++e) acc[i][j][e] = 0.0f;

  const int lrow = lane % kMfma;  // row (A) / column (B) within an MFMA block
  const int lgrp = lane / kMfma;  // the lane's 8-wide k group of an MFMA step

  // A fragment (rows of A) and B fragment (columns of B) of k step ks of
  // the slab at sA.  The per-lane LDS offsets are computed once: fragment fm
  // (fn) and k step ks only add constants, because the swizzles repeat
  // every 32 K-contiguous rows and every 16 N-contiguous k rows.
  constexpr int KS = BK / kKStep;
  static_assert(BK % kKStep == 0, "BK must be whole MFMA k steps");
  static_assert((kMfma / G::RPK) % KCH == 0, "A/B_T swizzle must repeat every block of rows");
  static_assert(kMfma == 16 ? (BT || G::RPN <= 2) : (4 * (16 / G::RPN)) % NCH == 0,
                "B swizzle must repeat every 16 k rows");
  uint32_t a_lds[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = wm * WTM + lrow;
    a_lds[ks] = (uint32_t)(r * BK * 2 + (((ks * (kKStep / 8) + lgrp) ^ G::swz_k(r)) << 4));
  }
  constexpr int BL = BT ? KS : 2 * FN;
  uint32_t b_lds[BL];
  if constexpr (BT) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = wn * WTN + lrow;
      b_lds[ks] = (uint32_t)(G::A_BYTES + r * BK * 2 + (((ks * (kKStep / 8) + lgrp) ^ G::swz_k(r)) << 4));
    }
  } else {
    // two transposing reads per fragment: lane (g, i) = (lane / 16, lane % 16)
    // reads k rows 8 (g / CH) + i / 4 (+ 4), columns 16 (g % CH) + 4 (i % 4) ..,
    // CH = kMfma / 16 column halves per block (a 16-lane group then holds
    // column i of its 16 columns at 8 consecutive k)
    constexpr int CH = kMfma / 16;
    const int g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int ncol = wn * WTN + fn * kMfma + (g % CH) * 16 + (i & 3) * 4;
      const int nc = ncol >> 3, nb = (ncol & 7) * 2;
      const int kr0 = (g / CH) * 8 + (i >> 2), kr1 = kr0 + 4;
      b_lds[2 * fn] = (uint32_t)(G::A_BYTES + kr0 * BN * 2 + ((nc ^ G::swz_n(kr0)) << 4) + nb);
      b_lds[2 * fn + 1] = (uint32_t)(G::A_BYTES + kr1 * BN * 2 + ((nc ^ G::swz_n(kr1)) << 4) + nb);
    }
  }
  auto read_a = [&](const uint8_t* sA, int ks, int fm) -> V8 {
    return *(const V8*)(sA + a_lds[ks] + fm * kMfma * BK * 2);
  };
  auto read_b = [&](const uint8_t* sA, int ks, int fn) -> V8 {
    if constexpr (BT) {
      return *(const V8*)(sA + b_lds[ks] + fn * kMfma * BK * 2);
    } else {
      const u32x2 lo = lds_read_tr(sA + b_lds[2 * fn] + ks * kKStep * BN * 2, T{});
      const u32x2 hi = lds_read_tr(sA + b_lds[2 * fn + 1] + ks * kKStep * BN * 2, T{});
      const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
      return __builtin_bit_cast(V8, w);
    }
  };

  // MFMAs [lo, hi) of a slab's KS x FM x FN (k step major), on registers;
  // between(q) is placed after MFMA q.  Within a k step the blocks are
  // visited in a snake: along fn for even fm, back for odd fm, so that two
  // consecutive MFMAs always share one source fragment (the A fragment
  // within a row, the B fragment across a row change).  Each accumulator
  // block still sums its k steps in order, so results do not change; fewer
  // operand changes cost less power, and the power-limited clock rose with
  // it (interleaved, one box: C3 +0.9-2.0 %, C4 +1.0-1.6 %, the FFN GEMMs
  // +0.2-0.7 % against rows always taken along fn).
  auto mfma_range_with = [&](const V8 (&af)[KS][FM], const V8 (&bf)[KS][FN], int lo, int hi,
                             auto&& between) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int fn = (fm & 1) ? FN - 1 - f : f;
          const int q = (ks * FM + fm) * FN + f;
          if (q >= lo && q < hi) {
            acc[fm][fn] = mfma_op(bf[ks][fn], af[ks][fm], acc[fm][fn]);
            between(q);
          }
        }
  };
  auto mfma_range = [&](const V8 (&af)[KS][FM], const V8 (&bf)[KS][FN], int lo, int hi) {
    mfma_range_with(af, bf, lo, hi, [&](int) {});
  };
  // A compute phase of the ping-pong schedules issues the slab's kNMfma
  // MFMAs from registers between two barriers.  (Issuing its last 2-8 after
  // the closing barrier, so that they would cover the barrier's hand-over,
  // measured 1-12 % slower on every large shape.)
  constexpr int kNMfma = KS * FM * FN;

  auto compute = [&](const uint8_t* sA) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      V8 af[FM], bf[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) af[fm] = read_a(sA, ks, fm);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) bf[fn] = read_b(sA, ks, fn);
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int fn = (fm & 1) ? FN - 1 - f : f;  // the snake of mfma_range_with
          acc[fm][fn] = mfma_op(bf[fn], af[fm], acc[fm][fn]);
        }
    }
  };

  if constexpr (SCHED == 2) {
    // Ping-pong (as schedule 1) with A fetched in double-wide slabs.  A is
    // K-contiguous, and a 32-wide slab gives each load instruction 16 rows x
    // 64 bytes, half a 128-byte line per row; a 64-wide A slab gives 8 rows
    // x 128 bytes.  A lives in a ring of 3 double slabs (pair q = slabs 2q,
    // 2q + 1 of the range), B in a ring of 4 slabs, 160 KiB together.  The
    // load phase of slab i issues B slab i + 3 and, in the second slab of a
    // pair, A pair q + 2 (see the loop).  B stored [N,K] is fetched in pairs
    // too, in a ring of 2 (below).  The compute phases issue nothing but
    // MFMAs.
    static_assert(SCHED != 2 || NS == 4, "schedule 2 issues B three slabs ahead");
    constexpr int BK2 = 2 * BK, KCH2 = BK2 / 8, RPB2 = 1024 / (BK2 * 2);
    constexpr int RPK2 = (BK2 * 2 >= 256) ? 1 : 256 / (BK2 * 2);
    constexpr int A2_BYTES = BM * BK2 * 2;
    constexpr int A2_CH = A2_BYTES / (NT * 16);  // A loads per wave per pair
    constexpr int NA = 3;
    static_assert(A2_BYTES % (NT * 16) == 0 && 64 % KCH2 == 0, "load split");
    static_assert((kMfma / RPK2) % KCH2 == 0, "A swizzle must repeat every block of rows");
    static_assert(A2_CH + 2 * G::B_CH < 64, "vmcnt range");
    auto swz2 = [](int r) { return (r / RPK2) % KCH2; };
    uint8_t* const a_ring = smem;
    uint8_t* const b_ring = smem + NA * A2_BYTES;
    // B stored [N,K] is K-contiguous as well and is then also fetched in
    // double-wide slabs, in a ring of 2 pairs: pair q + 1 goes into the
    // stage of pair q - 1 in the first load phase after that stage is free
    // (that of slab 2q) and is waited for in the next one (slab 2q + 1).
    // Its loads have half the time to land that A's have, but every B load
    // instruction then reads 8 whole 128-byte lines instead of 16 halves
    // (measured on the [N,K] form of the 65536 x 8192 x 16384 GEMM: +10 %).
    constexpr bool BPAIR = BT;
    constexpr int B2_BYTES = BN * BK2 * 2;
    constexpr int B2_CH = B2_BYTES / (NT * 16);  // B loads per wave per pair
    static_assert(!BPAIR || (B2_BYTES % (NT * 16) == 0 && NA * A2_BYTES + 2 * B2_BYTES <= SMEM_BYTES),
                  "B pair ring");
    static_assert(!BPAIR || A2_CH + B2_CH < 64, "vmcnt range");
    // Each wave's loads of one slab (or pair) fill GS consecutive 1 KiB LDS
    // blocks per M0 write (buffer_load16_lds_group): load j of the wave fills
    // block wave * CH + j and carries the immediate offset 1024 (j % GS).  The
    // descriptors start kShift bytes below the operand so that every offset
    // stays non-negative: voff = global offset + kShift - 1024 (j % GS).
    // (With GS = 1, load j fills block j * NW + wave, one M0 write per load.)
    constexpr int GS_A = GEMMEPI_M0_GROUPS ? (A2_CH < 4 ? A2_CH : 4) : 1;
    constexpr int GS_B = GEMMEPI_M0_GROUPS ? (G::B_CH < 4 ? G::B_CH : 4) : 1;
    constexpr int GS_BP = GEMMEPI_M0_GROUPS ? (B2_CH < 4 ? B2_CH : 4) : 1;
    static_assert(A2_CH % GS_A == 0 && G::B_CH % GS_B == 0 && (!BPAIR || B2_CH % GS_BP == 0),
                  "load groups");
    auto blk_of = [&](int j, int ch, int gs) { return gs > 1 ? wave * ch + j : j * NW + wave; };
    constexpr uint32_t kShift = 3072;
    uint32_t b2_off[B2_CH];
    int b2_k[B2_CH];
    uint32_t b2_lds[2][KS];
    if constexpr (BPAIR) {
#pragma unroll
      for (int i = 0; i < B2_CH; ++i) {
        const int blk = blk_of(i, B2_CH, GS_BP);
        const int r = blk * RPB2 + lane / KCH2;
        const int kc = (lane % KCH2) ^ swz2(r);
        b2_off[i] = (n0 + r < N) ? (uint32_t)((r * p.ldb + kc * 8) * 2) + kShift - 1024u * (i % GS_BP)
                                 : kOOB;
        b2_k[i] = kc * 8;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int r = wn * WTN + lrow;
          const int chunk = h * (BK / 8) + ks * (kKStep / 8) + lgrp;
          b2_lds[h][ks] = (uint32_t)(r * BK2 * 2 + ((chunk ^ swz2(r)) << 4));
        }
    }
    // B stored [K,N] in single slabs: offsets of this wave's blocks, and
    // which of them lie beyond K in the last slab
    uint32_t bs_off[G::B_CH];
    uint32_t bs_tail = 0;
    if constexpr (!BPAIR) {
#pragma unroll
      for (int i = 0; i < G::B_CH; ++i) {
        const int blk = blk_of(i, G::B_CH, GS_B);
        const int kr = blk * G::B_RPB + lane / NCH;
        const int nc = (lane % NCH) ^ G::swz_n(kr);
        bs_off[i] = (n0 + nc * 8 < N) ? (uint32_t)((kr * p.ldb + nc * 8) * 2) + kShift - 1024u * (i % GS_B)
                                      : kOOB;
        if (k_last + kr >= K) bs_tail |= 1u << i;
      }
    }
    uint32_t a2_off[A2_CH];
    int a2_k[A2_CH];
#pragma unroll
    for (int i = 0; i < A2_CH; ++i) {
      const int blk = blk_of(i, A2_CH, GS_A);
      const int r = blk * RPB2 + lane / KCH2;
      const int kc = (lane % KCH2) ^ swz2(r);
      a2_off[i] = (m0 + r < M) ? (uint32_t)((r * p.lda + kc * 8) * 2) + kShift - 1024u * (i % GS_A) : kOOB;
      a2_k[i] = kc * 8;
    }
    const int k_stop = min(K, kt_end * BK);  // A columns at or past it read zero
    // all loads of A pair q into A stage `stage`
    auto issue_a2 = [&](int q, int stage) {
      const int slab0 = kt_begin + 2 * q;
      const bool none = slab0 >= kt_end;
      const int k0 = none ? 0 : slab0 * BK;
      const uint32_t st_addr =
          __builtin_amdgcn_readfirstlane(lds_addr_of(a_ring + stage * A2_BYTES));
      const __amdgpu_buffer_rsrc_t rA = make_rsrc(Abase + (size_t)k0 * 2 - kShift);
      static_for<A2_CH / GS_A>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        uint32_t v[GS_A];
#pragma unroll
        for (int t = 0; t < GS_A; ++t) {
          const int j = g * GS_A + t;
          v[t] = (none || k0 + a2_k[j] >= k_stop) ? kOOB : a2_off[j];
        }
        buffer_load16_lds_group<GS_A>(rA, st_addr + blk_of(g * GS_A, A2_CH, GS_A) * 1024, v);
      });
    };
    // all loads of B pair q (B stored [N,K]) into B pair stage `stage`
    auto issue_bp = [&](int q, int stage) {
      const int slab0 = kt_begin + 2 * q;
      const bool none = slab0 >= kt_end;
      const int k0 = none ? 0 : slab0 * BK;
      const uint32_t st_addr =
          __builtin_amdgcn_readfirstlane(lds_addr_of(b_ring + stage * B2_BYTES));
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + (size_t)k0 * 2 - kShift);
      static_for<(BPAIR ? B2_CH : GS_BP) / GS_BP>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        uint32_t v[GS_BP];
#pragma unroll
        for (int t = 0; t < GS_BP; ++t) {
          const int j = g * GS_BP + t;
          v[t] = (none || k0 + b2_k[j] >= k_stop) ? kOOB : b2_off[j];
        }
        buffer_load16_lds_group<GS_BP>(rB, st_addr + blk_of(g * GS_BP, B2_CH, GS_BP) * 1024, v);
      });
    };
    // all loads of B slab kt (B stored [K,N]) into B stage `stage`
    auto issue_b2 = [&](int kt, int stage) {
      const bool none = kt >= kt_end;
      const int k0 = none ? 0 : kt * BK;
      const bool tail = kt == KT - 1;
      const uint32_t st_addr =
          __builtin_amdgcn_readfirstlane(lds_addr_of(b_ring + stage * G::B_BYTES));
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(Bbase + (size_t)k0 * p.ldb * 2 - kShift);
      static_for<(BPAIR ? GS_B : G::B_CH) / GS_B>([&](auto g_c) {
        constexpr int g = decltype(g_c)::value;
        uint32_t v[GS_B];
#pragma unroll
        for (int t = 0; t < GS_B; ++t) {
          const int j = g * GS_B + t;
          v[t] = (none || (tail && ((bs_tail >> j) & 1u))) ? kOOB : bs_off[j];
        }
        buffer_load16_lds_group<GS_B>(rB, st_addr + blk_of(g * GS_B, G::B_CH, GS_B) * 1024, v);
      });
    };
    uint32_t a2_lds[2][KS];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int r = wm * WTM + lrow;
        const int chunk = h * (BK / 8) + ks * (kKStep / 8) + lgrp;
        a2_lds[h][ks] = (uint32_t)(r * BK2 * 2 + ((chunk ^ swz2(r)) << 4));
      }
    if constexpr (BPAIR) {
      // prologue: A pair 0, B pair 0, A pair 1; then wait for pair 0
      issue_a2(0, 0);
      issue_bp(0, 0);
      issue_a2(1, 1);
      wait_vmcnt<A2_CH>();
    } else {
    // prologue, in this order (the waits count on it): A pair 0, B slabs 0
    // and 1, A pair 1, B slab 2; then wait for slab 0
    issue_a2(0, 0);
    issue_b2(kt_begin, 0);
    issue_b2(kt_begin + 1, 1);
    issue_a2(1, 1);
    issue_b2(kt_begin + 2, 2);
    wait_vmcnt<G::B_CH + A2_CH + G::B_CH>();
    }
    __syncthreads();
    const int grp = wave >> 2;
    if (grp == 1) phase_barrier();
    const int npairs = (kt_end - kt_begin + 1) / 2;  // an odd range ends in a zero slab
    int a_cur = 0;                                   // A stage of pair q
    for (int q = 0; q < npairs; ++q) {
      static_for<2>([&](auto h_c) {
        constexpr int h = decltype(h_c)::value;
        const int i = 2 * q + h;  // slab index in the range
        const uint8_t* sa = a_ring + a_cur * A2_BYTES;
        const uint8_t* sb = b_ring + (i & 3) * G::B_BYTES - G::A_BYTES;
        const uint8_t* sbp = b_ring + (q & 1) * B2_BYTES;
        V8 af[KS][FM], bf[KS][FN];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int fm = 0; fm < FM; ++fm)
            af[ks][fm] = *(const V8*)(sa + a2_lds[h][ks] + fm * kMfma * BK2 * 2);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            if constexpr (BPAIR)
              bf[ks][fn] = *(const V8*)(sbp + b2_lds[h][ks] + fn * kMfma * BK2 * 2);
            else
              bf[ks][fn] = read_b(sb, ks, fn);
          }
        }
        // The load phase also issues this wave's loads of B slab i + 3 and,
        // in the second slab of a pair, of A pair q + 2, after its fragment
        // reads.  Each load written straight to LDS holds up the issuing
        // wave for ~25 cycles; here that wave would otherwise idle at the
        // barrier, while in the compute phase it delayed the MFMAs.  The
        // stages are free: slab i - 1 and pair q - 1 were last read in the
        // other group's load phase before the last barrier.  A load issued
        // in load phase s is waited for two load phases later, so at this
        // wait the loads of this phase and the previous one may stay in
        // flight (between them one A pair and two B slabs).
        const int a_next = (a_cur + 2 >= NA) ? a_cur + 2 - NA : a_cur + 2;
        if constexpr (BPAIR) {
          // first slab of pair q: B pair q + 1 into the stage of pair q - 1;
          // second slab: A pair q + 2.  The wait of the second slab leaves
          // only that A pair in flight, so B pair q + 1 and A pair q + 1
          // have landed before slab 2q + 2 is read.
          if constexpr (h == 0) {
            issue_bp(q + 1, (q + 1) & 1);
            wait_vmcnt<A2_CH + B2_CH>();
          } else {
            issue_a2(q + 2, a_next);
            wait_vmcnt<A2_CH>();
          }
        } else {
        if constexpr (h == 1) {
          issue_a2(q + 2, a_next);
        }
        issue_b2(kt_begin + i + 3, (i + 3) & 3);
        wait_vmcnt<A2_CH + 2 * G::B_CH>();
        }
        phase_barrier();
        mfma_range(af, bf, 0, kNMfma);
        phase_barrier();
      });
      a_cur = (a_cur + 1 == NA) ? 0 : a_cur + 1;
    }
    if (grp == 0) phase_barrier();
    wait_vmcnt<0>();
    __syncthreads();
  } else {
  // prologue: the first NS-1 slabs (or placeholders) in flight, wait for the first
#pragma unroll
  for (int s = 0; s < NS - 1; ++s) issue(kt_begin + s, smem + s * G::STAGE);
  wait_vmcnt<(NS - 2) * G::LPS>();
  __syncthreads();
  int cur = 0;                      // stage of slab kt
  int nxt = NS - 1;                 // stage that receives slab kt + NS - 1
  if constexpr (SCHED == 1) {
    // Ping-pong.  Waves w and w + 4 of the workgroup share a SIMD; they are
    // in the two groups grp = w / 4.  Each wave alternates a load phase --
    // read all of its fragments of slab kt into registers, issue its A
    // share of the slab NS - 1 ahead, wait for its share of slab kt + 1 --
    // and a compute phase of FM * FN * KS MFMAs on registers, between the
    // first of which it issues its B share of that slab.  Group 1 starts
    // one phase late, so while one group multiplies the other loads, and
    // the barrier that ends a phase only hands the matrix cores over.  Slab
    // s is read in phases 2s (group 0) and 2s + 1 (group 1); its stage is
    // refilled (slab s + NS) from phase 2s + 2 on and read again in phase
    // 2s + 2 NS, after both groups' waits for it.
    const int grp = wave >> 2;
    if (grp == 1) phase_barrier();
    for (int kt = kt_begin; kt < kt_end; ++kt) {
      V8 af[KS][FM], bf[KS][FN];
      const uint8_t* st = smem + cur * G::STAGE;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) af[ks][fm] = read_a(st, ks, fm);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) bf[ks][fn] = read_b(st, ks, fn);
      }
      // Refill the stage of slab kt - 1 (both groups' load phases of it
      // ended before the last barrier) with slab kt + NS - 1.  A load
      // written straight to LDS holds up the issuing wave for ~25 cycles,
      // so the A loads are issued here, in the load phase, where the wave
      // would otherwise idle at the barrier; the B loads stay between the
      // first MFMAs of the compute phase, so that the load phase (fragment
      // reads, then loads) does not outgrow the compute phase.  Measured on
      // the FFN shapes against all loads in one phase: +3 to +6 %.
#pragma unroll
      for (int j = 0; j < A_CH; ++j) issue_one(kt + NS - 1, smem + nxt * G::STAGE, j);
      // own share of slab kt + 1 landed: slabs (or placeholders) up to
      // kt + NS - 2 were issued in full; of slab kt + NS - 1 only the A
      // loads just issued may stay in flight
      wait_vmcnt<(NS - 3) * G::LPS + A_CH>();
      phase_barrier();
      static_assert(kNMfma >= B_CH, "the B loads go between the first MFMAs");
      mfma_range_with(af, bf, 0, kNMfma, [&](int q) {
        if (q < B_CH) issue_one(kt + NS - 1, smem + nxt * G::STAGE, A_CH + q);
      });
      phase_barrier();
      cur = (cur + 1 == NS) ? 0 : cur + 1;
      nxt = (nxt + 1 == NS) ? 0 : nxt + 1;
    }
    if (grp == 0) phase_barrier();
    // the placeholder loads of the last compute phases write into the ring,
    // which the epilogue reuses
    wait_vmcnt<0>();
    __syncthreads();
  } else
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    // the stage of slab kt-1 is free: every wave passed the last barrier
    const bool more = kt + NS - 1 < kt_end;
    if (more) issue(kt + NS - 1, smem + nxt * G::STAGE);
    compute(smem + cur * G::STAGE);
    // slab kt+1 must have landed; slabs kt+2 .. kt+NS-1 may stay in flight
    if (more)
      wait_vmcnt<(NS - 2) * G::LPS>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    cur = (cur + 1 == NS) ? 0 : cur + 1;
    nxt = (nxt + 1 == NS) ? 0 : nxt + 1;
  }
  }  // schedules 0 and 1

  if constexpr (GEMMEPI_LDS_POISON != 0) {
    // every load has landed (the drain above): poison the whole ring before
    // the epilogue (and the split-K arrival flag) reuse it
    for (int i = tid; i < SMEM_BYTES / 16; i += NT)
      *(u32x4*)(smem + 16 * i) = u32x4{~0u, ~0u, ~0u, ~0u};
    __syncthreads();
  }

  // ---- split-K: partial tiles through the workspace ---------------------------
  // Each split writes its fp32 accumulators to its slot of the workspace.
  // The slot is written and read with the agent-scope coherence bit, which
  // keeps the accesses coherent across the XCDs' L2 caches on their own; a
  // fence would instead write back and invalidate the whole L2 of the XCD,
  // which measured ~0.7 us per workgroup.  (Agent-scope atomic loads and
  // stores carry the same bit but move 4 bytes per lane; 16 per lane
  // measured up to 5 % faster on split-K launches.)  A split
  // waits for its stores to complete, then counts its arrival; the split
  // that arrives last sums all slots in split order (the result does not
  // depend on arrival order), resets the count and runs the epilogue.
  // Nothing waits on another workgroup, so no ordering of the workgroups
  // can stall the grid.
  if (p.splits > 1) {
    constexpr int QE = FM * FN * kAccN;  // floats per thread
    constexpr int G4 = kAccN / 4;        // 16-byte groups per accumulator block
    // A slot holds group g (4 consecutive elements of a block) of thread t at
    // bytes 16 (g NT + t): each store or load of a wave is one contiguous
    // 1 KiB.  The accesses carry the agent-scope coherence bit (sc1, the bit
    // agent-scope atomics are built with), 16 bytes per lane.
    constexpr int kSc1 = 16;
    float* const slots = p.ws + (size_t)tile_id * p.splits * (BM * BN);
    const __amdgpu_buffer_rsrc_t rslot = make_rsrc(slots);
    auto slot_off = [&](int s, int blk, int g4) -> uint32_t {
      return (uint32_t)s * (QE * NT * 4u) + (uint32_t)((blk * G4 + g4) * NT + tid) * 16u;
    };
    static_for<FM>([&](auto fm_c) {
      constexpr int fm = decltype(fm_c)::value;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int g4 = 0; g4 < G4; ++g4) {
          const u32x4 w = {__float_as_uint(acc[fm][fn][4 * g4]), __float_as_uint(acc[fm][fn][4 * g4 + 1]),
                           __float_as_uint(acc[fm][fn][4 * g4 + 2]), __float_as_uint(acc[fm][fn][4 * g4 + 3])};
          __builtin_amdgcn_raw_buffer_store_b128(w, rslot, slot_off(split, fm * FN + fn, g4), 0, kSc1);
        }
    });
    wait_vmcnt<0>();  // this thread's slot stores are complete
    __syncthreads();  // ... and every thread's
    // the flag lives in the (drained) staging ring: a separate LDS variable
    // would push the largest rings past the 160 KiB of a CU
    uint32_t& s_last = *(uint32_t*)smem;
    if (tid == 0) {
      const uint32_t before = __hip_atomic_fetch_add(&p.counters[tile_id], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      const uint32_t last = before == (uint32_t)(p.splits - 1) ? 1u : 0u;
      if (last) __hip_atomic_store(&p.counters[tile_id], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    const uint32_t is_last = s_last;
    __syncthreads();  // every thread has read the flag before the epilogue reuses the ring
    if (is_last == 0u) return;  // uniform over the workgroup
    // the reduction moves 16 or 32 floats per thread per step (hoisting all
    // loads of a slot would spill the accumulators)
    constexpr int FNG = kAccN == 16 ? (FN > 2 ? 1 : FN) : (FN > 4 ? 4 : FN);  // blocks per step
    static_assert(FN % FNG == 0, "split-K load steps");
    // Two splits on the 32 x 32 MFMA tiles (the small tiles, whose
    // accumulators leave registers to spare): only the other split's slot is
    // read; this split's partial is still in its accumulators.  The paths
    // below form (0 + partial 0) + partial 1; here split 0 forms
    // (0 + acc) + slot 1 and split 1 forms (0 + slot 0) + acc, the same bits
    // (a + b == b + a exactly), so the result still does not depend on which
    // split arrived last.  The loads of each step are issued one step
    // ahead.  (On the 256-wide tiles a second path here costs spills.)
    if (kAccN == 16 && p.splits == 2) {
      constexpr bool kAhead = true;
      constexpr int NF = FN / FNG, NSTEP = FM * NF;
      float v[kAhead ? 2 : 1][FNG][kAccN];
      auto issue = [&](auto st_c) {
        constexpr int st = decltype(st_c)::value;
        constexpr int fm = st / NF, f0 = (st % NF) * FNG, b = kAhead ? (st & 1) : 0;
#pragma unroll
        for (int j = 0; j < FNG; ++j)
#pragma unroll
          for (int g4 = 0; g4 < G4; ++g4) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                rslot, slot_off(1 - split, fm * FN + f0 + j, g4), 0, kSc1);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[b][j][4 * g4 + e] = __uint_as_float(w[e]);
          }
      };
      if constexpr (kAhead) issue(std::integral_constant<int, 0>{});
      const bool first = split == 0;
      static_for<NSTEP>([&](auto st_c) {
        constexpr int st = decltype(st_c)::value;
        constexpr int fm = st / NF, f0 = (st % NF) * FNG, b = kAhead ? (st & 1) : 0;
        if constexpr (!kAhead)
          issue(st_c);
        else if constexpr (st + 1 < NSTEP)
          issue(std::integral_constant<int, st + 1>{});
#pragma unroll
        for (int j = 0; j < FNG; ++j)
#pragma unroll
          for (int r = 0; r < kAccN; ++r) {
            const float a = acc[fm][f0 + j][r], c = v[b][j][r];
            acc[fm][f0 + j][r] = (0.0f + (first ? a : c)) + (first ? c : a);
          }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else if constexpr (QE <= 64 && (FM * (FN / FNG)) % 2 == 0) {
      // tiles with at most 64 accumulators per thread: the slots in split
      // order, each step's loads issued one step ahead (into the other of two
      // register sets; a slot has an even number of steps, so a step's set is
      // the same in every slot), the next slot's first step after a slot's
      // last.  This split's own term comes from a copy of its accumulators
      // instead of its slot.  (The second set makes the 256-wide tiles spill.)
      constexpr int NF = FN / FNG, SPS = FM * NF;
      float own[FM][FN][kAccN];
      static_for<FM>([&](auto fm_c) {
        constexpr int fm = decltype(fm_c)::value;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
          for (int r = 0; r < kAccN; ++r) own[fm][fn][r] = acc[fm][fn][r];
      });
      float v[2][FNG][kAccN];
      auto load = [&](int s, int fm, int f0, float (&dst)[FNG][kAccN]) {
        if (s == split) return;  // uniform: the own term is in registers
#pragma unroll
        for (int j = 0; j < FNG; ++j)
#pragma unroll
          for (int g4 = 0; g4 < G4; ++g4) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                rslot, slot_off(s, fm * FN + f0 + j, g4), 0, kSc1);
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[j][4 * g4 + e] = __uint_as_float(w[e]);
          }
      };
      load(0, 0, 0, v[0]);
      for (int s = 0; s < p.splits; ++s) {
        const bool mine = s == split;
        static_for<SPS>([&](auto st_c) {
          constexpr int st = decltype(st_c)::value;
          constexpr int fm = st / NF, f0 = (st % NF) * FNG, b = st & 1;
          if constexpr (st + 1 < SPS)
            load(s, (st + 1) / NF, ((st + 1) % NF) * FNG, v[b ^ 1]);
          else if (s + 1 < p.splits)
            load(s + 1, 0, 0, v[b ^ 1]);
#pragma unroll
          for (int j = 0; j < FNG; ++j)
#pragma unroll
            for (int r = 0; r < kAccN; ++r)
              acc[fm][f0 + j][r] =
                  (s == 0 ? 0.0f : acc[fm][f0 + j][r]) + (mine ? own[fm][f0 + j][r] : v[b][j][r]);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
    } else {
      // every other tile shape: step by step, the sum over the slots in split
      // order, this split's own term taken from its accumulators rather than
      // read back from its slot (each element still sums the same terms in
      // the same order)
      static_for<FM>([&](auto fm_c) {
        constexpr int fm = decltype(fm_c)::value;
#pragma unroll
        for (int f0 = 0; f0 < FN; f0 += FNG) {
          float t[FNG][kAccN];
          for (int s = 0; s < p.splits; ++s) {
            float v[FNG][kAccN];
            if (s == split) {
#pragma unroll
              for (int j = 0; j < FNG; ++j)
#pragma unroll
                for (int r = 0; r < kAccN; ++r) v[j][r] = acc[fm][f0 + j][r];
            } else {
#pragma unroll
              for (int j = 0; j < FNG; ++j)
#pragma unroll
                for (int g4 = 0; g4 < G4; ++g4) {
                  const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
                      rslot, slot_off(s, fm * FN + f0 + j, g4), 0, kSc1);
#pragma unroll
                  for (int e = 0; e < 4; ++e) v[j][4 * g4 + e] = __uint_as_float(w[e]);
                }
            }
#pragma unroll
            for (int j = 0; j < FNG; ++j)
#pragma unroll
              for (int r = 0; r < kAccN; ++r) t[j][r] = (s == 0 ? 0.0f : t[j][r]) + v[j][r];
          }
#pragma unroll
          for (int j = 0; j < FNG; ++j)
#pragma unroll
            for (int r = 0; r < kAccN; ++r) acc[fm][f0 + j][r] = t[j][r];
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    }
  }

  // ---- epilogue on the accumulators -----------------------------------------
  // In block (fm, fn) a lane owns local row rl = wrow0 + kMfma fm + lrow and
  // the columns cl + kColStride g + {0,1,2,3} (g < kAccN / 4, element
  // r = 4 g + e), with cl = wcol0 + kMfma fn + 4 lgrp.  The results are
  // rounded into an LDS copy of the output tile (free since the main loop's
  // last barrier) and then written to HBM row by row with 16-byte stores:
  // written straight from the accumulator layout, every store instruction
  // would touch 16 or 32 rows.
  const int epi = p.epi;
  const int wrow0 = wm * WTM;
  const int wcol0 = wn * WTN;
  uint8_t* const so = smem;                                  // [BM][BN] of T
  float* const red = (float*)(smem + G::OUT_BYTES);          // [WM][BN] fp32
  float* const bsl = (float*)(smem + G::OUT_BYTES + G::RED_BYTES);  // bias slice, fp32

  constexpr int NG = kAccN / 4;         // 4-column groups per lane and block
  constexpr int BPW = 32 / kMfma;       // blocks per 32-column mask word
  auto stage = [&](int rl, int cl, const float (&y)[kAccN]) {
    uint8_t* row = so + rl * (BN * 2) + (cl & 7) * 2;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int c = cl + kColStride * g;
      const u32x2 w = {pack2(y[4 * g], y[4 * g + 1], T{}), pack2(y[4 * g + 2], y[4 * g + 3], T{})};
      *(u32x2*)(row + (((c >> 3) ^ G::swz_o(rl)) << 4)) = w;
    }
  };

  // the tile [BM][BN] of a dtype [M, ldo] matrix into the staging buffer,
  // row by row with 16-byte loads (zeros outside the matrix)
  constexpr int CPR = BN / 8, RPP = NT / CPR;
  auto load_tile = [&](const T* src) {
    const int ch = tid % CPR;
    const int n = n0 + ch * 8;
    const bool vec_load = (p.ldo & 7) == 0;
    for (int rl = tid / CPR; rl < BM; rl += RPP) {
      const int m = m0 + rl;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (src != nullptr && m < M && n < N) {
        const T* q = src + (size_t)m * p.ldo + n;
        if (vec_load && n + 7 < N) {
          v = *(const u32x4*)q;
        } else {
          const uint16_t* s16 = (const uint16_t*)q;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (n + e < N) v[e >> 1] |= (uint32_t)s16[e] << (16 * (e & 1));
        }
      }
      *(u32x4*)(so + rl * (BN * 2) + ((ch ^ G::swz_o(rl)) << 4)) = v;
    }
  };
  // the staged value at local row rl, local column c (4-column groups)
  auto staged4 = [&](int rl, int c_loc) -> uint8_t* {
    return so + rl * (BN * 2) + (((c_loc >> 3) ^ G::swz_o(rl)) << 4) + (c_loc & 7) * 2;
  };

  if (epi == EPI_DRELU_BGRAD || epi == EPI_DGELU_BGRAD) {
    // DRELU: dZ = mask ? acc : 0.  DGELU: dZ = acc * gelu'(z), z the saved
    // pre-activation (its tile is staged through LDS first and each dZ is
    // written over its z).  bgrad[n] += sum over this tile's rows of dZ.
    const bool dgelu = epi == EPI_DGELU_BGRAD;
    if (dgelu) {
      load_tile((const T*)p.aux);
      __syncthreads();
    }
    float cs[FN][kAccN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int r = 0; r < kAccN; ++r) cs[fn][r] = 0.0f;
    static_for<FM>([&](auto fm_c) {
      constexpr int fm = decltype(fm_c)::value;
      const int rl = wrow0 + fm * kMfma + lrow;
      const int m = m0 + rl;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int cl = wcol0 + fn * kMfma + 4 * lgrp;  // local column of element r = 0
        float y[kAccN];
        if (dgelu) {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const u32x2 zw = *(const u32x2*)staged4(rl, cl + kColStride * g);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint16_t zb = (uint16_t)(zw[e >> 1] >> (16 * (e & 1)));
              const float zz = to_f32(__builtin_bit_cast(T, zb));
              y[4 * g + e] = acc[fm][fn][4 * g + e] * gelu_grad(zz);
            }
          }
        } else {
          // the mask word holding this block's columns, shifted to the
          // lane's first column (a block never straddles a word)
          const int c0 = n0 + cl;
          const uint32_t mw = (m < M && c0 < N) ? p.aux[(size_t)m * p.aux_ld + (c0 >> 5)] >> (c0 & 31)
                                                : 0u;
#pragma unroll
          for (int r = 0; r < kAccN; ++r) {
            const int bit = kColStride * (r >> 2) + (r & 3);
            y[r] = ((mw >> bit) & 1u) ? acc[fm][fn][r] : 0.0f;
          }
        }
#pragma unroll
        for (int r = 0; r < kAccN; ++r) cs[fn][r] += y[r];
        stage(rl, cl, y);
      }
    });
    // sum over the rows held by the lanes of the same lane group
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int r = 0; r < kAccN; ++r) {
        float v = cs[fn][r];
#pragma unroll
        for (int o = 1; o < kMfma; o <<= 1) v += __shfl_xor(v, o);
        cs[fn][r] = v;
      }
    if (lrow == 0) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int r = 0; r < kAccN; ++r)
          red[wm * BN + wcol0 + fn * kMfma + kColStride * (r >> 2) + 4 * lgrp + (r & 3)] = cs[fn][r];
    }
  } else if (epi == EPI_BIAS_RES_NORM) {
    // Single-pass GEMM + bias + residual + norm.  y = acc + bias + residual
    // is formed in fp32 from the accumulators (never rounded before the
    // norm), once for the row sums and again, bit for bit the same, for the
    // normalisation (the accumulators stay unchanged, so no second copy of
    // the tile is held in registers; the residual stays staged in LDS until
    // each lane overwrites its own elements with the result).
    // The row sums of y and y^2 of the whole row (all tiles_n workgroups of
    // this tile row) meet in fp64 in row_sums: each workgroup adds its
    // partial sums, then counts its arrival; when all have arrived, each
    // reads the row statistics, normalises its own tile and writes it once.
    // The host runs this form only when the whole grid fits on the chip at
    // once, so every workgroup of the tile row is resident and the wait
    // ends; the wait is still bounded, and a workgroup that gives up sets
    // bit 1 of row_sync[0] and writes NaN rows.
    load_tile((const T*)p.residual);
    float* const gsl = bsl + BN;      // gamma slice
    float* const esl = bsl + 2 * BN;  // beta slice
    uint32_t* const wait_ok = (uint32_t*)(bsl + 3 * BN);
    const bool has_beta = p.beta != nullptr;
    {
      const T* bias = (const T*)p.bias;
      const T* gamma = (const T*)p.gamma;
      const T* beta = (const T*)p.beta;
      for (int i = tid; i < BN; i += NT) {
        const bool in = n0 + i < N;
        bsl[i] = (bias != nullptr && in) ? to_f32(bias[n0 + i]) : 0.0f;
        gsl[i] = in ? to_f32(gamma[n0 + i]) : 0.0f;
        esl[i] = (has_beta && in) ? to_f32(beta[n0 + i]) : 0.0f;
      }
    }
    __syncthreads();
    double* red64 = (double*)(smem + G::OUT_BYTES);  // [WN][BM][2]
    static_for<FM>([&](auto fm_c) {
      constexpr int fm = decltype(fm_c)::value;
      // one row block at a time: interleaving them would hold the LDS reads
      // of all blocks in registers beside the live accumulators
      __builtin_amdgcn_sched_barrier(0);
      const int rl = wrow0 + fm * kMfma + lrow;
      const int m = m0 + rl;
      double s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int cl = wcol0 + fn * kMfma + 4 * lgrp;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int c_loc = cl + kColStride * g;
          const u32x2 rw = *(const u32x2*)staged4(rl, c_loc);
          const f32x4 b4 = *(const f32x4*)(bsl + c_loc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t rb = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
            const float y = acc[fm][fn][4 * g + e] + b4[e] + to_f32(__builtin_bit_cast(T, rb));
            if (n0 + c_loc + e < N && m < M) {
              s1 += (double)y;
              s2 += (double)y * (double)y;
            }
          }
        }
      }
#pragma unroll
      for (int o = kMfma; o < 64; o <<= 1) {
        s1 += __shfl_xor(s1, o);
        s2 += __shfl_xor(s2, o);
      }
      if (lgrp == 0) {
        red64[(wn * BM + rl) * 2] = s1;
        red64[(wn * BM + rl) * 2 + 1] = s2;
      }
    });
    __syncthreads();
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      if (m >= M) continue;
      double s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        s1 += red64[(w * BM + r) * 2];
        s2 += red64[(w * BM + r) * 2 + 1];
      }
      unsafeAtomicAdd(&p.row_sums[2 * (size_t)m], s1);
      unsafeAtomicAdd(&p.row_sums[2 * (size_t)m + 1], s2);
    }
    // every thread's sums have reached the device-coherent level before
    // thread 0 counts this workgroup in (as in the split-K arrival)
    wait_vmcnt<0>();
    __syncthreads();
    if (tid == 0) {
      uint32_t* const arrived = p.row_sync + 1 + tm;
      __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      uint32_t ok = 1u;
      for (uint32_t polls = 0;
           __hip_atomic_load(arrived, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)p.tiles_n;
           ++polls) {
        if (polls >= p.norm_wait_polls) {
          ok = 0u;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      if (tm == 0 && tn == 0) __hip_atomic_fetch_or(p.row_sync, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (!ok) __hip_atomic_fetch_or(p.row_sync, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *wait_ok = ok;
    }
    __syncthreads();
    const bool ok = *wait_ok != 0u;
    // row statistics in fp64 from the complete sums (the red64 slots are
    // free again: every read of them preceded the last barrier)
    float* const msl = (float*)(smem + G::OUT_BYTES);  // [BM] mean
    float* const rsl = msl + BM;                        // [BM] rstd
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      float mu = 0.0f, rs = 0.0f;
      if (m < M) {
        const double s1 = __hip_atomic_load(&p.row_sums[2 * (size_t)m], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        const double s2 = __hip_atomic_load(&p.row_sums[2 * (size_t)m + 1], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        const double mean = p.layernorm ? s1 / N : 0.0;
        double var = s2 / N - mean * mean;
        if (var < 0.0) var = 0.0;
        const double rstd = ok ? 1.0 / sqrt(var + (double)p.eps) : __builtin_nan("");
        if (tn == 0) {
          p.stats[2 * (size_t)m] = mean;
          p.stats[2 * (size_t)m + 1] = rstd;
        }
        mu = (float)mean;
        rs = (float)rstd;
      }
      msl[r] = mu;
      rsl[r] = rs;
    }
    __syncthreads();
    static_for<FM>([&](auto fm_c) {
      constexpr int fm = decltype(fm_c)::value;
      __builtin_amdgcn_sched_barrier(0);
      const int rl = wrow0 + fm * kMfma + lrow;
      const float mu = msl[rl], rs = rsl[rl];
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int cl = wcol0 + fn * kMfma + 4 * lgrp;
        float y[kAccN];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int c_loc = cl + kColStride * g;
          const u32x2 rw = *(const u32x2*)staged4(rl, c_loc);
          const f32x4 b4 = *(const f32x4*)(bsl + c_loc);
          const f32x4 g4 = *(const f32x4*)(gsl + c_loc);
          const f32x4 e4 = *(const f32x4*)(esl + c_loc);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint16_t rb = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
            const float yv = acc[fm][fn][4 * g + e] + b4[e] + to_f32(__builtin_bit_cast(T, rb));
            float v = (yv - mu) * rs * g4[e];
            if (has_beta) v += e4[e];
            y[4 * g + e] = v;
          }
        }
        stage(rl, cl, y);
      }
    });
  } else if (epi == EPI_BIAS_RES_SUMS) {
    // y = acc + bias[n] + residual[m, n].  The residual tile is first copied
    // into the staging buffer with row-contiguous 16-byte loads (zeros
    // outside the matrix); each lane then reads its values from there, adds
    // them and writes the rounded y back in place.  Partial row sums of the
    // rounded y and y^2 are kept in fp64 (the norm's variance is formed from
    // them by subtraction).
    load_tile((const T*)p.residual);
    {
      const T* bias = (const T*)p.bias;  // per column; may be null
      for (int i = tid; i < BN; i += NT)
        bsl[i] = (bias != nullptr && n0 + i < N) ? to_f32(bias[n0 + i]) : 0.0f;
    }
    __syncthreads();
    double* red64 = (double*)(smem + G::OUT_BYTES);  // [WN][BM][2]
    static_for<FM>([&](auto fm_c) {
      constexpr int fm = decltype(fm_c)::value;
      const int rl = wrow0 + fm * kMfma + lrow;
      const int m = m0 + rl;
      double s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int cl = wcol0 + fn * kMfma + 4 * lgrp;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int c_loc = cl + kColStride * g;
          uint8_t* at = staged4(rl, c_loc);
          const u32x2 rw = *(const u32x2*)at;
          const f32x4 b4 = *(const f32x4*)(bsl + c_loc);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int c = n0 + c_loc + e;
            const uint16_t rb = (uint16_t)(rw[e >> 1] >> (16 * (e & 1)));
            const float z = acc[fm][fn][4 * g + e] + b4[e] + to_f32(__builtin_bit_cast(T, rb));
            y[e] = to_f32(from_f32<T>(z));  // the value stored
            if (c < N && m < M) {
              s1 += (double)y[e];
              s2 += (double)y[e] * (double)y[e];
            }
          }
          const u32x2 w = {pack2(y[0], y[1], T{}), pack2(y[2], y[3], T{})};
          *(u32x2*)at = w;
        }
      }
      // the lanes with the same lrow hold the row's other column groups
#pragma unroll
      for (int o = kMfma; o < 64; o <<= 1) {
        s1 += __shfl_xor(s1, o);
        s2 += __shfl_xor(s2, o);
      }
      if (lgrp == 0) {
        red64[(wn * BM + rl) * 2] = s1;
        red64[(wn * BM + rl) * 2 + 1] = s2;
      }
    });
  } else {
    // The bias slice of this tile (its BN columns, or its BM rows) goes to
    // LDS once as fp32, zeros outside the matrix; each lane then reads the
    // values of 4 consecutive columns with one 16-byte LDS read.  The element
    // loop is compiled once per epilogue kind, so that it holds no run-time
    // branches on the kind.
    const bool per_col = p.bias_per_col != 0;
    {
      const T* bias = (const T*)p.bias;
      const int len = per_col ? BN : BM, base = per_col ? n0 : m0, lim = per_col ? N : M;
      for (int i = tid; i < len; i += NT)
        bsl[i] = (epi != EPI_DEFAULT && base + i < lim) ? to_f32(bias[base + i]) : 0.0f;
    }
    __syncthreads();
    auto run = [&](auto kind_c) {
      constexpr int KIND = decltype(kind_c)::value;
      constexpr bool gelu = KIND == EPI_GELU_BIAS || KIND == EPI_GELU_AUX_BIAS;
      constexpr bool relu = KIND == EPI_RELU_BIAS || KIND == EPI_RELU_AUX_BIAS;
      static_for<FM>([&](auto fm_c) {
        constexpr int fm = decltype(fm_c)::value;
        const int rl = wrow0 + fm * kMfma + lrow;
        const int m = m0 + rl;
        const float brow = per_col ? 0.0f : bsl[rl];
        uint32_t wbits = 0;  // mask word being assembled (BPW blocks)
        static_for<FN>([&](auto fn_c) {
          constexpr int fn = decltype(fn_c)::value;
          const int cl = wcol0 + fn * kMfma + 4 * lgrp;  // local column of element r = 0
          float y[kAccN], zs[kAccN];
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const f32x4 b4 = per_col ? *(const f32x4*)(bsl + cl + kColStride * g)
                                     : f32x4{brow, brow, brow, brow};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * g + e;
              const float z = acc[fm][fn][r] + b4[e];
              zs[r] = z;
              if constexpr (gelu)
                y[r] = gelu_erf(z);
              else if constexpr (relu)
                y[r] = z > 0.0f ? z : 0.0f;
              else
                y[r] = z;
              if constexpr (KIND == EPI_RELU_AUX_BIAS) {
                const int c = n0 + cl + kColStride * g + e;
                if (z > 0.0f && c < N) wbits |= 1u << (c & 31);
              }
            }
          }
          stage(rl, cl, y);
          if constexpr (KIND == EPI_GELU_AUX_BIAS) {
            // z = acc + bias, rounded, straight into aux: 8-byte stores of
            // 4 consecutive columns per lane and group
            if (m < M) {
              T* zrow = (T*)p.aux + (size_t)m * p.ldo;
#pragma unroll
              for (int g = 0; g < NG; ++g) {
                const int c = n0 + cl + kColStride * g;
                if ((p.ldo & 3) == 0 && c + 3 < N) {
                  const u32x2 w = {pack2(zs[4 * g], zs[4 * g + 1], T{}),
                                   pack2(zs[4 * g + 2], zs[4 * g + 3], T{})};
                  *(u32x2*)(zrow + c) = w;
                } else {
#pragma unroll
                  for (int e = 0; e < 4; ++e)
                    if (c + e < N) zrow[c + e] = from_f32<T>(zs[4 * g + e]);
                }
              }
            }
          }
          if constexpr (KIND == EPI_RELU_AUX_BIAS && (fn + 1) % BPW == 0) {
            // the word's other bits are held by the lanes with the same lrow
#pragma unroll
            for (int o = kMfma; o < 64; o <<= 1) wbits |= __shfl_xor(wbits, o);
            const int cword = n0 + wcol0 + (fn + 1 - BPW) * kMfma;  // first column of the word
            if (lgrp == 0 && m < M && cword < N) {
              uint32_t* mrow = p.aux + (size_t)m * p.aux_ld;
              const int word = cword >> 5;
              mrow[word] = wbits;
              if (word == p.aux_words - 1)
                for (int w = p.aux_words; w < p.aux_ld; ++w) mrow[w] = 0u;
            }
            wbits = 0;
          }
        });
      });
    };
    switch (epi) {
      case EPI_RELU_BIAS: run(std::integral_constant<int, EPI_RELU_BIAS>{}); break;
      case EPI_RELU_AUX_BIAS: run(std::integral_constant<int, EPI_RELU_AUX_BIAS>{}); break;
      case EPI_GELU_BIAS: run(std::integral_constant<int, EPI_GELU_BIAS>{}); break;
      case EPI_GELU_AUX_BIAS: run(std::integral_constant<int, EPI_GELU_AUX_BIAS>{}); break;
      default: run(std::integral_constant<int, EPI_BIAS>{}); break;  // DEFAULT: the bias slice is zero
    }
  }
  __syncthreads();

  // the staged tile -> dst: thread t copies 16-byte chunk t % CPR of local
  // row t / CPR (+ RPP per pass), so a wave writes whole row segments
  auto store_tile = [&](T* dst_base) {
    const size_t ldo = (size_t)p.ldo;
    const bool vec_store = (p.ldo & 7) == 0;  // 16-byte aligned rows
    const int ch = tid % CPR;
    const int n = n0 + ch * 8;
#pragma unroll 4
    for (int rl = tid / CPR; rl < BM; rl += RPP) {
      const u32x4 v = *(const u32x4*)(so + rl * (BN * 2) + ((ch ^ G::swz_o(rl)) << 4));
      const int m = m0 + rl;
      if (m >= M || n >= N) continue;
      T* dst = dst_base + (size_t)m * ldo + n;
      if (vec_store && n + 7 < N) {
        if constexpr (GEMMEPI_NT_OUT)
          __builtin_nontemporal_store(v, (u32x4*)dst);
        else
          *(u32x4*)dst = v;
      } else {
        uint16_t* d16 = (uint16_t*)dst;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n + e < N) d16[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  };
  store_tile((T*)p.out);


  if (epi == EPI_BIAS_RES_SUMS) {
    const double* red64 = (const double*)(smem + G::OUT_BYTES);
    for (int r = tid; r < BM; r += NT) {
      const int m = m0 + r;
      if (m >= M) continue;
      double s1 = 0.0, s2 = 0.0;
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        s1 += red64[(w * BM + r) * 2];
        s2 += red64[(w * BM + r) * 2 + 1];
      }
      unsafeAtomicAdd(&p.stats[2 * (size_t)m], s1);
      unsafeAtomicAdd(&p.stats[2 * (size_t)m + 1], s2);
    }
  }
  if (epi == EPI_DRELU_BGRAD || epi == EPI_DGELU_BGRAD) {
    for (int c = tid; c < BN; c += NT) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < WM; ++w) s += red[w * BN + c];
      if (n0 + c < N) unsafeAtomicAdd(&p.bgrad[n0 + c], s);
    }
  }
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int NS, bool BT, int SCHED, int MT>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
  static_assert(SCHED >= 0 && SCHED <= 2, "schedule");
  static_assert(SCHED == 0 || WM * WN == 8, "ping-pong pairs waves w and w + 4 on each SIMD");
  static_assert(SCHED != 1 || NS >= 3, "ping-pong issues each slab NS - 1 ahead from a compute phase");
  static_assert(SCHED != 1 || (BK / MfmaShape<MT>::kKStep) * (BM / WM / MT) * (BN / WN / MT) >=
                                  GemmTile<BM, BN, BK, WM, WN, NS, MT>::B_CH,
                "ping-pong issues one B load after each of the first MFMAs of a compute phase");
  const int blocks = a.tiles_m * a.tiles_n * (a.splits > 1 ? a.splits : 1);
  hipLaunchKernelGGL((gemm_kernel<T, BM, BN, BK, WM, WN, NS, BT, SCHED, MT>), dim3(blocks), dim3(WM * WN * 64),
                     0, s, a);
  return hipGetLastError();
}

template <typename T, bool BT>
hipError_t blocks_per_cu_by_tile(int tile, int* n) {
  switch (tile) {
#define GEMMEPI_CASE(id, bm, bn, bk, wm, wn, ns, pp, mt)                                     \
  case id:                                                                                 \
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(                                   \
        n, gemm_kernel<T, bm, bn, bk, wm, wn, ns, BT, pp, mt>, wm * wn * 64, 0);
    GEMMEPI_TILES(GEMMEPI_CASE)
#undef GEMMEPI_CASE
    default:
      return hipErrorInvalidValue;
  }
}

template <typename T, bool BT>
hipError_t launch_by_tile(int tile, const GemmArgs& a, hipStream_t s) {
  switch (tile) {
#define GEMMEPI_CASE(id, bm, bn, bk, wm, wn, ns, pp, mt) \
  case id:                                               \
    return launch_tile<T, bm, bn, bk, wm, wn, ns, BT, pp, mt>(a, s);
    GEMMEPI_TILES(GEMMEPI_CASE)
#undef GEMMEPI_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace gemmepi
