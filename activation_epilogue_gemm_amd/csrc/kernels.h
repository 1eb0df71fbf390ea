// Internal interface between the C-ABI host code and the HIP kernels of
// libgemmepi.  Not installed; callers use include/gemmepi.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gemmepi {

enum Epi : int {
  EPI_DEFAULT = 0,
  EPI_BIAS = 1,
  EPI_RELU_BIAS = 2,
  EPI_RELU_AUX_BIAS = 3,
  EPI_GELU_BIAS = 4,
  EPI_DRELU_BGRAD = 5,
  EPI_BIAS_RES_RMSNORM = 6,
  EPI_BIAS_RES_LAYERNORM = 7,
  EPI_GELU_AUX_BIAS = 8,
  EPI_DGELU_BGRAD = 9,
  // GEMM-kernel epilogue of both norms (not a public value): y = acc + bias
  // + residual rounded to out, fp64 partial row sums of y and y^2 added into
  // stats
  EPI_BIAS_RES_SUMS = 16,
  // GEMM-kernel epilogue of the single-pass norm (not a public value): y =
  // acc + bias + residual kept in fp32 registers; the workgroups of a tile
  // row add fp64 partial row sums of y and y^2 into row_sums, count their
  // arrival in row_sync and wait for the whole row; each then normalises its
  // own tile and writes it once
  EPI_BIAS_RES_NORM = 17
};

enum DType : int { DT_F16 = 0, DT_BF16 = 1 };

// Arguments of the tiled MFMA GEMM kernel (passed by value).
struct GemmArgs {
  const void* A;     // [M, lda] row-major
  const void* B;     // [K, ldb] or, transposed, [N, ldb]
  const void* bias;  // [M] or [N] in the input dtype (BIAS-type epilogues)
  uint32_t* aux;     // packed mask [M, aux_ld] (out for RELU_AUX, in for DRELU), or
                     // the pre-activation z [M, ldo] in the output dtype (out for
                     // GELU_AUX, in for DGELU)
  void* out;         // [M, ldo]
  float* bgrad;      // [N] fp32, pre-zeroed (DRELU_BGRAD)
  const void* residual;  // [M, ldo] in the output dtype or null (BIAS_RES_SUMS)
  double* stats;     // [M][2] fp64: row sums of y, y^2, pre-zeroed (BIAS_RES_SUMS);
                     // (mean, rstd) written by the tile-column-0 workgroups (BIAS_RES_NORM)
  // single-pass norm (BIAS_RES_NORM)
  const void* gamma;   // [N] in the input dtype
  const void* beta;    // [N] in the input dtype, or null
  float eps;
  int layernorm;       // 1: LayerNorm, 0: RMSNorm
  double* row_sums;    // [M][2] fp64 sums of y and y^2, pre-zeroed
  uint32_t* row_sync;  // [0]: status (bit 0 ran, bit 1 a wait gave up); [1 + tm]: arrivals
                       // of tile row tm; pre-zeroed
  uint32_t norm_wait_polls;  // polls of the row wait before a workgroup gives up
  int M, N, K;
  int lda, ldb, ldo;
  int aux_ld;        // words per mask row
  int aux_words;     // ceil(N / 32): valid words per mask row
  int epi;           // Epi
  int bias_per_col;  // bias indexed by n (1) or by m (0)
  int tiles_m, tiles_n;
  int group_m;       // rows of tiles per raster group
  int xcd_remap;     // 1: give each XCD a contiguous run of tiles
  // chip-block raster (used when sb_m > 0): the grid runs in rounds of
  // sb_m x sb_n tiles, one tile per CU; XCD x owns the sub-block
  // (x / xcd_n, x % xcd_n) of (sb_m / xcd_m) x (sb_n / xcd_n) tiles.
  int sb_m, sb_n, xcd_m, xcd_n;
  // split-K (splits > 1): workgroup split * tiles + t runs k slabs
  // [split * kt_split, min(KT, (split + 1) * kt_split)) of tile t and writes
  // its fp32 partial tile to ws; the last of the tile's splits to arrive
  // (counters) sums the partials in split order and runs the epilogue
  int splits, kt_split;
  float* ws;           // [tiles][splits][BM * BN] fp32 partial tiles
  uint32_t* counters;  // [tiles] arrival counts; zero before and after a launch
};

// Arguments of the thin-M decode kernel.
struct DecodeArgs {
  const void* x;     // [M, ldx] activations, M <= 16
  const void* W;     // [N, ldw] weights, K contiguous
  const void* bias;
  void* out;         // [M, ldo]
  int M, N, K;
  int ldx, ldw, ldo;
  int k_per_wave;    // K range of one wave (multiple of 32)
  int epi;
  int bias_per_col;
};

// One tile configuration of the tiled GEMM.
struct TileCfg {
  int bm, bn, bk, wm, wn, ns, sched;
  int mfma;  // 16: v_mfma_f32_16x16x32, 32: v_mfma_f32_32x32x16
  const char* name;
};

constexpr int kNumTiles = 10;
extern const TileCfg kTiles[kNumTiles];

// Launchers (defined in the per-dtype/per-layout instantiation files).
// Return hipSuccess or the launch error.
hipError_t launch_gemm(int dtype, bool b_trans, int tile, const GemmArgs& a, hipStream_t s);
// Polls of the single-pass norm's row wait before a workgroup gives up
// (each poll: one device-coherent load and a ~128-cycle sleep; the bound is
// in the seconds, where a normal wait lasts microseconds).
constexpr uint32_t kNormWaitPolls = 1u << 21;

// Workgroups of the tile's GEMM kernel that one CU holds at once
// (hipOccupancyMaxActiveBlocksPerMultiprocessor).
hipError_t gemm_blocks_per_cu(int dtype, bool b_trans, int tile, int* n);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s);
// The decode kernel for M tokens, N rows of W and reduction length K, and
// its launch shape (rows of W per workgroup, waves per workgroup).
enum DecodeKind : int {
  DECODE_MFMA = 0,       // 16 rows of W per workgroup, MFMA products (4-16 tokens)
  DECODE_ROWSTREAM = 1,  // 4 rows, 8 waves splitting K, VALU products (1-3 tokens;
                         // 4 when N > 4096 or K > 4096)
  DECODE_ROWWAVE = 2     // 4 rows, one per wave over all of K (1 token, K <= 4096)
};
DecodeKind decode_kind(int M, int N, int K);
int decode_rows(DecodeKind k);
int decode_waves(DecodeKind k);

// Unfused baseline kernels and helpers (elementwise.hip).
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// dst [N, K] = src [K, N] transposed, 16-bit elements; K and N multiples of 8
hipError_t launch_transpose16(const void* src, void* dst, int K, int N, hipStream_t s);
hipError_t launch_bias_add(int dtype, void* out, const void* bias, int M, int N, int ldo,
                           int per_col, hipStream_t s);
hipError_t launch_activation(int dtype, int epi, void* out, uint32_t* aux, int M, int N, int ldo,
                             int aux_ld, hipStream_t s);
hipError_t launch_mask_apply(int dtype, void* out, const uint32_t* aux, int M, int N, int ldo,
                             int aux_ld, hipStream_t s);
// out = out * gelu'(z), z the saved pre-activation [M, ldo] (unfused DGELU)
hipError_t launch_dgelu_apply(int dtype, void* out, const void* z, int M, int N, int ldo,
                              hipStream_t s);
hipError_t launch_colsum(int dtype, const void* dz, float* bgrad, int M, int N, int ldo,
                         hipStream_t s);
// out += residual (both [M, ldo]), rounded to the dtype
hipError_t launch_residual_add(int dtype, void* out, const void* residual, int M, int N, int ldo,
                               hipStream_t s);
// Row norm of out in place: statistics from stats (fp64 sums of y and y^2,
// from_stats = 1) or from the row itself; writes (mean, rstd) to stats.
hipError_t launch_norm_rows(int dtype, void* out, const void* gamma, const void* beta,
                            double* stats, int M, int N, int ldo, float eps, int layernorm,
                            int from_stats, hipStream_t s);

// The library's static device scratch (noalloc.hip): kScratchBytes per
// device, for the split-K workspace of gemmepi_execute_noalloc.  Returns the
// current device's address of it (looked up once per device).
constexpr size_t kScratchBytes = (size_t)80 << 20;
hipError_t scratch_pointer(void** ptr);

// per-dtype launcher tables filled by each instantiation file
using GemmLauncher = hipError_t (*)(const GemmArgs&, hipStream_t);
hipError_t launch_gemm_f16_bn(int tile, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_f16_bt(int tile, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16_bn(int tile, const GemmArgs& a, hipStream_t s);
hipError_t launch_gemm_bf16_bt(int tile, const GemmArgs& a, hipStream_t s);
hipError_t blocks_per_cu_f16_bn(int tile, int* n);
hipError_t blocks_per_cu_f16_bt(int tile, int* n);
hipError_t blocks_per_cu_bf16_bn(int tile, int* n);
hipError_t blocks_per_cu_bf16_bt(int tile, int* n);

}  // namespace gemmepi
