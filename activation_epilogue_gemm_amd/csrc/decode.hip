// Thin-M ("decode") GEMM with the fused epilogue, for gfx950.
//
//   out[t, n] = epilogue( sum_k x[t,k] * W[n,k] + bias )     t < M <= 16
//
// With one to sixteen tokens the weight matrix is read once and every
// element of it is used for at most 16 multiply-adds, so the kernel is
// bound by the HBM read of W, not by arithmetic (ops-nn MatMul fusion
// article, section "Why MatMul is the core bottleneck of LLM inference":
// the [hidden, hidden] fp16 weight must be streamed from HBM at every
// decode step).  The design therefore maximises bytes in flight:
//   * a workgroup owns 16 consecutive output columns n (16 rows of W) and
//     splits K over its 8 wavefronts;
//   * each wave issues all of its 128-bit W loads for a 512-wide k window
//     before consuming any, so one workgroup keeps its whole 16 x K slice
//     of W in flight;
//   * every load instruction reads whole 512-byte row segments (two rows of
//     W, or two token rows of x, per instruction), and the MFMA fragments
//     are read from swizzled LDS copies of the window, one 256-wide half at
//     a time (loading W or x in fragment form, 16 rows x 64 bytes per
//     instruction, was 11-20 % slower);
//   * the products run on v_mfma_f32_16x16x32 with W rows as the 16-row
//     operand and the (zero-padded) tokens as the 16-column operand, which
//     keeps the multiply-adds off the VALU entirely;
//   * the 8 per-wave partial tiles are summed through LDS, then the
//     epilogue (bias, activation, rounding) runs on the sum and the
//     [M x 16] result is stored once.
#include "gemm_mfma.hpp"

namespace gemmepi {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Cache policy of the weight loads (the aux operand of the buffer load):
// 0 = normal, 2 = non-temporal (streamed, evict-first in L2).  The weight
// is read once per call.  Measured over 16 rotated 4096 x 4096 weights,
// interleaved on one box, non-temporal against normal: 6.95 against 7.55 us
// at one token, 7.21 against 7.71 at two, 9.16 against 9.61 at eight, 10.46
// against 10.59 at sixteen, but 8.93 against 8.85 at four, so the MFMA
// kernel streams non-temporally from 8 tokens on.
#ifndef GEMMEPI_DECODE_W_POLICY
#define GEMMEPI_DECODE_W_POLICY 2
#endif

constexpr int kDecodeWaves = 8;
constexpr int kDecodeUnroll = 16;            // 32-wide k steps per W batch
constexpr int kDecodeWin = 32 * kDecodeUnroll;  // k window of one batch (512)
constexpr int kDecodeHalf = kDecodeWin / 2;     // k of one LDS half (256)

// One wave's LDS copy of a 256-wide half window, [rows][256 k] fp16 (512
// bytes per row: 16 rows of W, or the token rows of x), with the 16-byte
// chunk c (0..31) of row r stored at chunk c ^ (r & 15).  The MFMA fragment
// read (16 lanes = 16 rows at the same logical chunk) then touches 16
// distinct 16-byte bank groups of the 256-byte bank line, and the row
// writes (32 lanes = 32 chunks of one row) stay conflict-free.
__device__ __forceinline__ uint32_t half_off(int r, int chunk) {
  return (uint32_t)(r * (kDecodeHalf * 2) + ((chunk ^ (r & 15)) << 4));
}

// TB: token bucket (4, 8 or 16) >= M, so the x loads unroll.  (One to three
// tokens take the row-streaming kernel below.)
template <typename T, int TB>
__global__ void __launch_bounds__(kDecodeWaves * 64) decode_kernel(const DecodeArgs p) {
  static_assert(TB == 4 || TB == 8 || TB == 16, "token bucket");
  using V8 = typename Frag<T>::type;
  constexpr int kWPolicy = GEMMEPI_DECODE_W_POLICY;
  constexpr int XI = TB / 2;                  // x load instructions per half (2 tokens each)
  constexpr int WI = 8;                       // W load instructions per half (2 rows each)
  __shared__ f32x4 red[kDecodeWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t wtile[kDecodeWaves][16 * kDecodeHalf * 2];
  __shared__ __attribute__((aligned(16))) uint8_t xtile[kDecodeWaves][TB * kDecodeHalf * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int r16 = lane & 15;        // fragment row: W row within the block / token index
  const int kg = lane >> 4;         // k group of this lane within a 32-wide step
  const int rh = lane >> 5;         // row of a load instruction's pair (0 or 1)
  const int lc = lane & 31;         // 16-byte chunk of a load instruction's row
  const int kbeg = wave * p.k_per_wave;
  const int kend = min(p.K, kbeg + p.k_per_wave);
  const int Mt = p.M;
  const int epi = p.epi;

  // The epilogue's bias values (lane: token t = r16, columns n0 + 4 kg + r)
  // are requested up front and converted only in the epilogue, so no wait
  // for them delays the weight stream.  Out-of-range entries read zero.
  const __amdgpu_buffer_rsrc_t rBias = make_rsrc(p.bias ? p.bias : p.W);
  const bool want_bias = epi != EPI_DEFAULT && r16 < Mt;
  uint16_t braw[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + kg * 4 + r;
    const bool ok = want_bias && (p.bias_per_col ? n < p.N : true);
    const uint32_t off = ok ? (uint32_t)(p.bias_per_col ? n : r16) * 2u : kOOB;
    braw[r] = __builtin_amdgcn_raw_buffer_load_b16(rBias, off, 0, 0);
  }

  const __amdgpu_buffer_rsrc_t rW = make_rsrc((const uint8_t*)p.W + (size_t)n0 * p.ldw * 2);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.x);
  uint8_t* const wt = wtile[wave];
  uint8_t* const xt = xtile[wave];

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = kbeg; k < kend; k += kDecodeWin) {
    // All loads of the window, in the order they are consumed: per half,
    // the token rows (instruction i: tokens 2i and 2i + 1), then the W rows
    // (instruction j: rows 2j and 2j + 1); lane (rh, lc) reads the 8 k of
    // chunk lc of its row.
    u32x4 xl[2][XI], wl[2][WI];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kk = k + h * kDecodeHalf + lc * 8;
      const bool k_ok = kk < kend;
#pragma unroll
      for (int i = 0; i < XI; ++i) {
        const int t = 2 * i + rh;
        xl[h][i] = buffer_load16(rX, (k_ok && t < Mt) ? (uint32_t)(t * p.ldx + kk) * 2u : kOOB);
      }
#pragma unroll
      for (int j = 0; j < WI; ++j) {
        const int r = 2 * j + rh;
        wl[h][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rW, (k_ok && n0 + r < p.N) ? (uint32_t)(r * p.ldw + kk) * 2u : kOOB, 0, kWPolicy);
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // the half's rows into this wave's LDS tiles (the previous half's
      // fragment reads were issued before these writes and LDS keeps a
      // wave's operations in order)
#pragma unroll
      for (int i = 0; i < XI; ++i) *(u32x4*)(xt + half_off(2 * i + rh, lc)) = xl[h][i];
#pragma unroll
      for (int j = 0; j < WI; ++j) *(u32x4*)(wt + half_off(2 * j + rh, lc)) = wl[h][j];
      // 8 MFMA steps of 32 k: W rows as the 16-row operand, the tokens
      // (rows past TB read as zero) as the 16-column operand
#pragma unroll
      for (int u = 0; u < kDecodeUnroll / 2; ++u) {
        const u32x4 wf = *(const u32x4*)(wt + half_off(r16, 4 * u + kg));
        u32x4 xf = u32x4{0u, 0u, 0u, 0u};
        if (r16 < TB) xf = *(const u32x4*)(xt + half_off(r16, 4 * u + kg));
        acc = mfma16(__builtin_bit_cast(V8, wf), __builtin_bit_cast(V8, xf), acc);
      }
    }
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) s += red[w][lane];

  // lane holds D[i = 4*(lane/16) + r][j = lane % 16]: n = n0 + i, t = j
  const int t = r16;
  if (t >= Mt) return;
  T* out = (T*)p.out;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + kg * 4 + r;
    if (n >= p.N) continue;
    const float z = s[r] + to_f32(__builtin_bit_cast(T, braw[r]));
    float y = z;
    if (epi == EPI_GELU_BIAS) y = gelu_erf(z);
    else if (epi == EPI_RELU_BIAS) y = z > 0.0f ? z : 0.0f;
    out[(size_t)t * p.ldo + n] = from_f32<T>(y);
  }
}

// ---- row-streaming decode for one to three tokens ------------------------
// With M <= 3 the products are too few to need the matrix cores, and the
// weight stream is best read the way a plain streaming read is fastest: one
// contiguous 1 KiB per load instruction, and many small workgroups (the
// stream-read sweep of the benchmark peaks at 32 KiB per workgroup).  A
// workgroup owns R consecutive rows of W (R = 4: 32 KiB of a 4096-wide
// row block); wave w covers k in [512 w, 512 w + 512) + 4096 j, and lane l
// of it the 8 consecutive k at 8 l, so load r of a lane reads row r's
// 16 bytes there and the wave's 64 lanes read 1 KiB of one row.  Each lane
// multiplies its W chunks with the same k chunk of every token on the VALU
// (v_dot2: fp32 accumulation of exact fp16/bf16 products), the R x TB
// partial sums are reduced over the wave's lanes (DPP, below), then over
// the 8 waves through LDS, and wave 0 applies the epilogue.
// (each vector element is copied to a scalar before the bit cast: this
// compiler's __builtin_bit_cast of an ext_vector element expression reads
// element 0 whatever the index)
// Sum of v over the 64 lanes of a wave, left in lane 63 (other lanes hold
// partial sums).  DPP moves within rows of 16 lanes (quad permutations, then
// the half-row and row mirrors) leave every lane with its row's sum; the row
// broadcasts of lane 15 and lane 31 then fold rows 0..2 into row 3.  Each
// step is a VALU operation with a DPP source, a few cycles, where a
// cross-lane shuffle through the LDS crossbar costs an LDS round trip.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_add(float v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), Ctrl, RowMask, 0xF,
                                                false);
  return v + __builtin_bit_cast(float, moved);
}
__device__ __forceinline__ float wave_sum_to_lane63(float v) {
  v = dpp_add<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_add<0x140, 0xF>(v);  // row_mirror
  v = dpp_add<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_add<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float c, _Float16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wi = w[i], xi = x[i];
    c = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, wi), __builtin_bit_cast(f16x2, xi), c,
                               false);
  }
  return c;
}
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float c, __bf16) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wi = w[i], xi = x[i];
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wi), __builtin_bit_cast(bf16x2, xi),
                                        c, false);
  }
  return c;
}

template <typename T, int R, int TB>
__global__ void __launch_bounds__(kDecodeWaves * 64) gemv_kernel(const DecodeArgs p) {
  static_assert(R * TB <= 64, "one epilogue lane of wave 0 per output");
  __shared__ float red[kDecodeWaves][R * TB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * R;
  const int Mt = p.M;
  // the epilogue lane's bias value (wave 0, lane = r * TB + t) is requested
  // before the weight stream, so its latency is not added after the
  // reduction; out-of-range entries read zero
  const int er = lane / TB, et = lane - (lane / TB) * TB;
  const bool want_bias = wave == 0 && lane < R * TB && p.epi != EPI_DEFAULT && et < Mt &&
                         (!p.bias_per_col || n0 + er < p.N);
  const __amdgpu_buffer_rsrc_t rBias = make_rsrc(p.bias ? p.bias : p.W);
  const uint16_t braw = __builtin_amdgcn_raw_buffer_load_b16(
      rBias, want_bias ? (uint32_t)(p.bias_per_col ? n0 + er : et) * 2u : kOOB, 0, 0);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc((const uint8_t*)p.W + (size_t)n0 * p.ldw * 2);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.x);
  float acc[R][TB];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[r][t] = 0.0f;
  constexpr int kWin = kDecodeWaves * 512;  // k covered by one pass of the workgroup
  for (int kw = 0; kw < p.K; kw += kWin) {
    const int k = kw + wave * 512 + lane * 8;
    const bool k_ok = k < p.K;
    u32x4 wv[R], xv[TB];
#pragma unroll
    for (int r = 0; r < R; ++r)
      wv[r] = __builtin_amdgcn_raw_buffer_load_b128(
          rW, (k_ok && n0 + r < p.N) ? (uint32_t)(r * p.ldw + k) * 2u : kOOB, 0,
          GEMMEPI_DECODE_W_POLICY);
#pragma unroll
    for (int t = 0; t < TB; ++t)
      xv[t] = buffer_load16(rX, (k_ok && t < Mt) ? (uint32_t)(t * p.ldx + k) * 2u : kOOB);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < TB; ++t) acc[r][t] = dot8(wv[r], xv[t], acc[r][t], T{});
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int t = 0; t < TB; ++t) acc[r][t] = wave_sum_to_lane63(acc[r][t]);
  if (lane == 63) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < TB; ++t) red[wave][r * TB + t] = acc[r][t];
  }
  __syncthreads();
  if (wave != 0 || lane >= R * TB) return;
  const int n = n0 + er;
  if (n >= p.N || et >= Mt) return;
  float z = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) z += red[w][lane];
  if (p.epi != EPI_DEFAULT) z += to_f32(__builtin_bit_cast(T, braw));
  float y = z;
  if (p.epi == EPI_GELU_BIAS) y = gelu_erf(z);
  else if (p.epi == EPI_RELU_BIAS) y = z > 0.0f ? z : 0.0f;
  ((T*)p.out)[(size_t)et * p.ldo + n] = from_f32<T>(y);
}

// ---- one token: one row of W per wave -----------------------------------
// A workgroup of 4 waves owns 4 rows of W, wave w row n0 + w over a whole
// 4096-wide k chunk (8 loads of 1 KiB: lane l the 8 k at 512 j + 8 l).  The
// token row of the chunk (8 KiB, L2-hot) is loaded first, by all 256
// threads, and shared through LDS while the weight loads are in flight; each
// wave then reduces its own row over its lanes (DPP) and its lane 63 applies
// the epilogue and stores: no reduction across waves after the weight has
// landed.  Measured over the 16 rotated 4096 x 4096 weights, interleaved on
// one box, against the 8-wave row-streaming kernel below: 6.80 against 6.96
// us at one token, 7.26 against 7.22 at two, 8.01 against 7.91 at three; so
// it serves one token (with K <= 4096, the chunk of LDS it holds).
template <typename T>
__global__ void __launch_bounds__(256) gemv_rowwave_kernel(const DecodeArgs p) {
  constexpr int kChunk = 4096;                 // k per pass: 512 chunks of 8
  __shared__ u32x4 xs[kChunk / 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = blockIdx.x * 4 + wave;
  const bool n_ok = n < p.N;
  // the bias of the epilogue lane, requested before the weight stream
  const __amdgpu_buffer_rsrc_t rBias = make_rsrc(p.bias ? p.bias : p.W);
  const bool want_bias = lane == 63 && p.epi != EPI_DEFAULT && n_ok;
  const uint16_t braw = __builtin_amdgcn_raw_buffer_load_b16(
      rBias, want_bias ? (uint32_t)(p.bias_per_col ? n : 0) * 2u : kOOB, 0, 0);
  const __amdgpu_buffer_rsrc_t rW = make_rsrc((const uint8_t*)p.W + (size_t)(n_ok ? n : 0) * p.ldw * 2);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.x);
  float acc = 0.0f;
  for (int kc = 0; kc < p.K; kc += kChunk) {
    u32x4 xl[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = kc + (tid + 256 * i) * 8;
      xl[i] = buffer_load16(rX, k < p.K ? (uint32_t)k * 2u : kOOB);
    }
    u32x4 wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = kc + 512 * j + lane * 8;
      wv[j] = __builtin_amdgcn_raw_buffer_load_b128(
          rW, (k < p.K && n_ok) ? (uint32_t)k * 2u : kOOB, 0, GEMMEPI_DECODE_W_POLICY);
    }
    __syncthreads();  // every wave has read the previous chunk's token row
#pragma unroll
    for (int i = 0; i < 2; ++i) xs[tid + 256 * i] = xl[i];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = dot8(wv[j], xs[64 * j + lane], acc, T{});
  }
  acc = wave_sum_to_lane63(acc);
  if (lane != 63 || !n_ok) return;
  float z = acc;
  if (p.epi != EPI_DEFAULT) z += to_f32(__builtin_bit_cast(T, braw));
  float y = z;
  if (p.epi == EPI_GELU_BIAS) y = gelu_erf(z);
  else if (p.epi == EPI_RELU_BIAS) y = z > 0.0f ? z : 0.0f;
  ((T*)p.out)[n] = from_f32<T>(y);
}

// Rows per workgroup of the row-streaming kernel for M tokens; 0: the MFMA
// decode kernel above.  Measured over the 16 rotated 4096 x 4096 weights
// against the MFMA kernel (its row-segment loads; 2- and 4-token buckets for
// the comparison), interleaved on one box: 6.97 against 7.99 us at M = 1,
// 7.22 against 8.04 at M = 2, 7.94 against 7.94-8.03 at M = 3, but 8.18
// against 7.96 at M = 4; from five tokens on the row-streaming kernel falls
// far behind (13.1-13.9 us at M = 5..8 with the earlier MFMA kernel at
// 9.1-9.2: each workgroup re-reads every token row, 64 MiB in all at 8
// tokens, and the VALU products grow with M).  Rows per workgroup, interleaved on one box
// (M = 1 / 2 / 3 / 4): 4 rows 7.03 / 7.26 / 8.12 / 8.22 us, 8 rows 7.17 /
// 7.47 / 8.78 / 8.47, 2 rows 7.00 / 7.65 / 8.67 / 9.45.
// Four tokens stay on the MFMA kernel only while it runs in one round of
// one 16-row workgroup per CU (N <= 16 x 256) with one 512-wide k window per
// wave (K <= 8 x 512); past that its workgroups queue for a second round, or
// each wave walks its windows one after another, and the row-streaming
// kernel is faster.  Four tokens over rotated weights, interleaved on one
// box, MFMA against row streaming: 7.95 against 8.18 us at N = K = 4096,
// but 18.89 against 17.94 at N 4096 x K 11008, 19.65 against 17.10 at
// N 11008 x K 4096 and 20.72 against 18.83 at N 12288 x K 4096.
#ifndef GEMMEPI_GEMV_ROWS
#define GEMMEPI_GEMV_ROWS 4
#endif
DecodeKind decode_kind(int M, int N, int K) {
  if (M == 1 && K <= 4096) return DECODE_ROWWAVE;
  if (M <= 3) return DECODE_ROWSTREAM;
  if (M == 4 && (N > 16 * 256 || K > kDecodeWaves * kDecodeWin)) return DECODE_ROWSTREAM;
  return DECODE_MFMA;
}
int decode_rows(DecodeKind k) {
  return k == DECODE_MFMA ? 16 : (k == DECODE_ROWSTREAM ? GEMMEPI_GEMV_ROWS : 4);
}
int decode_waves(DecodeKind k) { return k == DECODE_ROWWAVE ? 4 : kDecodeWaves; }

// R rows of W per workgroup (GEMMEPI_GEMV_ROWS), TB = 1, 2 or 4 tokens
template <typename T>
static void launch_gemv_t(const DecodeArgs& a, hipStream_t s) {
  constexpr int R = GEMMEPI_GEMV_ROWS;
  static_assert(R == 1 || R == 2 || R == 4 || R == 8, "rows per workgroup");
  const dim3 block(kDecodeWaves * 64);
  const dim3 grid((a.N + R - 1) / R);
  if (a.M <= 1)
    hipLaunchKernelGGL((gemv_kernel<T, R, 1>), grid, block, 0, s, a);
  else if (a.M <= 2)
    hipLaunchKernelGGL((gemv_kernel<T, R, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((gemv_kernel<T, R, 4>), grid, block, 0, s, a);
}

template <typename T>
static void launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16), block(kDecodeWaves * 64);
  if (a.M <= 4)
    hipLaunchKernelGGL((decode_kernel<T, 4>), grid, block, 0, s, a);
  else if (a.M <= 8)
    hipLaunchKernelGGL((decode_kernel<T, 8>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, 16>), grid, block, 0, s, a);
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 16) return hipErrorInvalidValue;
  const DecodeKind kind = a.K % 8 == 0 ? decode_kind(a.M, a.N, a.K) : DECODE_MFMA;
  if (kind == DECODE_ROWWAVE) {
    const dim3 grid((a.N + 3) / 4), block(256);
    if (dtype == DT_F16)
      hipLaunchKernelGGL((gemv_rowwave_kernel<_Float16>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((gemv_rowwave_kernel<__bf16>), grid, block, 0, s, a);
  } else if (kind == DECODE_ROWSTREAM) {
    if (dtype == DT_F16)
      launch_gemv_t<_Float16>(a, s);
    else
      launch_gemv_t<__bf16>(a, s);
  } else if (dtype == DT_F16) {
    launch_decode_t<_Float16>(a, s);
  } else {
    launch_decode_t<__bf16>(a, s);
  }
  return hipGetLastError();
}

}  // namespace gemmepi
