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
//     (16 steps) before consuming any, so one workgroup keeps its whole
//     16 x K slice of W in flight;
//   * the token rows x[t, window] are loaded once per wave, one contiguous
//     1 KiB load per token, into a swizzled LDS window from which the MFMA
//     fragments are read (loading them in fragment form would cost one
//     vector memory instruction per k step even for a single token);
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

constexpr int kDecodeWaves = 8;
constexpr int kDecodeUnroll = 16;            // 32-wide k steps per W batch
constexpr int kDecodeWin = 32 * kDecodeUnroll;  // k window of one batch (512)

// One wave's copy of the x window: [16 tokens][512 k] fp16 = 16 KiB, with the
// 16-byte chunk c of token row t stored at chunk c ^ t, so that the MFMA
// fragment read (16 lanes = 16 token rows at the same logical chunk) and the
// row writes (64 lanes = 64 chunks of one row) are both bank-conflict-free.
__device__ __forceinline__ uint32_t xwin_off(int t, int chunk) {
  return (uint32_t)(t * (kDecodeWin * 2) + ((chunk ^ t) << 4));
}

// TB: token bucket (1, 2, 4, 8 or 16) >= M, so the x loads unroll.
template <typename T, int TB>
__global__ void __launch_bounds__(kDecodeWaves * 64) decode_kernel(const DecodeArgs p) {
  using V8 = typename Frag<T>::type;
  __shared__ f32x4 red[kDecodeWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xwin[kDecodeWaves][TB * kDecodeWin * 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int r16 = lane & 15;        // W row within the block / token index
  const int kg = lane >> 4;         // k group of this lane within a 32-wide step
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
  const bool w_ok = n0 + r16 < p.N;
  const uint32_t w_row = (uint32_t)(r16 * p.ldw) * 2u;
  uint8_t* xw = xwin[wave];

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = kbeg; k < kend; k += kDecodeWin) {
    // x first (TB contiguous 1 KiB loads), then the whole W window (16
    // steps: lane row r16, 8 k values of step u at k + 32 u + 8 kg)
    u32x4 xl[TB];
#pragma unroll
    for (int t = 0; t < TB; ++t) {
      const int kk = k + lane * 8;
      xl[t] = buffer_load16(rX, (t < Mt && kk < kend) ? (uint32_t)(t * p.ldx + kk) * 2u : kOOB);
    }
    u32x4 wv[kDecodeUnroll];
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      const int kk = k + u * 32 + kg * 8;
      wv[u] = buffer_load16(rW, (kk < kend && w_ok) ? w_row + (uint32_t)kk * 2u : kOOB);
    }
#pragma unroll
    for (int t = 0; t < TB; ++t) *(u32x4*)(xw + xwin_off(t, lane)) = xl[t];
    u32x4 xf[kDecodeUnroll];
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      xf[u] = u32x4{0u, 0u, 0u, 0u};
      if (r16 < TB) xf[u] = *(const u32x4*)(xw + xwin_off(r16, u * 4 + kg));
    }
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u)
      acc = mfma16(__builtin_bit_cast(V8, wv[u]), __builtin_bit_cast(V8, xf[u]), acc);
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

template <typename T>
static void launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.N + 15) / 16), block(kDecodeWaves * 64);
  if (a.M <= 1)
    hipLaunchKernelGGL((decode_kernel<T, 1>), grid, block, 0, s, a);
  else if (a.M <= 2)
    hipLaunchKernelGGL((decode_kernel<T, 2>), grid, block, 0, s, a);
  else if (a.M <= 4)
    hipLaunchKernelGGL((decode_kernel<T, 4>), grid, block, 0, s, a);
  else if (a.M <= 8)
    hipLaunchKernelGGL((decode_kernel<T, 8>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<T, 16>), grid, block, 0, s, a);
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) {
  if (a.M < 1 || a.M > 16) return hipErrorInvalidValue;
  if (dtype == DT_F16)
    launch_decode_t<_Float16>(a, s);
  else
    launch_decode_t<__bf16>(a, s);
  return hipGetLastError();
}

}  // namespace gemmepi
