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
//   * each wave issues all of its 128-bit W and x loads for up to 16
//     k-steps before consuming any, so one workgroup keeps its whole
//     16 x K slice of W in flight;
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
constexpr int kDecodeUnroll = 16;

template <typename T>
__global__ void __launch_bounds__(kDecodeWaves * 64) decode_kernel(const DecodeArgs p) {
  using V8 = typename Frag<T>::type;
  __shared__ f32x4 red[kDecodeWaves][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n0 = blockIdx.x * 16;
  const int r16 = lane & 15;        // W row within the block / token index
  const int kq = (lane >> 4) * 8;   // k offset of this lane within a 32-wide step
  const int kbeg = wave * p.k_per_wave;
  const int kend = min(p.K, kbeg + p.k_per_wave);

  const __amdgpu_buffer_rsrc_t rW = make_rsrc((const uint8_t*)p.W + (size_t)n0 * p.ldw * 2);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(p.x);
  const bool w_ok = n0 + r16 < p.N;
  const bool x_ok = r16 < p.M;
  const uint32_t w_row = (uint32_t)(r16 * p.ldw) * 2u;
  const uint32_t x_row = (uint32_t)(r16 * p.ldx) * 2u;

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = kbeg; k < kend; k += 32 * kDecodeUnroll) {
    u32x4 wv[kDecodeUnroll], xv[kDecodeUnroll];
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u) {
      const int kk = k + u * 32 + kq;
      const bool in = kk < kend;
      wv[u] = buffer_load16(rW, (in && w_ok) ? w_row + (uint32_t)kk * 2u : kOOB);
      xv[u] = buffer_load16(rX, (in && x_ok) ? x_row + (uint32_t)kk * 2u : kOOB);
    }
#pragma unroll
    for (int u = 0; u < kDecodeUnroll; ++u)
      acc = mfma16(__builtin_bit_cast(V8, wv[u]), __builtin_bit_cast(V8, xv[u]), acc);
  }

  red[wave][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
  f32x4 s = red[0][lane];
#pragma unroll
  for (int w = 1; w < kDecodeWaves; ++w) s += red[w][lane];

  // lane holds D[i = 4*(lane/16) + r][j = lane % 16]: n = n0 + i, t = j
  const int t = r16;
  if (t >= p.M) return;
  const T* bias = (const T*)p.bias;
  T* out = (T*)p.out;
  const int epi = p.epi;
  const float brow = (epi != EPI_DEFAULT && !p.bias_per_col) ? to_f32(bias[t]) : 0.0f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int n = n0 + (lane >> 4) * 4 + r;
    if (n >= p.N) continue;
    float z = s[r];
    if (epi != EPI_DEFAULT) z += p.bias_per_col ? to_f32(bias[n]) : brow;
    float y = z;
    if (epi == EPI_GELU_BIAS) y = gelu_erf(z);
    else if (epi == EPI_RELU_BIAS) y = z > 0.0f ? z : 0.0f;
    out[(size_t)t * p.ldo + n] = from_f32<T>(y);
  }
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t s) {
  const int blocks = (a.N + 15) / 16;
  if (dtype == DT_F16)
    hipLaunchKernelGGL(decode_kernel<_Float16>, dim3(blocks), dim3(kDecodeWaves * 64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_kernel<__bf16>, dim3(blocks), dim3(kDecodeWaves * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace gemmepi
