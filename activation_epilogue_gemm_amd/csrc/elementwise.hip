// Unfused baseline: the separate elementwise kernels that follow a plain
// GEMM when the epilogue is not fused.  Each one reads the GEMM result from
// HBM and writes it back, which is the traffic and the extra launches the
// fused kernel removes ("Fusing bias addition with matrix multiplication
// using nvmath-python", paragraph 1; ops-nn MatMul fusion article, section
// "Level 1: basic fusion", the three-step native flow).  They are written
// to stream at HBM speed (128-bit accesses, grid-stride loops) so that the
// measured fusion gain is against a competent baseline.
//
// Also the fp32 zero-fill used before the bias-gradient reduction and the
// row-statistics accumulation (a kernel, not hipMemsetAsync, so that a
// captured stream replays it correctly), and the row norm that finishes
// the structurally fused GEMM + residual + norm operator.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_mfma.hpp"
#include "kernels.h"

namespace gemmepi {

namespace {

constexpr int kThreads = 256;

inline int grid_for(int64_t work, int64_t per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

template <typename T>
__device__ __forceinline__ void unpack8(u32x4 w, float (&f)[8]) {
  const T* h = reinterpret_cast<const T*>(&w);
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = to_f32(h[e]);
}
template <typename T>
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 w;
  T* h = reinterpret_cast<T*>(&w);
#pragma unroll
  for (int e = 0; e < 8; ++e) h[e] = from_f32<T>(f[e]);
  return w;
}

// out = round(out + bias); 8 elements per thread when rows are 16 B aligned.
template <typename T>
__global__ void bias_add_kernel(T* out, const T* bias, int M, int N, int ldo, int per_col, int vec) {
  const int cpr = vec ? N / 8 : N;
  const int64_t total = (int64_t)M * cpr;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = c / cpr;
    const int j = (int)(c - m * cpr);
    if (vec) {
      const int n = j * 8;
      u32x4* ptr = (u32x4*)(out + m * ldo + n);
      float f[8];
      unpack8<T>(*ptr, f);
      const float bm = per_col ? 0.0f : to_f32(bias[m]);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] += per_col ? to_f32(bias[n + e]) : bm;
      *ptr = pack8<T>(f);
    } else {
      T* q = out + m * ldo + j;
      *q = from_f32<T>(to_f32(*q) + to_f32(per_col ? bias[j] : bias[m]));
    }
  }
}

// In-place ReLU or GELU, no mask; with zsave the pre-activation is first
// copied there (GELU_AUX_BIAS).
template <typename T>
__global__ void act_kernel(T* out, T* zsave, int M, int N, int ldo, int epi, int vec) {
  const int cpr = vec ? N / 8 : N;
  const int64_t total = (int64_t)M * cpr;
  const bool gelu = epi == EPI_GELU_BIAS || epi == EPI_GELU_AUX_BIAS;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = c / cpr;
    const int j = (int)(c - m * cpr);
    if (vec) {
      u32x4* ptr = (u32x4*)(out + m * ldo + j * 8);
      const u32x4 zw = *ptr;
      if (zsave) *(u32x4*)(zsave + m * ldo + j * 8) = zw;
      float f[8];
      unpack8<T>(zw, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = gelu ? gelu_erf(f[e]) : (f[e] > 0.0f ? f[e] : 0.0f);
      *ptr = pack8<T>(f);
    } else {
      T* q = out + m * ldo + j;
      if (zsave) zsave[m * ldo + j] = *q;
      const float z = to_f32(*q);
      *q = from_f32<T>(gelu ? gelu_erf(z) : (z > 0.0f ? z : 0.0f));
    }
  }
}

// out = round(out * gelu'(z)), z the saved pre-activation (unfused DGELU).
template <typename T>
__global__ void dgelu_apply_kernel(T* out, const T* z, int M, int N, int ldo, int vec) {
  const int cpr = vec ? N / 8 : N;
  const int64_t total = (int64_t)M * cpr;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = c / cpr;
    const int j = (int)(c - m * cpr);
    if (vec) {
      const int64_t at = m * ldo + j * 8;
      float f[8], zz[8];
      unpack8<T>(*(const u32x4*)(out + at), f);
      unpack8<T>(*(const u32x4*)(z + at), zz);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= gelu_grad(zz[e]);
      *(u32x4*)(out + at) = pack8<T>(f);
    } else {
      const int64_t at = m * ldo + j;
      out[at] = from_f32<T>(to_f32(out[at]) * gelu_grad(to_f32(z[at])));
    }
  }
}

// In-place ReLU that also writes the packed mask.  Four consecutive lanes
// own the 32 columns of one mask word (8 each) and OR their bytes together;
// every row is padded to aux_ld words so groups never straddle rows.
template <typename T>
__global__ void relu_mask_kernel(T* out, uint32_t* aux, int M, int N, int ldo, int aux_ld,
                                 int aux_words, int vec) {
  const int64_t slots_per_row = (int64_t)aux_words * 4;
  const int64_t total = (int64_t)M * slots_per_row;
  for (int64_t s = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; s < total;
       s += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = s / slots_per_row;
    const int rem = (int)(s - m * slots_per_row);
    const int word = rem >> 2, sub = rem & 3;
    const int n = word * 32 + sub * 8;
    uint32_t bits = 0;
    if (vec && n + 8 <= N) {
      u32x4* ptr = (u32x4*)(out + m * ldo + n);
      float f[8];
      unpack8<T>(*ptr, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bits |= (f[e] > 0.0f ? 1u : 0u) << e;
        f[e] = f[e] > 0.0f ? f[e] : 0.0f;
      }
      *ptr = pack8<T>(f);
    } else {
      for (int e = 0; e < 8 && n + e < N; ++e) {
        T* q = out + m * ldo + n + e;
        const float z = to_f32(*q);
        bits |= (z > 0.0f ? 1u : 0u) << e;
        *q = from_f32<T>(z > 0.0f ? z : 0.0f);
      }
    }
    uint32_t w = bits << (sub * 8);
    w |= __shfl_xor(w, 1);
    w |= __shfl_xor(w, 2);
    if (sub == 0) {
      uint32_t* row = aux + m * aux_ld;
      row[word] = w;
      if (word == aux_words - 1)
        for (int x = aux_words; x < aux_ld; ++x) row[x] = 0u;
    }
  }
}

// dZ = mask ? G : 0, in place.
template <typename T>
__global__ void mask_apply_kernel(T* out, const uint32_t* aux, int M, int N, int ldo, int aux_ld,
                                  int vec) {
  const int cpr = vec ? N / 8 : N;
  const int64_t total = (int64_t)M * cpr;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = c / cpr;
    const int j = (int)(c - m * cpr);
    if (vec) {
      const int n = j * 8;
      const uint32_t w = aux[m * aux_ld + (n >> 5)] >> (n & 31);
      u32x4* ptr = (u32x4*)(out + m * ldo + n);
      float f[8];
      unpack8<T>(*ptr, f);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = ((w >> e) & 1u) ? f[e] : 0.0f;
      *ptr = pack8<T>(f);
    } else {
      const uint32_t w = aux[m * aux_ld + (j >> 5)] >> (j & 31);
      T* q = out + m * ldo + j;
      if (!(w & 1u)) *q = from_f32<T>(0.0f);
    }
  }
}

// bgrad[n] += sum over a block of rows of dz[m][n] (fp32), bgrad pre-zeroed.
// Block = 4 waves; each thread sums 8 columns over the wave's row slice,
// the 4 slices are combined in LDS, then one atomic per column per block.
constexpr int kColsumRows = 256;  // rows per block (64 per wave)

template <typename T>
__global__ void __launch_bounds__(256) colsum_kernel(const T* dz, float* bgrad, int M, int N,
                                                     int ldo) {
  __shared__ float part[4][64 * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = (blockIdx.x * 64 + lane) * 8;
  const int m_beg = blockIdx.y * kColsumRows + wave * (kColsumRows / 4);
  const int m_end = min(M, m_beg + kColsumRows / 4);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (n < N) {
    int m = m_beg;
    for (; m + 8 <= m_end; m += 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const u32x4*)(dz + (int64_t)(m + u) * ldo + n);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float f[8];
        unpack8<T>(v[u], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f[e];
      }
    }
    for (; m < m_end; ++m) {
      float f[8];
      unpack8<T>(*(const u32x4*)(dz + (int64_t)m * ldo + n), f);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += f[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[wave][lane * 8 + e] = acc[e];
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 8; i += 256) {
    const int col = blockIdx.x * 512 + i;
    if (col < N) unsafeAtomicAdd(&bgrad[col], part[0][i] + part[1][i] + part[2][i] + part[3][i]);
  }
}

// Scalar fallback for rows that are not 16 B aligned: one thread per column.
template <typename T>
__global__ void colsum_scalar_kernel(const T* dz, float* bgrad, int M, int N, int ldo) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float s = 0.0f;
  for (int m = 0; m < M; ++m) s += to_f32(dz[(int64_t)m * ldo + n]);
  bgrad[n] = s;
}

// dst[n, k] = src[k, n]: a [K, N] matrix of 16-bit elements (N contiguous)
// copied to [N, K] (K contiguous), so that the tiled GEMM can read B with
// K-contiguous slabs.  One 64 x 64 tile per workgroup: 16-byte loads along
// n into LDS rows of k (padded by 16 bytes, so that the column gathers of
// the write-out hit distinct banks), then 16-byte stores along k.  K and N
// are multiples of 8, so no 16-byte chunk straddles an edge.
constexpr int kTr = 64;
constexpr int kTrPad = kTr + 8;  // LDS row pitch in elements
__global__ void __launch_bounds__(256) transpose16_kernel(const uint16_t* __restrict__ src,
                                                          uint16_t* __restrict__ dst, int K, int N,
                                                          int tiles_n) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kTr][kTrPad];  // [k][n]
  const int tk = blockIdx.x / tiles_n, tn = blockIdx.x - tk * tiles_n;
  const int k0 = tk * kTr, n0 = tn * kTr;
  const int t = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = t + 256 * j;
    const int kr = c >> 3, cc = c & 7;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + kr < K && n0 + cc * 8 < N)
      v = *(const u32x4*)(src + (size_t)(k0 + kr) * N + n0 + cc * 8);
    *(u32x4*)&tile[kr][cc * 8] = v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = t + 256 * j;
    const int nr = c >> 3, kc = c & 7;
    if (n0 + nr >= N || k0 + kc * 8 >= K) continue;
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = tile[kc * 8 + i][nr];
    const u32x4 w = {e[0] | (uint32_t)e[1] << 16, e[2] | (uint32_t)e[3] << 16,
                     e[4] | (uint32_t)e[5] << 16, e[6] | (uint32_t)e[7] << 16};
    *(u32x4*)(dst + (size_t)(n0 + nr) * K + k0 + kc * 8) = w;
  }
}

// out = round(out + residual), both [M, ldo]; the unfused path's residual
// connection.
template <typename T>
__global__ void residual_add_kernel(T* out, const T* res, int M, int N, int ldo, int vec) {
  const int cpr = vec ? N / 8 : N;
  const int64_t total = (int64_t)M * cpr;
  for (int64_t c = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; c < total;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = c / cpr;
    const int j = (int)(c - m * cpr);
    if (vec) {
      const int64_t at = m * ldo + j * 8;
      float f[8], r[8];
      unpack8<T>(*(const u32x4*)(out + at), f);
      unpack8<T>(*(const u32x4*)(res + at), r);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] += r[e];
      *(u32x4*)(out + at) = pack8<T>(f);
    } else {
      const int64_t at = m * ldo + j;
      out[at] = from_f32<T>(to_f32(out[at]) + to_f32(res[at]));
    }
  }
}

// Sum of a double over the 256 threads of the block; every thread gets it.
__device__ __forceinline__ double block_sum256(double v, double* scratch) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

// Row norm in place (ops-nn MatMul fusion article, section "Level 2:
// structural fusion"): one block per row at a time.  The row statistics
// come from stats (fp64 sums of y and y^2 added by the GEMM epilogue) or,
// for the unfused path, from the row itself; then
//   out = (y - mean) * rstd * gamma (+ beta),  rstd = 1 / sqrt(var + eps)
// with mean = 0 and var = mean(y^2) for RMSNorm.  (mean, rstd) are written
// back to stats.
template <typename T>
__global__ void __launch_bounds__(256) norm_rows_kernel(T* out, const T* gamma, const T* beta,
                                                        double* stats, int M, int N, int ldo,
                                                        float eps, int layernorm, int from_stats,
                                                        int vec) {
  __shared__ double scratch[2][4];
  const int tid = threadIdx.x;
  for (int m = blockIdx.x; m < M; m += gridDim.x) {
    T* row = out + (size_t)m * ldo;
    double s1, s2;
    if (from_stats) {
      s1 = stats[2 * (size_t)m];
      s2 = stats[2 * (size_t)m + 1];
    } else {
      double a = 0.0, b = 0.0;
      if (vec) {
        for (int n = tid * 8; n < N; n += 256 * 8) {
          float f[8];
          unpack8<T>(*(const u32x4*)(row + n), f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a += (double)f[e];
            b += (double)f[e] * (double)f[e];
          }
        }
      } else {
        for (int n = tid; n < N; n += 256) {
          const double v = (double)to_f32(row[n]);
          a += v;
          b += v * v;
        }
      }
      s1 = block_sum256(a, scratch[0]);
      s2 = block_sum256(b, scratch[1]);
    }
    const double mean = layernorm ? s1 / N : 0.0;
    double var = s2 / N - mean * mean;
    if (var < 0.0) var = 0.0;
    const double rstd = 1.0 / sqrt(var + (double)eps);
    const float fmean = (float)mean, frstd = (float)rstd;
    if (vec) {
      for (int n = tid * 8; n < N; n += 256 * 8) {
        float f[8], g[8], bt[8];
        unpack8<T>(*(const u32x4*)(row + n), f);
        unpack8<T>(*(const u32x4*)(gamma + n), g);
        if (layernorm && beta != nullptr) unpack8<T>(*(const u32x4*)(beta + n), bt);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          f[e] = (f[e] - fmean) * frstd * g[e];
          if (layernorm && beta != nullptr) f[e] += bt[e];
        }
        *(u32x4*)(row + n) = pack8<T>(f);
      }
    } else {
      for (int n = tid; n < N; n += 256) {
        float v = (to_f32(row[n]) - fmean) * frstd * to_f32(gamma[n]);
        if (layernorm && beta != nullptr) v += to_f32(beta[n]);
        row[n] = from_f32<T>(v);
      }
    }
    __syncthreads();  // every thread has read stats[m] and scratch
    if (tid == 0) {
      stats[2 * (size_t)m] = mean;
      stats[2 * (size_t)m + 1] = rstd;
    }
  }
}
}  // namespace

hipError_t launch_transpose16(const void* src, void* dst, int K, int N, hipStream_t s) {
  if (K < 1 || N < 1 || K % 8 || N % 8) return hipErrorInvalidValue;
  const int tiles_k = (K + kTr - 1) / kTr, tiles_n = (N + kTr - 1) / kTr;
  const int64_t blocks = (int64_t)tiles_k * tiles_n;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose16_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     (const uint16_t*)src, (uint16_t*)dst, K, N, tiles_n);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_for(n, kThreads)), dim3(kThreads), 0, s, p, n, v);
  return hipGetLastError();
}

static inline int vec_ok(const void* p, int N, int ldo) {
  return ((uintptr_t)p % 16 == 0) && (N % 8 == 0) && (ldo % 8 == 0);
}

hipError_t launch_bias_add(int dtype, void* out, const void* bias, int M, int N, int ldo,
                           int per_col, hipStream_t s) {
  const int vec = vec_ok(out, N, ldo);
  const int64_t work = (int64_t)M * (vec ? N / 8 : N);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(bias_add_kernel<_Float16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0,
                       s, (_Float16*)out, (const _Float16*)bias, M, N, ldo, per_col, vec);
  else
    hipLaunchKernelGGL(bias_add_kernel<__bf16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0, s,
                       (__bf16*)out, (const __bf16*)bias, M, N, ldo, per_col, vec);
  return hipGetLastError();
}

hipError_t launch_activation(int dtype, int epi, void* out, uint32_t* aux, int M, int N, int ldo,
                             int aux_ld, hipStream_t s) {
  const int vec = vec_ok(out, N, ldo);
  void* zsave = epi == EPI_GELU_AUX_BIAS ? (void*)aux : nullptr;
  if (epi == EPI_RELU_AUX_BIAS) {
    const int aux_words = (N + 31) / 32;
    const int64_t work = (int64_t)M * aux_words * 4;
    if (dtype == DT_F16)
      hipLaunchKernelGGL(relu_mask_kernel<_Float16>, dim3(grid_for(work, kThreads)), dim3(kThreads),
                         0, s, (_Float16*)out, aux, M, N, ldo, aux_ld, aux_words, vec);
    else
      hipLaunchKernelGGL(relu_mask_kernel<__bf16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0,
                         s, (__bf16*)out, aux, M, N, ldo, aux_ld, aux_words, vec);
  } else {
    const int64_t work = (int64_t)M * (vec ? N / 8 : N);
    if (dtype == DT_F16)
      hipLaunchKernelGGL(act_kernel<_Float16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0, s,
                         (_Float16*)out, (_Float16*)zsave, M, N, ldo, epi, vec);
    else
      hipLaunchKernelGGL(act_kernel<__bf16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0, s,
                         (__bf16*)out, (__bf16*)zsave, M, N, ldo, epi, vec);
  }
  return hipGetLastError();
}

hipError_t launch_dgelu_apply(int dtype, void* out, const void* z, int M, int N, int ldo,
                              hipStream_t s) {
  const int vec = vec_ok(out, N, ldo) && ((uintptr_t)z % 16 == 0);
  const int64_t work = (int64_t)M * (vec ? N / 8 : N);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(dgelu_apply_kernel<_Float16>, dim3(grid_for(work, kThreads)),
                       dim3(kThreads), 0, s, (_Float16*)out, (const _Float16*)z, M, N, ldo, vec);
  else
    hipLaunchKernelGGL(dgelu_apply_kernel<__bf16>, dim3(grid_for(work, kThreads)),
                       dim3(kThreads), 0, s, (__bf16*)out, (const __bf16*)z, M, N, ldo, vec);
  return hipGetLastError();
}

hipError_t launch_mask_apply(int dtype, void* out, const uint32_t* aux, int M, int N, int ldo,
                             int aux_ld, hipStream_t s) {
  const int vec = vec_ok(out, N, ldo);
  const int64_t work = (int64_t)M * (vec ? N / 8 : N);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(mask_apply_kernel<_Float16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0,
                       s, (_Float16*)out, aux, M, N, ldo, aux_ld, vec);
  else
    hipLaunchKernelGGL(mask_apply_kernel<__bf16>, dim3(grid_for(work, kThreads)), dim3(kThreads), 0,
                       s, (__bf16*)out, aux, M, N, ldo, aux_ld, vec);
  return hipGetLastError();
}

hipError_t launch_colsum(int dtype, const void* dz, float* bgrad, int M, int N, int ldo,
                         hipStream_t s) {
  if (vec_ok(dz, N, ldo)) {
    dim3 grid((N / 8 + 63) / 64, (M + kColsumRows - 1) / kColsumRows);
    if (dtype == DT_F16)
      hipLaunchKernelGGL(colsum_kernel<_Float16>, grid, dim3(256), 0, s, (const _Float16*)dz, bgrad, M,
                         N, ldo);
    else
      hipLaunchKernelGGL(colsum_kernel<__bf16>, grid, dim3(256), 0, s, (const __bf16*)dz, bgrad, M, N,
                         ldo);
  } else {
    if (dtype == DT_F16)
      hipLaunchKernelGGL(colsum_scalar_kernel<_Float16>, dim3((N + 255) / 256), dim3(256), 0, s,
                         (const _Float16*)dz, bgrad, M, N, ldo);
    else
      hipLaunchKernelGGL(colsum_scalar_kernel<__bf16>, dim3((N + 255) / 256), dim3(256), 0, s,
                         (const __bf16*)dz, bgrad, M, N, ldo);
  }
  return hipGetLastError();
}

hipError_t launch_residual_add(int dtype, void* out, const void* residual, int M, int N, int ldo,
                               hipStream_t s) {
  const int vec = vec_ok(out, N, ldo) && ((uintptr_t)residual % 16 == 0);
  const int64_t work = (int64_t)M * (vec ? N / 8 : N);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(residual_add_kernel<_Float16>, dim3(grid_for(work, kThreads)),
                       dim3(kThreads), 0, s, (_Float16*)out, (const _Float16*)residual, M, N, ldo,
                       vec);
  else
    hipLaunchKernelGGL(residual_add_kernel<__bf16>, dim3(grid_for(work, kThreads)),
                       dim3(kThreads), 0, s, (__bf16*)out, (const __bf16*)residual, M, N, ldo,
                       vec);
  return hipGetLastError();
}

hipError_t launch_norm_rows(int dtype, void* out, const void* gamma, const void* beta,
                            double* stats, int M, int N, int ldo, float eps, int layernorm,
                            int from_stats, hipStream_t s) {
  const int vec = vec_ok(out, N, ldo) && ((uintptr_t)gamma % 16 == 0) &&
                  (beta == nullptr || (uintptr_t)beta % 16 == 0);
  const dim3 grid(M < 65536 ? M : 65536), block(256);
  if (dtype == DT_F16)
    hipLaunchKernelGGL(norm_rows_kernel<_Float16>, grid, block, 0, s, (_Float16*)out,
                       (const _Float16*)gamma, (const _Float16*)beta, stats, M, N, ldo, eps,
                       layernorm, from_stats, vec);
  else
    hipLaunchKernelGGL(norm_rows_kernel<__bf16>, grid, block, 0, s, (__bf16*)out,
                       (const __bf16*)gamma, (const __bf16*)beta, stats, M, N, ldo, eps, layernorm,
                       from_stats, vec);
  return hipGetLastError();
}

}  // namespace gemmepi
