// float32 "TN" GEMM for float32 blocks: C[m, n] = sum_k A[m, k] * W[n, k],
// any M, N, K, same B-row layouts and epilogues as the bf16 matrix-core
// kernel.  gfx950's float32 matrix and vector peaks are equal (157 TFLOP/s),
// so this path uses plain FMAs: a 64 x 64 output tile per 256-thread
// workgroup, K in steps of 16 through LDS (k-major so each thread reads its
// 4 rows / 4 columns as broadcasts), 4 x 4 outputs per thread.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int TM = 64, TN = 64, TK = 16, PAD = 4;

__device__ __forceinline__ const float* brow_f32(const GemmArgs& a, int mode, int which, int64_t n) {
  if (mode == kModeGated) return static_cast<const float*>(a.B[which]) + n * a.K;
  const int s = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
  const int64_t start = s == 0 ? 0 : a.seg_end[s - 1];
  return static_cast<const float*>(a.B[s]) + (n - start) * a.K;
}

template <int MODE, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int NB = MODE == kModeGated ? 2 : 1;
  __shared__ float As[TK][TM + PAD];
  __shared__ float Bs[NB][TK][TN + PAD];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int m0 = blockIdx.y * TM, n0 = blockIdx.x * TN;
  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.bump_n; i += 256) a.bump[i] += a.bump_by;

  // Each thread stages 4 elements of A and 4 of each B per K step.
  const float* A = static_cast<const float*>(a.A);
  const float* brows[NB][4];
  int lrow[4], lk[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + 256 * i;
    lrow[i] = e / TK;
    lk[i] = e % TK;
    const int64_t n = min((int64_t)n0 + lrow[i], (int64_t)a.N - 1);
#pragma unroll
    for (int w = 0; w < NB; ++w) brows[w][i] = brow_f32(a, MODE, w, n);
  }
  float acc[NB][4][4] = {};
  for (int k0 = 0; k0 < a.K; k0 += TK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = k0 + lk[i];
      const int m = m0 + lrow[i];
      As[lk[i]][lrow[i]] = (m < a.M && k < a.K) ? A[(int64_t)m * a.lda + k] : 0.f;
#pragma unroll
      for (int w = 0; w < NB; ++w) Bs[w][lk[i]][lrow[i]] = (k < a.K) ? brows[w][i][k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float av[4], bv[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty + 16 * i];
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[w][j] = Bs[w][k][tx + 16 * j];
#pragma unroll
      for (int w = 0; w < NB; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[w][i][j] = fmaf(av[i], bv[w][j], acc[w][i][j]);
    }
    __syncthreads();
  }
  float* C = static_cast<float*>(a.C);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty + 16 * i;
    if (m >= a.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx + 16 * j;
      if (n >= a.N) continue;
      if (EPI == kEpiGated) {
        const float g = acc[0][i][j] + (a.bias[0] ? a.bias[0][n] : 0.f);
        const float u = acc[NB - 1][i][j] + (a.bias[1] ? a.bias[1][n] : 0.f);
        C[m * a.ldc + n] = act_fn(a.act, g) * u;
      } else if (EPI == kEpiResid) {
        const float v = acc[0][i][j] + (a.bias[0] ? a.bias[0][n] : 0.f);
        C[m * a.ldc + n] = a.resid ? a.resid[m * a.ldr + n] + v : v;
      } else {
        const int s = n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
        const float b = a.bias[s] ? a.bias[s][n - (s == 0 ? 0 : a.seg_end[s - 1])] : 0.f;
        const float v = acc[0][i][j] + b;
        C[m * a.ldc + n] = a.act != kActNone ? act_fn(a.act, v) : v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmArgs& a, int mode, int epi, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  dim3 grid((a.N + TN - 1) / TN, (a.M + TM - 1) / TM);
  if (mode == kModeGated) {
    if (epi != kEpiGated) return hipErrorInvalidValue;
    hipLaunchKernelGGL((gemm_f32_kernel<kModeGated, kEpiGated>), grid, dim3(256), 0, s, a);
  } else if (epi == kEpiResid) {
    hipLaunchKernelGGL((gemm_f32_kernel<kModeSeg, kEpiResid>), grid, dim3(256), 0, s, a);
  } else if (epi == kEpiStore) {
    hipLaunchKernelGGL((gemm_f32_kernel<kModeSeg, kEpiStore>), grid, dim3(256), 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqa
