// RMSNorm of float32 rows: y = x / sqrt(mean(x^2) + eps) * g, g = w or 1 + w.
//
// DantinoX "Core Layers" page, Normalisation / RMSNorm equations (eps inside
// the square root, no bias); mojolearn TransformerBlock ``norm`` parameter
// ('rmsnorm_offset' scales by 1 + w).  One workgroup per row: the row is read
// once into registers (float4 loads), the sum of squares is reduced across the
// wavefront with lane shuffles and across waves through LDS, and the scaled
// row is written in the GEMM operand type.  The same pass flags non-finite
// inputs (a plain store of 1 into a status word) at no extra bytes.  A
// second entry point first forms the row as a residual plus the K-split
// partial sums of the o_proj GEMM (fusing that GEMM's reduction).
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int NT = 256;
constexpr int MAXV = 8;  // float4 per thread held in registers: rows up to 8192

template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, float a, float b, float c, float d);
template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{from_f32<bf16>(a), from_f32<bf16>(b), from_f32<bf16>(c),
                                        from_f32<bf16>(d)};
}

// Vector path: d % 4 == 0 and d <= NT * 4 * MAXV.
// sum over z < splits of p[z * stride] (4 floats), in split order; the loads of
// 8 splits are issued together (indices clamp, surplus terms are masked) so
// their latencies overlap instead of forming a chain.
__device__ __forceinline__ f32x4 sum_splits(const float* p, int64_t stride, int splits) {
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int z0 = 0; z0 < splits; z0 += 8) {
    f32x4 t[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) t[u] = *reinterpret_cast<const f32x4*>(p + min(z0 + u, splits - 1) * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (z0 + u < splits) acc += t[u];
  }
  return acc;
}

// With `part` set (the fused K-split reduction of the o_proj GEMM), the row is
// x[row] + sum over z < splits of part[z, row, :] and is also stored to x1.
template <typename OutT>
__global__ __launch_bounds__(NT) void rmsnorm_vec_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w, OutT* __restrict__ out,
                                                        int d, float eps, int offset, int* flag,
                                                        const float* __restrict__ part, int splits,
                                                        float* __restrict__ x1) {
  __shared__ float red[NT / WAVE];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * d;
  const int64_t pstride = (int64_t)gridDim.x * d;
  f32x4 v[MAXV];
  float ss = 0.f;
  bool bad = false;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int idx = (threadIdx.x + i * NT) * 4;
    if (idx < d) {
      v[i] = *reinterpret_cast<const f32x4*>(xr + idx);
      if (part) v[i] += sum_splits(part + row * d + idx, pstride, splits);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ss += v[i][e] * v[i][e];
        bad |= !__builtin_isfinite(v[i][e]);
      }
    }
  }
  const float tot = block_sum<NT>(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  OutT* o = out + row * d;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int idx = (threadIdx.x + i * NT) * 4;
    if (idx < d) {
      if (part) *reinterpret_cast<f32x4*>(x1 + row * d + idx) = v[i];
      f32x4 g = *reinterpret_cast<const f32x4*>(w + idx);
      if (offset) g = g + 1.0f;
      store4<OutT>(o + idx, v[i][0] * r * g[0], v[i][1] * r * g[1], v[i][2] * r * g[2], v[i][3] * r * g[3]);
    }
  }
  if (bad && flag) *flag = 1;
}

// Generic path: any d (two reads of the row).
template <typename OutT>
__global__ __launch_bounds__(NT) void rmsnorm_any_kernel(const float* __restrict__ x,
                                                        const float* __restrict__ w, OutT* __restrict__ out,
                                                        int d, float eps, int offset, int* flag) {
  __shared__ float red[NT / WAVE];
  const int64_t row = blockIdx.x;
  const float* xr = x + row * d;
  float ss = 0.f;
  bool bad = false;
  for (int i = threadIdx.x; i < d; i += NT) {
    const float t = xr[i];
    ss += t * t;
    bad |= !__builtin_isfinite(t);
  }
  const float tot = block_sum<NT>(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)d + eps);
  for (int i = threadIdx.x; i < d; i += NT) {
    const float g = offset ? 1.0f + w[i] : w[i];
    out[row * d + i] = from_f32<OutT>(xr[i] * r * g);
  }
  if (bad && flag) *flag = 1;
}

template <typename OutT>
hipError_t launch_t(const float* x, const float* w, void* out, int rows, int d, float eps, int offset,
                    int* flag, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 4 == 0 && d <= NT * 4 * MAXV)
    hipLaunchKernelGGL(rmsnorm_vec_kernel<OutT>, dim3(rows), dim3(NT), 0, s, x, w,
                       static_cast<OutT*>(out), d, eps, offset, flag, nullptr, 0, nullptr);
  else
    hipLaunchKernelGGL(rmsnorm_any_kernel<OutT>, dim3(rows), dim3(NT), 0, s, x, w,
                       static_cast<OutT*>(out), d, eps, offset, flag);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm(const float* x, const float* w, void* out, int out_type, int rows, int d,
                          float eps, int offset, int* flag, hipStream_t s) {
  return out_type == kBF16 ? launch_t<bf16>(x, w, out, rows, d, eps, offset, flag, s)
                           : launch_t<float>(x, w, out, rows, d, eps, offset, flag, s);
}

bool rmsnorm_fuses_reduce(int d) { return d % 4 == 0 && d <= NT * 4 * MAXV; }

hipError_t launch_resid_rmsnorm(const float* part, int splits, const float* resid, float* x1, const float* w,
                                void* out, int out_type, int rows, int d, float eps, int offset, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!rmsnorm_fuses_reduce(d) || splits < 1 || !part || !x1) return hipErrorInvalidValue;
  if (out_type == kBF16)
    hipLaunchKernelGGL(rmsnorm_vec_kernel<bf16>, dim3(rows), dim3(NT), 0, s, resid, w, static_cast<bf16*>(out), d,
                       eps, offset, nullptr, part, splits, x1);
  else
    hipLaunchKernelGGL(rmsnorm_vec_kernel<float>, dim3(rows), dim3(NT), 0, s, resid, w, static_cast<float*>(out), d,
                       eps, offset, nullptr, part, splits, x1);
  return hipGetLastError();
}

}  // namespace gqa
