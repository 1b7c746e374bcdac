// Row normalisation of float32 rows, with the residual and projection
// plumbing around it fused into the same pass.
//
// Norm kinds (mojolearn TransformerBlock ``norm``; formulas of the DantinoX
// "Core Layers" page, Normalisation):
//   RMSNorm      y = x / sqrt(mean(x^2) + eps) * g, g = w (or 1 + w, 'rmsnorm_offset')
//   LayerNorm    y = (x - mu) / sqrt(var + eps) * w (+ b), var the population
//                variance (mean of squared deviations)
// A launch applies, per row, in this order (each step optional):
//   t = x, or the sum over z of part[z] (+ bias)   part = K-split partials
//   t = out_norm(t)                                sandwich norm of a sublayer output
//   t = resid + t; x1 = t                          residual add, stored float32
//   out = norm(t)                                  the next GEMM's operand
// which covers the block's input norm, the post-attention norm, the decode
// form that also sums the o_proj GEMM's K-split partials, and Gemma's
// sandwich norms (post_attention_layernorm on the attention output,
// post_feedforward_layernorm on the MLP output; the dew DecoderBlock page's
// output norms).  Non-finite values of x set a status word (a plain store).
//
// Rows with d % 4 == 0 (up to 16384) are held in registers (float4 loads) by
// one workgroup; other rows (up to 12288) are staged in LDS.  Reductions:
// lane shuffles within a wavefront, LDS across the 4 wavefronts.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int NT = 256;

template <typename OutT>
__device__ __forceinline__ void store4(OutT* p, f32x4 v);
template <>
__device__ __forceinline__ void store4<float>(float* p, f32x4 v) {
  *reinterpret_cast<f32x4*>(p) = v;
}
template <>
__device__ __forceinline__ void store4<bf16>(bf16* p, f32x4 v) {
  *reinterpret_cast<bf16x4*>(p) = bf16x4{from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]),
                                        from_f32<bf16>(v[3])};
}

// Statistics of a row: y = (v - shift) * r * g (+ b).
struct RowStats {
  float shift, r;
};

template <int MAXV>
__device__ __forceinline__ RowStats stats_vec(const f32x4 (&v)[MAXV], int d, float eps, int kind, float* red) {
  float shift = 0.f;
  if (kind == kNormLayer) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)  // pieces past the row add nothing (they may hold a previous norm's value)
      s += (threadIdx.x + i * NT) * 4 < d ? (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]) : 0.f;
    shift = block_sum<NT>(s, red) / (float)d;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const float live = (threadIdx.x + i * NT) * 4 < d ? 1.f : 0.f;  // pieces past the row add nothing
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float c = (v[i][e] - shift) * live;
      ss += c * c;
    }
  }
  return RowStats{shift, 1.0f / sqrtf(block_sum<NT>(ss, red) / (float)d + eps)};
}

__device__ __forceinline__ f32x4 norm4(f32x4 v, RowStats st, const NormSpec& n, int idx) {
  f32x4 g = *reinterpret_cast<const f32x4*>(n.w + idx);
  if (n.kind == kNormRmsOffset) g = g + 1.0f;
  f32x4 y;
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = (v[e] - st.shift) * st.r * g[e];
  if (n.b) y += *reinterpret_cast<const f32x4*>(n.b + idx);
  return y;
}

// MAXV float4 per thread held in registers: rows up to NT * 4 * MAXV.  The
// steps a launch uses are template flags (PART: the row comes from K-split
// partials instead of x; ONORM: sandwich output norm; NORM: the operand norm),
// so each form compiles to straight-line code without the others' registers.
template <typename OutT, int MAXV, bool PART, bool ONORM, bool NORM>
__global__ __launch_bounds__(NT) void norm_vec_kernel(NormArgs a) {
  __shared__ float red[NT / WAVE];
  const int d = a.d;
  const int64_t row = blockIdx.x;
  const int64_t off = row * d;
  const int64_t pstride = (int64_t)gridDim.x * d;
  // Piece i of this thread is columns idx(i) .. idx(i) + 3.  Loads are
  // unconditional at a clamped column (d % 4 == 0, so d - 4 is a piece) and
  // out-of-row pieces are zeroed by a select: branch-free code keeps the row
  // in registers instead of copying it at every conditional load.
  int ci[MAXV];
  bool in[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int idx = (threadIdx.x + i * NT) * 4;
    in[i] = idx < d;
    ci[i] = in[i] ? idx : d - 4;
  }
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
  auto ld = [&](const float* p, int i) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p + ci[i]);
    return in[i] ? t : zero;
  };
  f32x4 v[MAXV];
  bool bad = false;
  if constexpr (!PART) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) v[i] = ld(a.x + off, i);
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) bad |= !__builtin_isfinite(v[i][e]);  // (zeroed pieces are finite)
  } else {  // splits summed in order, U splits' loads in flight together
    constexpr int U = MAXV <= 4 ? 4 : (MAXV <= 8 ? 2 : 1);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) v[i] = zero;
#pragma unroll 1
    for (int z0 = 0; z0 < a.splits; z0 += U) {
      f32x4 t[U][MAXV];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float* pz = a.part + min(z0 + u, a.splits - 1) * pstride + off;  // clamped; surplus masked
#pragma unroll
        for (int i = 0; i < MAXV; ++i) t[u][i] = ld(pz, i);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (z0 + u < a.splits)
#pragma unroll
          for (int i = 0; i < MAXV; ++i) v[i] += t[u][i];
    }
  }
  if (a.bias) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) v[i] += ld(a.bias, i);
  }
  if constexpr (ONORM) {
    const RowStats st = stats_vec(v, d, a.eps, a.out_norm.kind, red);
#pragma unroll
    for (int i = 0; i < MAXV; ++i) v[i] = norm4(v[i], st, a.out_norm, ci[i]);
  }
  if (a.resid) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i) v[i] = ld(a.resid + off, i) + v[i];
  }
  if (a.x1) {
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (in[i]) *reinterpret_cast<f32x4*>(a.x1 + off + ci[i]) = v[i];
  }
  if constexpr (NORM) {
    const RowStats st = stats_vec(v, d, a.eps, a.norm.kind, red);
    OutT* o = static_cast<OutT*>(a.out) + off;
#pragma unroll
    for (int i = 0; i < MAXV; ++i)
      if (in[i]) store4<OutT>(o + ci[i], norm4(v[i], st, a.norm, ci[i]));
  }
  if (bad && a.flag) *a.flag = 1;
}

// Any d: the row lives in LDS (dynamic, d floats); each thread walks it with
// stride NT.
__device__ __forceinline__ RowStats stats_lds(const float* t, int d, float eps, int kind, float* red) {
  float shift = 0.f;
  if (kind == kNormLayer) {
    float s = 0.f;
    for (int i = threadIdx.x; i < d; i += NT) s += t[i];
    shift = block_sum<NT>(s, red) / (float)d;
  }
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += NT) {
    const float c = t[i] - shift;
    ss += c * c;
  }
  return RowStats{shift, 1.0f / sqrtf(block_sum<NT>(ss, red) / (float)d + eps)};
}

__device__ __forceinline__ float norm1(float v, RowStats st, const NormSpec& n, int i) {
  const float g = n.kind == kNormRmsOffset ? 1.0f + n.w[i] : n.w[i];
  const float y = (v - st.shift) * st.r * g;
  return n.b ? y + n.b[i] : y;
}

template <typename OutT>
__global__ __launch_bounds__(NT) void norm_lds_kernel(NormArgs a) {
  extern __shared__ float t[];
  __shared__ float red[NT / WAVE];
  const int d = a.d;
  const int64_t row = blockIdx.x;
  const int64_t off = row * d;
  const int64_t pstride = (int64_t)gridDim.x * d;
  bool bad = false;
  for (int i = threadIdx.x; i < d; i += NT) {
    float v = 0.f;
    if (a.x) {
      v = a.x[off + i];
      bad |= !__builtin_isfinite(v);
    }
    if (a.part)
      for (int z = 0; z < a.splits; ++z) v += a.part[z * pstride + off + i];
    if (a.bias) v += a.bias[i];
    t[i] = v;
  }
  __syncthreads();
  if (a.out_norm.w) {
    const RowStats st = stats_lds(t, d, a.eps, a.out_norm.kind, red);
    for (int i = threadIdx.x; i < d; i += NT) t[i] = norm1(t[i], st, a.out_norm, i);
    __syncthreads();
  }
  for (int i = threadIdx.x; i < d; i += NT) {
    if (a.resid) t[i] = a.resid[off + i] + t[i];
    if (a.x1) a.x1[off + i] = t[i];
  }
  __syncthreads();
  if (a.norm.w) {
    const RowStats st = stats_lds(t, d, a.eps, a.norm.kind, red);
    OutT* o = static_cast<OutT*>(a.out) + off;
    for (int i = threadIdx.x; i < d; i += NT) o[i] = from_f32<OutT>(norm1(t[i], st, a.norm, i));
  }
  if (bad && a.flag) *a.flag = 1;
}

template <typename OutT, int MAXV>
hipError_t launch_vec(const NormArgs& a, int rows, hipStream_t s) {
  const bool part = a.part != nullptr, onorm = a.out_norm.w != nullptr, norm = a.norm.w != nullptr;
#define GQA_NORM_VEC(P, O, N)                                                                   \
  if (part == P && onorm == O && norm == N) {                                                  \
    hipLaunchKernelGGL((norm_vec_kernel<OutT, MAXV, P, O, N>), dim3(rows), dim3(NT), 0, s, a); \
    return hipGetLastError();                                                                  \
  }
  GQA_NORM_VEC(false, false, true)   // input / post-attention norm
  GQA_NORM_VEC(true, false, true)    // x1 = resid + sum of o_proj partials, then the norm
  GQA_NORM_VEC(false, true, true)    // sandwich: x1 = resid + onorm(o_proj), then the norm
  GQA_NORM_VEC(true, true, true)
  GQA_NORM_VEC(false, true, false)   // sandwich: y = x1 + onorm(down)
  GQA_NORM_VEC(true, true, false)
#undef GQA_NORM_VEC
  return hipErrorInvalidValue;
}

}  // namespace

// Register rows up to 16384 (d % 4 == 0); LDS rows (other d) up to 12288
// floats (48 KB of the workgroup's LDS).
bool norm_supported(int d) { return d > 0 && (d % 4 == 0 ? d <= NT * 4 * 16 : d <= 12288); }

hipError_t launch_norm(const NormArgs& a, int out_type, int rows, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (!norm_supported(a.d) || (a.part && a.splits < 1) || (a.norm.w && !a.out) || (!a.x && !a.part))
    return hipErrorInvalidValue;
  if (!a.norm.w && !a.out_norm.w) return hipErrorInvalidValue;
  const bool bf = out_type == kBF16;
  // the smallest register row that holds d
  if (a.d % 4 == 0) {
    if (a.d <= NT * 4 * 2) return bf ? launch_vec<bf16, 2>(a, rows, s) : launch_vec<float, 2>(a, rows, s);
    if (a.d <= NT * 4 * 4) return bf ? launch_vec<bf16, 4>(a, rows, s) : launch_vec<float, 4>(a, rows, s);
    if (a.d <= NT * 4 * 8) return bf ? launch_vec<bf16, 8>(a, rows, s) : launch_vec<float, 8>(a, rows, s);
    return bf ? launch_vec<bf16, 16>(a, rows, s) : launch_vec<float, 16>(a, rows, s);
  }
  const size_t lds = (size_t)a.d * 4;
  if (bf)
    hipLaunchKernelGGL(norm_lds_kernel<bf16>, dim3(rows), dim3(NT), lds, s, a);
  else
    hipLaunchKernelGGL(norm_lds_kernel<float>, dim3(rows), dim3(NT), lds, s, a);
  return hipGetLastError();
}

}  // namespace gqa
