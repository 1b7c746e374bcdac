// Device helpers shared by the block's HIP kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define WAVE 64

namespace gqa {

// Storage conversions.  bf16 -> f32 is exact; f32 -> bf16 rounds to nearest
// even (the hardware conversion on gfx950).
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// e^x through the hardware base-2 exponential: e^x = 2^(x log2 e).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
constexpr float kLog2e = 1.4426950408889634f;

// 1 / x with the hardware reciprocal (1 ulp): the elementwise activations are
// rounded to bf16 (or feed bf16 products) right after, so IEEE division's
// ~10-instruction sequence buys nothing.  rcp(inf) = 0.
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from its definition tanh(x) = 1 - 2 / (e^{2x} + 1); saturates to +-1
// (e^{2x} -> inf gives 1, e^{2x} -> 0 gives -1).
__device__ __forceinline__ float tanh_exp(float x) {
  float e = exp2_fast(2.0f * kLog2e * x);
  return 1.0f - 2.0f * rcp_fast(e + 1.0f);
}

// Logistic sigmoid 1 / (1 + e^{-z}) and SiLU(z) = z * sigmoid(z).
__device__ __forceinline__ float sigmoid(float z) { return rcp_fast(1.0f + exp2_fast(-kLog2e * z)); }
__device__ __forceinline__ float silu(float z) { return z * sigmoid(z); }

// GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).
__device__ __forceinline__ float gelu_tanh(float z) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  float u = c * (z + 0.044715f * z * z * z);
  return 0.5f * z * (1.0f + tanh_exp(u));
}

// GELU, exact form: z * Phi(z) = 0.5 z (1 + erf(z / sqrt(2))) (DantinoX
// "Core Layers" page, Feed-Forward Network / GELU; erff from the device math
// library).
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.7071067811865476f)); }

// The MLP activation named by an ActKind value (launch.h).
__device__ __forceinline__ float act_fn(int act, float g) {
  if (act == kActGeluTanh) return gelu_tanh(g);
  if (act == kActGelu) return gelu_erf(g);
  if (act == kActNone) return g;
  return silu(g);
}
template <int ACT>
__device__ __forceinline__ float act_t(float g) {
  if constexpr (ACT == kActGeluTanh) return gelu_tanh(g);
  else if constexpr (ACT == kActGelu) return gelu_erf(g);
  else if constexpr (ACT == kActNone) return g;
  else return silu(g);
}
template <int V>
struct IntC {
  static constexpr int value = V;
};
// Calls f(IntC<ACT>{}) for the run-time activation, so an epilogue loop is
// compiled once per activation with no per-element branch.
template <typename F>
__device__ __forceinline__ void with_act(int act, F&& f) {
  switch (act) {
    case kActGeluTanh: f(IntC<kActGeluTanh>{}); break;
    case kActGelu: f(IntC<kActGelu>{}); break;
    case kActNone: f(IntC<kActNone>{}); break;
    default: f(IntC<kActSilu>{}); break;
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Value of lane (l ^ 32): the gfx950 swap of the upper half of one register
// with the lower half of another (v_permlane32_swap), no LDS round trip.
// Start position of row b for a call of L tokens, from the device lengths.
// A start that would put a position below zero or at / past `limit` (the
// cache capacity without a window, else the RoPE tables' rows) is clamped
// into range, so no access leaves the cache or the tables, and *flag (if
// given) is set; the host reports it as a position error.  The host checks
// its own mirror of the lengths before every call; this guards replays of
// captured steps, which advance only the device copy.
__device__ __forceinline__ int guarded_start(const int* lengths, int b, int L, int limit, int* flag) {
  const int s = lengths ? lengths[b] : 0;
  const int hi = max(limit - L, 0);
  if (s < 0 || s > hi) {
    if (flag) *flag = 1;
    return min(max(s, 0), hi);
  }
  return s;
}
// The limit above for a cache of `cap` slots (window 0: slot = position) and
// tables of max_pos rows.
__device__ __forceinline__ int position_limit(int window, int cap, int max_pos) {
  return window > 0 ? max_pos : min(cap, max_pos);
}

__device__ __forceinline__ float xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// All-reduce sum over each row of 16 lanes with DPP moves (no LDS):
// quad_perm [1,0,3,2] and [2,3,0,1], then row_half_mirror and row_mirror.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  return x;
}

// Sum over a workgroup of NT threads (NT a multiple of 64, <= 1024).
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  if (l == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / WAVE; ++i) t += red[i];
  __syncthreads();
  return t;
}

}  // namespace gqa
