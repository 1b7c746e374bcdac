// Kernels of the block's backward (gradients of a zero-state prefill:
// mojolearn TransformerBlock.backward).  The forward is recomputed with the
// forward kernels; the weight-gradient and input-gradient products run on the
// forward GEMMs ("TN": both operands K-contiguous) over transposed operands
// made here.  What is new:
//
//  * transpose_kernel: [R, C] -> [C, Rp] through a 64x64 LDS tile, zero rows
//    past R (Rp pads the token count so it can be a GEMM's K), with an element
//    type conversion (float32 GEMM outputs become bf16 operands).
//  * swiglu_bwd_kernel: a = silu(g) u and, from da, dg = da u silu'(g),
//    du = da silu(g) with silu'(g) = s (1 + g (1 - s)), s = sigmoid(g).
//  * rms_bwd_kernel: RMSNorm y = x r w, r = (mean(x^2) + eps)^(-1/2):
//    dx = r (g - x^ mean(g x^)), g = dy w, x^ = x r, plus the residual
//    gradient; dy x^ per element for the weight gradient (column sums).
//  * colsum_kernel: deterministic column sums (row chunks, then chunks in order).
//  * rope_bwd_pack_kernel: RoPE's backward is the rotation by the opposite
//    angle (DantinoX "Core Layers" page, Positional Encoding / RoPE: a 2x2
//    rotation per pair); packs dq | dk | dv into the q/k/v GEMM's row layout.
//  * attention: softmax backward dS = P (dP - D), D = rowsum(dO O) = rowsum(P dP)
//    (DantinoX page, Flash Attention: recompute P from the row's log-sum-exp
//    instead of storing it).  attn_bwd_q_kernel: one wave per (token, query
//    head): pass 1 forms the row's log-sum-exp, then D, then pass 2 dq.
//    attn_bwd_kv_kernel: one wave per (row, key, kv head): dk and dv summed
//    over the group's query heads and the queries that see the key.  A wave
//    splits into 4 groups of 16 lanes, each on its own key (or query); a lane
//    holds head dimensions lane % 16 + 16 i.
#include "common.h"
#include "launch.h"

#include <cstdint>

namespace gqa {
namespace {

template <typename T>
__device__ __forceinline__ float ldf(const T* p) {
  return to_f32(*p);
}
template <>
__device__ __forceinline__ float ldf<float>(const float* p) {
  return *p;
}

// ---- transpose ----
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void transpose_kernel(const TI* __restrict__ in, int64_t ld, int R, int C,
                                                       TO* __restrict__ out, int64_t ldo, int Rp) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < R && c < C) ? ldf(in + (int64_t)r * ld + c) : 0.f;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < C && r < Rp) out[(int64_t)c * ldo + r] = from_f32<TO>(tile[tx][i]);
  }
}

// Vector form: 16-byte accesses on both sides (8 elements per thread along the
// input row when loading, along the output row when storing); needs ld, ldo
// and C multiples of 8 and 16-byte aligned bases.
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16> {
  typedef bf16x8 type;
};
template <>
struct Vec8<float> {
  struct type {
    f32x4 lo, hi;
  };
};
template <typename T>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const bf16x8 x = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = to_f32(x[e]);
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = a[e];
    v[4 + e] = b[e];
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float (&v)[8]);
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float (&v)[8]) {
  bf16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = from_f32<bf16>(v[e]);
  *reinterpret_cast<bf16x8*>(p) = x;
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void transpose_vec_kernel(const TI* __restrict__ in, int64_t ld, int R, int C,
                                                           TO* __restrict__ out, int64_t ldo, int Rp) {
  __shared__ float tile[64][65];
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = threadIdx.x + 256 * pass;
    const int r = idx >> 3, c8 = (idx & 7) * 8;
    float v[8];
    if (r0 + r < R && c0 + c8 < C) {  // C % 8 == 0: the 8 columns are all in or all out
      load8<TI>(in + (int64_t)(r0 + r) * ld + c0 + c8, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][c8 + e] = v[e];
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int idx = threadIdx.x + 256 * pass;
    const int oc = idx >> 3, r8 = (idx & 7) * 8;
    const int c = c0 + oc, r = r0 + r8;
    if (c >= C || r >= Rp) continue;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[r8 + e][oc];
    TO* o = out + (int64_t)c * ldo + r;
    if (r + 8 <= Rp) {
      store8<TO>(o, v);
    } else {
      for (int e = 0; e < Rp - r; ++e) o[e] = from_f32<TO>(v[e]);
    }
  }
}

// ---- SwiGLU ----
template <typename T>
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const float* __restrict__ gu, const float* __restrict__ da,
                                                        int64_t rows, int IT, T* __restrict__ act,
                                                        T* __restrict__ dgu) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * IT) return;
  const int64_t r = i / IT;
  const int c = (int)(i % IT);
  const float g = gu[r * 2 * IT + c], u = gu[r * 2 * IT + IT + c];
  const float s = sigmoid(g);
  const float sl = g * s;
  act[i] = from_f32<T>(sl * u);
  const float d = da[i];
  dgu[r * 2 * IT + c] = from_f32<T>(d * u * s * (1.0f + g * (1.0f - s)));
  dgu[r * 2 * IT + IT + c] = from_f32<T>(d * sl);
}

// ---- RMSNorm ----
template <typename T>
__global__ __launch_bounds__(256) void rms_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                     const float* __restrict__ w, const float* __restrict__ resid,
                                                     int d, float eps, float* __restrict__ dx, T* __restrict__ dx_op,
                                                     float* __restrict__ wpart) {
  __shared__ float red[4];
  const int64_t off = (int64_t)blockIdx.x * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) ss += x[off + i] * x[off + i];
  const float r = 1.0f / sqrtf(block_sum<256>(ss, red) / (float)d + eps);
  float gx = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) gx += dy[off + i] * w[i] * x[off + i] * r;
  const float m = block_sum<256>(gx, red) / (float)d;
  for (int i = threadIdx.x; i < d; i += 256) {
    const float xh = x[off + i] * r, g = dy[off + i] * w[i];
    const float v = resid[off + i] + r * (g - xh * m);
    dx[off + i] = v;
    if (dx_op) dx_op[off + i] = from_f32<T>(v);
    wpart[off + i] = dy[off + i] * xh;
  }
}

// Register form (d % 4 == 0, d <= 1024 * MAXV): each row read once, 16-byte
// accesses at clamped columns, out-of-row pieces zeroed by selects.
// A workgroup takes kRmsBwdRows consecutive rows and sums the weight
// gradient's summands dy * x^ of its rows per column in registers (rows in
// order), writing one partial row per chunk: the column sums then read
// rows / kRmsBwdRows partial rows instead of a [rows, d] array.
constexpr int kRmsBwdRows = 4;

template <typename T, int MAXV>
__global__ __launch_bounds__(256) void rms_bwd_vec_kernel(const float* __restrict__ dy, const float* __restrict__ x,
                                                         const float* __restrict__ w,
                                                         const float* __restrict__ resid, int rows, int d, float eps,
                                                         float* __restrict__ dx, T* __restrict__ dx_op,
                                                         float* __restrict__ wpart) {
  __shared__ float red[4];
  const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
  int ci[MAXV];
  bool in[MAXV];
  f32x4 wacc[MAXV];
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int idx = (threadIdx.x + i * 256) * 4;
    in[i] = idx < d;
    ci[i] = in[i] ? idx : d - 4;
    wacc[i] = zero;
  }
  const int row0 = blockIdx.x * kRmsBwdRows, row1 = min(rows, row0 + kRmsBwdRows);
  for (int row = row0; row < row1; ++row) {
  const int64_t off = (int64_t)row * d;
  f32x4 xv[MAXV], gv[MAXV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const f32x4 xx = *reinterpret_cast<const f32x4*>(x + off + ci[i]);
    const f32x4 yy = *reinterpret_cast<const f32x4*>(dy + off + ci[i]);
    const f32x4 ww = *reinterpret_cast<const f32x4*>(w + ci[i]);
    xv[i] = in[i] ? xx : zero;
    gv[i] = in[i] ? yy * ww : zero;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += xv[i][e] * xv[i][e];
  }
  const float r = 1.0f / sqrtf(block_sum<256>(ss, red) / (float)d + eps);
  float gx = 0.f;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) gx += gv[i][e] * xv[i][e];
  const float m = block_sum<256>(gx, red) * r / (float)d;  // mean(g x^)
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    if (!in[i]) continue;
    const f32x4 rs = *reinterpret_cast<const f32x4*>(resid + off + ci[i]);
    const f32x4 yy = *reinterpret_cast<const f32x4*>(dy + off + ci[i]);
    f32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xh = xv[i][e] * r;
      v[e] = rs[e] + r * (gv[i][e] - xh * m);
      wacc[i][e] += yy[e] * xh;
    }
    *reinterpret_cast<f32x4*>(dx + off + ci[i]) = v;
    if (dx_op) {
      T* o = dx_op + off + ci[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(v[e]);
    }
  }
  }  // row
  float* wp = wpart + (int64_t)blockIdx.x * d;
#pragma unroll
  for (int i = 0; i < MAXV; ++i)
    if (in[i]) *reinterpret_cast<f32x4*>(wp + ci[i]) = wacc[i];
}

// Column sums of a [R, C] float32 matrix: chunk z of rows -> part[z, c], then
// out[c] = sum over chunks in order.
__global__ __launch_bounds__(256) void colsum_part_kernel(const float* __restrict__ a, int R, int C, int rows_per,
                                                          float* __restrict__ part) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  const int r0 = blockIdx.y * rows_per, r1 = min(R, r0 + rows_per);
  float s = 0.f;
  // (unrolled so the loads are in flight together; the adds stay in row order)
#pragma unroll 8
  for (int r = r0; r < r1; ++r) s += a[(int64_t)r * C + c];
  part[(int64_t)blockIdx.y * C + c] = s;
}
__global__ __launch_bounds__(256) void colsum_final_kernel(const float* __restrict__ part, int nz, int C,
                                                           float* __restrict__ out) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= C) return;
  float s = 0.f;
#pragma unroll 8
  for (int z = 0; z < nz; ++z) s += part[(int64_t)z * C + c];
  out[c] = s;
}

// ---- RoPE backward + pack ----
// One thread per element of the packed row [T, ld]: columns past the q | k | v
// width are written as zeros (they pad the GEMM depth).
template <typename T>
__global__ __launch_bounds__(256) void rope_bwd_pack_kernel(BwdAttnArgs a, T* __restrict__ dqkv, int64_t ld) {
  const int hd = a.hd, half = hd / 2;
  const int64_t T_ = (int64_t)a.B * a.L;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T_ * ld) return;
  const int64_t tok = i / ld;
  const int c = (int)(i % ld);
  const int b = (int)(tok / a.L), t = (int)(tok % a.L);
  const int width = (a.H + 2 * a.KV) * hd;
  if (c >= width) {
    dqkv[i] = from_f32<T>(0.f);
    return;
  }
  const int slot = c / hd, e = c % hd;
  const float* src;
  int parts = 1;  // dk / dv: per-head partials, summed in order
  bool rot = true;
  if (slot < a.H) {
    src = a.dq + (tok * a.H + slot) * hd;
  } else if (slot < a.H + a.KV) {
    src = a.dk + (((int64_t)b * a.KV + (slot - a.H)) * a.L + t) * hd;
    parts = a.kv_parts;
  } else {
    src = a.dv + (((int64_t)b * a.KV + (slot - a.H - a.KV)) * a.L + t) * hd;
    parts = a.kv_parts;
    rot = false;
  }
  auto val = [&](int i) {
    float v = src[i];
    for (int z = 1; z < parts; ++z) v += src[z * a.kv_part_stride + i];
    return v;
  };
  float x = val(e);
  if (rot) {  // forward: y1 = x1 c - x2 s, y2 = x2 c + x1 s  ->  x = R(-angle) y
    const int p = e < half ? e : e - half;
    const float cs = a.cos_tab[(int64_t)t * half + p], sn = a.sin_tab[(int64_t)t * half + p];
    const float y1 = val(p), y2 = val(p + half);
    x = e < half ? y1 * cs + y2 * sn : y2 * cs - y1 * sn;
  }
  dqkv[i] = from_f32<T>(x);
}

// Vector form (hd % 8 == 0): a thread per 4 rotate-half pairs of one head slot
// (two 4-element stores), then threads that zero the padding 8 columns at a time.
template <typename T>
__device__ __forceinline__ void store4v(T* p, const f32x4& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{from_f32<bf16>(v[0]), from_f32<bf16>(v[1]), from_f32<bf16>(v[2]),
                                          from_f32<bf16>(v[3])};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
template <typename T>
__global__ __launch_bounds__(256) void rope_bwd_pack4_kernel(BwdAttnArgs a, T* __restrict__ dqkv, int64_t ld) {
  const int hd = a.hd, half = hd / 2, ng = half / 4;
  const int slots = a.H + 2 * a.KV;
  const int width = slots * hd;
  const int64_t T_ = (int64_t)a.B * a.L;
  const int64_t n_main = T_ * slots * ng;
  const int pad8 = (int)((ld - width) / 8);
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_main) {
    const int64_t k = i - n_main;
    if (k >= T_ * pad8) return;
    const int64_t tok = k / pad8;
    T* o = dqkv + tok * ld + width + (k % pad8) * 8;
    store4v<T>(o, f32x4{0.f, 0.f, 0.f, 0.f});
    store4v<T>(o + 4, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int g = (int)(i % ng);
  const int64_t hs = i / ng;
  const int slot = (int)(hs % slots);
  const int64_t tok = hs / slots;
  const int b = (int)(tok / a.L), t = (int)(tok % a.L);
  const int p = 4 * g;
  const float* src;
  int parts = 1;
  bool rot = true;
  if (slot < a.H) {
    src = a.dq + (tok * a.H + slot) * hd;
  } else if (slot < a.H + a.KV) {
    src = a.dk + (((int64_t)b * a.KV + (slot - a.H)) * a.L + t) * hd;
    parts = a.kv_parts;
  } else {
    src = a.dv + (((int64_t)b * a.KV + (slot - a.H - a.KV)) * a.L + t) * hd;
    parts = a.kv_parts;
    rot = false;
  }
  f32x4 y1 = *reinterpret_cast<const f32x4*>(src + p), y2 = *reinterpret_cast<const f32x4*>(src + p + half);
  for (int z = 1; z < parts; ++z) {
    y1 += *reinterpret_cast<const f32x4*>(src + z * a.kv_part_stride + p);
    y2 += *reinterpret_cast<const f32x4*>(src + z * a.kv_part_stride + p + half);
  }
  f32x4 x1 = y1, x2 = y2;
  if (rot) {  // x = R(-angle) y
    const f32x4 c = *reinterpret_cast<const f32x4*>(a.cos_tab + (int64_t)t * half + p);
    const f32x4 sn = *reinterpret_cast<const f32x4*>(a.sin_tab + (int64_t)t * half + p);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x1[e] = y1[e] * c[e] + y2[e] * sn[e];
      x2[e] = y2[e] * c[e] - y1[e] * sn[e];
    }
  }
  T* o = dqkv + tok * ld + slot * hd + p;
  store4v<T>(o, x1);
  store4v<T>(o + half, x2);
}

// Elementwise float32 -> operand type.
template <typename T>
__global__ __launch_bounds__(256) void convert_kernel(const float* __restrict__ in, T* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = from_f32<T>(in[i]);
}
// 8 elements per thread (n a multiple of 8, 16-byte aligned buffers): two
// 16-byte loads, one 16-byte store.
__global__ __launch_bounds__(256) void convert8_bf16_kernel(const float* __restrict__ in, bf16* __restrict__ out,
                                                           int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(in)[2 * i];
  const f32x4 b = reinterpret_cast<const f32x4*>(in)[2 * i + 1];
  bf16x8 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = from_f32<bf16>(a[e]);
    o[4 + e] = from_f32<bf16>(b[e]);
  }
  reinterpret_cast<bf16x8*>(out)[i] = o;
}

// ---- attention backward ----
constexpr int kMaxDpl = 16;  // head dims per lane (hd <= 256)

// 16-lane group sum (the group's lanes are adjacent and aligned).
__device__ __forceinline__ float group16_sum(float v) {
  v += __shfl_xor(v, 1, WAVE);
  v += __shfl_xor(v, 2, WAVE);
  v += __shfl_xor(v, 4, WAVE);
  v += __shfl_xor(v, 8, WAVE);
  return v;
}

template <typename T>
__device__ __forceinline__ const T* q_row(const BwdAttnArgs& a, int64_t tok, int h) {
  return static_cast<const T*>(a.q) + tok * a.ldq + (int64_t)h * a.hd;
}
template <typename T>
__device__ __forceinline__ const T* kv_row(const void* base, const BwdAttnArgs& a, int b, int j, int s) {
  return static_cast<const T*>(base) + (((int64_t)b * a.KV + j) * a.L + s) * a.hd;
}

// One wave per (token, query head).
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_q_kernel(BwdAttnArgs a) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, gl = lane & 15;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t T_ = (int64_t)a.B * a.L;
  if (wid >= T_ * a.H) return;
  const int64_t tok = wid / a.H;
  const int h = (int)(wid % a.H);
  const int b = (int)(tok / a.L), t = (int)(tok % a.L);
  const int j = h / (a.H / a.KV);
  const int dpl = (a.hd + 15) / 16;
  const float sl2 = a.scale * kLog2e;  // scores in log2 units
  float qv[kMaxDpl], dov[kMaxDpl], ov[kMaxDpl];
  const T* qp = q_row<T>(a, tok, h);
  const T* op = static_cast<const T*>(a.o) + tok * a.ldo + (int64_t)h * a.hd;
  const float* dop = a.dout + tok * a.ldo + (int64_t)h * a.hd;
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) {
    const int e = gl + 16 * i;
    const bool in = i < dpl && e < a.hd;
    qv[i] = in ? ldf(qp + e) : 0.f;
    dov[i] = in ? dop[e] : 0.f;
    ov[i] = in ? ldf(op + e) : 0.f;
  }
  const int lo = a.window > 0 ? max(0, t - a.window + 1) : 0;
  // pass 1: log-sum-exp (base 2) over keys lo..t
  float mx = -INFINITY, sum = 0.f;
  for (int s0 = lo; s0 <= t; s0 += 4) {
    const int s = s0 + grp;
    float part = 0.f;
    if (s <= t) {
      const T* kp = kv_row<T>(a.k, a, b, j, s);
#pragma unroll
      for (int i = 0; i < kMaxDpl; ++i) {
        const int e = gl + 16 * i;
        if (i < dpl && e < a.hd) part += qv[i] * ldf(kp + e);
      }
    }
    const float sc = s <= t ? group16_sum(part) * sl2 : -INFINITY;
    // combine the 4 groups' scores into the running (mx, sum)
    float m4 = fmaxf(sc, __shfl_xor(sc, 16, WAVE));
    m4 = fmaxf(m4, __shfl_xor(m4, 32, WAVE));
    const float nm = fmaxf(mx, m4);
    float e4 = s <= t ? exp2f(sc - nm) : 0.f;
    e4 += __shfl_xor(e4, 16, WAVE);
    e4 += __shfl_xor(e4, 32, WAVE);
    sum = sum * exp2f(mx - nm) + e4;
    mx = nm;
  }
  const float lse2 = mx + log2f(sum);
  // D = dO . O
  float dd = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) dd += dov[i] * ov[i];
  dd = group16_sum(dd);  // every group holds the same row
  if (lane == 0) {
    a.lse[wid] = lse2;
    a.dsum[wid] = dd;
  }
  // pass 2: dq = scale sum_s ds_s k_s, ds = p (dp - D)
  float dq[kMaxDpl];
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) dq[i] = 0.f;
  for (int s0 = lo; s0 <= t; s0 += 4) {
    const int s = s0 + grp;
    if (s > t) continue;  // (the group's lanes agree; group16_sum stays within the group)
    const T* kp = kv_row<T>(a.k, a, b, j, s);
    const T* vp = kv_row<T>(a.v, a, b, j, s);
    float kv[kMaxDpl], ps = 0.f, pd = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) {
      const int e = gl + 16 * i;
      const bool in = i < dpl && e < a.hd;
      kv[i] = in ? ldf(kp + e) : 0.f;
      ps += qv[i] * kv[i];
      pd += dov[i] * (in ? ldf(vp + e) : 0.f);
    }
    const float p = exp2f(group16_sum(ps) * sl2 - lse2);
    const float ds = p * (group16_sum(pd) - dd);
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) dq[i] += ds * kv[i];
  }
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) {
    float v = dq[i];
    v += __shfl_xor(v, 16, WAVE);
    v += __shfl_xor(v, 32, WAVE);
    dq[i] = v * a.scale;
  }
  if (grp == 0) {
    float* out = a.dq + (tok * a.H + h) * a.hd;
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) {
      const int e = gl + 16 * i;
      if (i < dpl && e < a.hd) out[e] = dq[i];
    }
  }
}

// One wave per (row, key position, kv head).
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_kv_kernel(BwdAttnArgs a) {
  const int lane = threadIdx.x & 63, grp = lane >> 4, gl = lane & 15;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t n = (int64_t)a.B * a.L * a.KV;
  if (wid >= n) return;
  const int j = (int)(wid % a.KV);
  const int64_t bs = wid / a.KV;
  const int b = (int)(bs / a.L), s = (int)(bs % a.L);
  const int G = a.H / a.KV;
  const int dpl = (a.hd + 15) / 16;
  const float sl2 = a.scale * kLog2e;
  float kv[kMaxDpl], vv[kMaxDpl], dk[kMaxDpl], dv[kMaxDpl];
  const T* kp = kv_row<T>(a.k, a, b, j, s);
  const T* vp = kv_row<T>(a.v, a, b, j, s);
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) {
    const int e = gl + 16 * i;
    const bool in = i < dpl && e < a.hd;
    kv[i] = in ? ldf(kp + e) : 0.f;
    vv[i] = in ? ldf(vp + e) : 0.f;
    dk[i] = dv[i] = 0.f;
  }
  const int hi = a.window > 0 ? min(a.L - 1, s + a.window - 1) : a.L - 1;  // last query that sees key s
  const int nq = (hi - s + 1) * G;  // (query, head) pairs, head fastest
  for (int i0 = 0; i0 < nq; i0 += 4) {
    const int idx = i0 + grp;
    if (idx >= nq) continue;
    const int t = s + idx / G, h = j * G + idx % G;
    const int64_t tok = (int64_t)b * a.L + t;
    const T* qp = q_row<T>(a, tok, h);
    const float* dop = a.dout + tok * a.ldo + (int64_t)h * a.hd;
    float qv[kMaxDpl], dov[kMaxDpl], ps = 0.f, pd = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) {
      const int e = gl + 16 * i;
      const bool in = i < dpl && e < a.hd;
      qv[i] = in ? ldf(qp + e) : 0.f;
      dov[i] = in ? dop[e] : 0.f;
      ps += qv[i] * kv[i];
      pd += dov[i] * vv[i];
    }
    const int64_t r = tok * a.H + h;
    const float p = exp2f(group16_sum(ps) * sl2 - a.lse[r]);
    const float ds = p * (group16_sum(pd) - a.dsum[r]);
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) {
      dv[i] += p * dov[i];
      dk[i] += ds * qv[i];
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxDpl; ++i) {
    float x = dk[i], y = dv[i];
    x += __shfl_xor(x, 16, WAVE);
    x += __shfl_xor(x, 32, WAVE);
    y += __shfl_xor(y, 16, WAVE);
    y += __shfl_xor(y, 32, WAVE);
    dk[i] = x * a.scale;
    dv[i] = y;
  }
  if (grp == 0) {
    const int64_t o = (((int64_t)b * a.KV + j) * a.L + s) * a.hd;
#pragma unroll
    for (int i = 0; i < kMaxDpl; ++i) {
      const int e = gl + 16 * i;
      if (i < dpl && e < a.hd) {
        a.dk[o + e] = dk[i];
        a.dv[o + e] = dv[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_transpose(const void* in, int in_type, int64_t ld, int R, int C, void* out, int out_type,
                            int64_t ldo, int Rp, hipStream_t s) {
  if (Rp <= 0 || C <= 0) return hipSuccess;
  if (Rp < R || ldo < Rp) return hipErrorInvalidValue;
  dim3 grid((C + 63) / 64, (Rp + 63) / 64);
  const size_t ie = in_type == kF32 ? 4 : 2, oe = out_type == kF32 ? 4 : 2;
  const bool vec = ld % 8 == 0 && ldo % 8 == 0 && C % 8 == 0 && reinterpret_cast<uintptr_t>(in) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out) % 16 == 0 && ie * 8 % 16 == 0 && oe * 8 % 16 == 0;
  if (vec) {
    if (in_type == kF32 && out_type == kF32)
      hipLaunchKernelGGL((transpose_vec_kernel<float, float>), grid, dim3(256), 0, s, static_cast<const float*>(in),
                         ld, R, C, static_cast<float*>(out), ldo, Rp);
    else if (in_type == kF32 && out_type == kBF16)
      hipLaunchKernelGGL((transpose_vec_kernel<float, bf16>), grid, dim3(256), 0, s, static_cast<const float*>(in),
                         ld, R, C, static_cast<bf16*>(out), ldo, Rp);
    else if (in_type == kBF16 && out_type == kBF16)
      hipLaunchKernelGGL((transpose_vec_kernel<bf16, bf16>), grid, dim3(256), 0, s, static_cast<const bf16*>(in),
                         ld, R, C, static_cast<bf16*>(out), ldo, Rp);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (in_type == kF32 && out_type == kF32)
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(256), 0, s, static_cast<const float*>(in), ld, R, C,
                       static_cast<float*>(out), ldo, Rp);
  else if (in_type == kF32 && out_type == kBF16)
    hipLaunchKernelGGL((transpose_kernel<float, bf16>), grid, dim3(256), 0, s, static_cast<const float*>(in), ld, R, C,
                       static_cast<bf16*>(out), ldo, Rp);
  else if (in_type == kBF16 && out_type == kBF16)
    hipLaunchKernelGGL((transpose_kernel<bf16, bf16>), grid, dim3(256), 0, s, static_cast<const bf16*>(in), ld, R, C,
                       static_cast<bf16*>(out), ldo, Rp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* gu, const float* da, int64_t rows, int IT, void* act, void* dgu, int elem,
                             hipStream_t s) {
  const int64_t n = rows * IT;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256));
  if (elem == kBF16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<bf16>, grid, dim3(256), 0, s, gu, da, rows, IT, static_cast<bf16*>(act),
                       static_cast<bf16*>(dgu));
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<float>, grid, dim3(256), 0, s, gu, da, rows, IT, static_cast<float*>(act),
                       static_cast<float*>(dgu));
  return hipGetLastError();
}

bool rms_bwd_vec_ok(int d) { return d % 4 == 0 && d <= 1024 * 16; }

template <typename T>
hipError_t rms_bwd_vec(const float* dy, const float* x, const float* w, const float* resid, int rows, int d, float eps,
                       float* dx, T* dx_op, float* wpart, hipStream_t s) {
  const dim3 grid((unsigned)((rows + kRmsBwdRows - 1) / kRmsBwdRows));
#define GQA_RMS_BWD(MV) \
  hipLaunchKernelGGL((rms_bwd_vec_kernel<T, MV>), grid, dim3(256), 0, s, dy, x, w, resid, rows, d, eps, dx, dx_op, wpart)
  if (d <= 1024 * 2) GQA_RMS_BWD(2);
  else if (d <= 1024 * 4) GQA_RMS_BWD(4);
  else if (d <= 1024 * 8) GQA_RMS_BWD(8);
  else GQA_RMS_BWD(16);
#undef GQA_RMS_BWD
  return hipGetLastError();
}

hipError_t launch_rms_bwd(const float* dy, const float* x, const float* w, const float* resid, int rows, int d,
                          float eps, float* dx, void* dx_op, int elem, float* wpart, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (rms_bwd_vec_ok(d))
    return elem == kBF16 ? rms_bwd_vec<bf16>(dy, x, w, resid, rows, d, eps, dx, static_cast<bf16*>(dx_op), wpart, s)
                         : rms_bwd_vec<float>(dy, x, w, resid, rows, d, eps, dx, static_cast<float*>(dx_op), wpart, s);
  if (elem == kBF16)
    hipLaunchKernelGGL(rms_bwd_kernel<bf16>, dim3(rows), dim3(256), 0, s, dy, x, w, resid, d, eps, dx,
                       static_cast<bf16*>(dx_op), wpart);
  else
    hipLaunchKernelGGL(rms_bwd_kernel<float>, dim3(rows), dim3(256), 0, s, dy, x, w, resid, d, eps, dx,
                       static_cast<float*>(dx_op), wpart);
  return hipGetLastError();
}

int rms_bwd_parts(int rows, int d) { return rms_bwd_vec_ok(d) ? (rows + kRmsBwdRows - 1) / kRmsBwdRows : rows; }

constexpr int kColsumRows = 32;  // rows per chunk: enough chunks to fill the GPU at 4k tokens
int colsum_chunks(int R) { return (R + kColsumRows - 1) / kColsumRows; }

hipError_t launch_colsum(const float* a, int R, int C, float* part, float* out, hipStream_t s) {
  if (C <= 0) return hipSuccess;
  const int nz = R > 0 ? colsum_chunks(R) : 0;
  if (nz > 0)
    hipLaunchKernelGGL(colsum_part_kernel, dim3((C + 255) / 256, nz), dim3(256), 0, s, a, R, C, kColsumRows, part);
  hipLaunchKernelGGL(colsum_final_kernel, dim3((C + 255) / 256), dim3(256), 0, s, part, nz, C, out);
  return hipGetLastError();
}

hipError_t launch_rope_bwd_pack(const BwdAttnArgs& a, void* dqkv, int64_t ld, int elem, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.L * ld;
  if (n == 0) return hipSuccess;
  if (ld < (int64_t)(a.H + 2 * a.KV) * a.hd) return hipErrorInvalidValue;
  const int width = (a.H + 2 * a.KV) * a.hd;
  if (a.hd % 8 == 0 && (ld - width) % 8 == 0 && ld % 4 == 0) {
    const int64_t n4 = (int64_t)a.B * a.L * ((a.H + 2 * a.KV) * (a.hd / 8) + (ld - width) / 8);
    dim3 g4((unsigned)((n4 + 255) / 256));
    if (elem == kBF16)
      hipLaunchKernelGGL(rope_bwd_pack4_kernel<bf16>, g4, dim3(256), 0, s, a, static_cast<bf16*>(dqkv), ld);
    else
      hipLaunchKernelGGL(rope_bwd_pack4_kernel<float>, g4, dim3(256), 0, s, a, static_cast<float*>(dqkv), ld);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (elem == kBF16)
    hipLaunchKernelGGL(rope_bwd_pack_kernel<bf16>, grid, dim3(256), 0, s, a, static_cast<bf16*>(dqkv), ld);
  else
    hipLaunchKernelGGL(rope_bwd_pack_kernel<float>, grid, dim3(256), 0, s, a, static_cast<float*>(dqkv), ld);
  return hipGetLastError();
}

hipError_t launch_convert(const float* in, void* out, int elem, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (elem == kBF16 && n % 8 == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0) {
    const int64_t n8 = n / 8;
    hipLaunchKernelGGL(convert8_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, in,
                       static_cast<bf16*>(out), n8);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (elem == kBF16)
    hipLaunchKernelGGL(convert_kernel<bf16>, grid, dim3(256), 0, s, in, static_cast<bf16*>(out), n);
  else
    hipLaunchKernelGGL(convert_kernel<float>, grid, dim3(256), 0, s, in, static_cast<float*>(out), n);
  return hipGetLastError();
}

hipError_t launch_attention_bwd(const BwdAttnArgs& a, int elem, hipStream_t s) {
  if (a.hd > 16 * kMaxDpl || a.hd % 2) return hipErrorInvalidValue;
  const int64_t nq = (int64_t)a.B * a.L * a.H, nk = (int64_t)a.B * a.L * a.KV;
  if (nq == 0) return hipSuccess;
  dim3 gq((unsigned)((nq + 3) / 4)), gk((unsigned)((nk + 3) / 4));
  if (elem == kBF16) {
    hipLaunchKernelGGL(attn_bwd_q_kernel<bf16>, gq, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_kv_kernel<bf16>, gk, dim3(256), 0, s, a);
  } else {
    hipLaunchKernelGGL(attn_bwd_q_kernel<float>, gq, dim3(256), 0, s, a);
    hipLaunchKernelGGL(attn_bwd_kv_kernel<float>, gk, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace gqa
