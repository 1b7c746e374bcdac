// Per-head q/k normalisation, RoPE and in-place KV-cache append.
//
// One wavefront per (token, head slot); head slots are the H query heads,
// then the KV key heads, then the KV value heads of the q|k|v projection row.
// For q and k: optional RMSNorm over head_dim (mojolearn ``qk_norm``: Qwen3
// style, before RoPE), then RoPE (DantinoX "Core Layers" page, Positional
// Encoding / RoPE: each pair rotated by p * theta_i) on Hugging Face's
// rotate-half pairs (i, i + r/2) of the first r = rope_dim dimensions,
// reading cos/sin from a float32 table [max_positions, r/2] indexed by the
// absolute position p = lengths[b] + t; the table already holds the block's
// frequencies (base, partial-rotary denominator, linear or Llama 3 scaling).
// Dimensions r .. hd-1 pass through (partial rotary, mojolearn ``rope_dim``),
// normalised like the rest under qk_norm.  Lane i holds pairs i, i + 64, ...
// so a pair never crosses lanes.
//
// bf16 blocks with head_dim 64 / 128 / 256 and rope_dim a multiple of 8 use
// the vector form (a thread per 8 elements); other shapes the wave-per-head
// form.
//
// With skip_q (vector form, no fused reduction) the grid covers the key and
// value slots only: the prefill attention kernel normalises and rotates q as
// it loads it.
//
// Outputs: q rotated in place; this call's keys (rotated) and values into
// knew/vnew [B, KV, L, hd]; and, with a cache, the same keys/values into
// slot p (full cache) or p mod W (sliding-window ring, mojolearn
// TransformerState).  Under a window only the last W positions of the call
// are stored, so the ring ends holding positions [start + L - W, start + L).
// A windowed call with L > 1 defers the ring write (defer_append) to
// kv_append, run after attention: its new positions reuse ring slots whose old
// keys the call's earlier queries still read.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(RopeArgs a) {
  const int lane = threadIdx.x & 63;
  const int slots = a.H + 2 * a.KV;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t T_ = (int64_t)a.B * a.L;
  if (gw >= T_ * slots) return;
  const int64_t tok = gw / slots;
  const int slot = (int)(gw % slots);
  const int b = (int)(tok / a.L), t = (int)(tok % a.L);
  if (a.row_len && t >= a.row_len[b]) return;  // padding of a packed ragged row
  const int64_t prow = a.row_start ? a.row_start[b] + t : tok;
  const int start = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), a.pos_flag);
  const int pos = start + t;
  const int hd = a.hd, half = hd / 2;
  const int QW = a.H * hd, KW = a.KV * hd;
  T* row = static_cast<T*>(a.qkv) + prow * a.ld;

  int kind, head;  // 0 = q, 1 = k, 2 = v
  T* src;
  if (slot < a.H) { kind = 0; head = slot; src = row + head * hd; }
  else if (slot < a.H + a.KV) { kind = 1; head = slot - a.H; src = row + QW + head * hd; }
  else { kind = 2; head = slot - a.H - a.KV; src = row + QW + KW + head * hd; }

  const int64_t new_off = (((int64_t)b * a.KV + head) * a.L + t) * hd;
  const bool to_cache = a.kcache && !a.defer_append && (a.window == 0 || t >= a.L - a.window);
  const int cslot = a.window > 0 ? pos % a.window : pos;
  const int64_t cache_off = (((int64_t)b * a.KV + head) * a.cap + cslot) * hd;

  if (kind == 2) {
    T* vn = static_cast<T*>(a.vnew) + new_off;
    T* vc = static_cast<T*>(a.vcache) + cache_off;
    for (int e = lane; e < hd; e += WAVE) {
      const T v = src[e];
      vn[e] = v;
      if (to_cache) vc[e] = v;
    }
    return;
  }

  // q or k: rotated pairs (p, p + rh) for p = lane, lane + 64, ... < rh, and
  // the pass-through dimensions e = rd + lane, rd + lane + 64, ... < hd
  constexpr int MAXP = 2, MAXR = 4;  // hd <= 256
  const int rd = a.rd, rh = rd / 2;
  float lo[MAXP], hi[MAXP], pt[MAXR];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int p = lane + i * WAVE;
    lo[i] = hi[i] = 0.f;
    if (p < rh) {
      lo[i] = to_f32(src[p]);
      hi[i] = to_f32(src[p + rh]);
      ss += lo[i] * lo[i] + hi[i] * hi[i];
    }
  }
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int e = rd + lane + i * WAVE;
    pt[i] = 0.f;
    if (e < hd) {
      pt[i] = to_f32(src[e]);
      ss += pt[i] * pt[i];
    }
  }
  const float* nw = kind == 0 ? a.q_norm : a.k_norm;
  float r = 1.f;
  if (nw) r = 1.0f / sqrtf(wave_sum(ss) / (float)hd + a.eps);
  auto gain = [&](int e) { return a.offset ? 1.0f + nw[e] : nw[e]; };
  const float* ct = a.cos_tab + (int64_t)pos * rh;
  const float* st = a.sin_tab + (int64_t)pos * rh;
  T* dst = kind == 0 ? src : static_cast<T*>(a.knew) + new_off;
  T* kc = (kind == 1 && to_cache) ? static_cast<T*>(a.kcache) + cache_off : nullptr;
#pragma unroll
  for (int i = 0; i < MAXP; ++i) {
    const int p = lane + i * WAVE;
    if (p >= rh) continue;
    float x1 = lo[i], x2 = hi[i];
    if (nw) {
      x1 = x1 * r * gain(p);
      x2 = x2 * r * gain(p + rh);
    }
    const float c = ct[p], sv = st[p];
    const T y1 = from_f32<T>(x1 * c - x2 * sv);
    const T y2 = from_f32<T>(x2 * c + x1 * sv);
    dst[p] = y1;
    dst[p + rh] = y2;
    if (kc) {
      kc[p] = y1;
      kc[p + rh] = y2;
    }
  }
#pragma unroll
  for (int i = 0; i < MAXR; ++i) {
    const int e = rd + lane + i * WAVE;
    if (e >= hd) continue;
    const T y = from_f32<T>(nw ? pt[i] * r * gain(e) : pt[i]);
    dst[e] = y;
    if (kc) kc[e] = y;
  }
}

// Vector form for bf16 activations and head_dim 64 / 128 / 256, rope_dim r a
// multiple of 8: a head slot is handled by hd/8 adjacent lanes, each owning 8
// elements as two 8-byte vectors.  Lane g < r/8 owns the rotated pairs
// (4g .. 4g+3, 4g+r/2 .. 4g+r/2+3); lane g >= r/8 owns the pass-through
// elements 8g .. 8g+7.  The qk-norm sum of squares is reduced across the
// head's lanes with shuffles.
// Grid: x = token (row-major over B, L), y = blocks of 256 (slot, lane)
// pairs of the token, so a thread finds its token and slot without 64-bit
// divisions (one uniform 32-bit division by L, a shift by the power-of-two GH).
template <int HD>
__global__ __launch_bounds__(256) void rope_append_vec_kernel(RopeArgs a) {
  constexpr int HALF = HD / 2, GH = HALF / 4;  // lanes per head slot
  static_assert((GH & (GH - 1)) == 0, "lanes per head slot: a power of two");
  const int q0 = a.skip_q ? a.H : 0;  // first head slot of the grid
  const int slots = a.H + 2 * a.KV - q0;
  const int64_t T_ = (int64_t)a.B * a.L;
  const int tok = blockIdx.x;
  const int hsl = blockIdx.y * 256 + threadIdx.x;  // (slot, lane) within the token
  bool live = hsl < slots * GH;
  const int slot = (live ? hsl / GH : 0) + q0;
  const int g = hsl % GH;
  const int b = tok / a.L, t = tok - b * a.L;
  // padding of a packed ragged row: not live (a whole head slot's lanes alike)
  if (a.row_len && t >= a.row_len[b]) live = false;
  const int64_t prow = a.row_start && live ? a.row_start[b] + t : (a.row_start ? 0 : tok);
  const int pos = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), a.pos_flag) + t;
  const int QW = a.H * HD, KW = a.KV * HD;
  bf16* row = static_cast<bf16*>(a.qkv) + prow * a.ld;
  int kind, head;  // 0 = q, 1 = k, 2 = v
  bf16* src;
  if (slot < a.H) { kind = 0; head = slot; src = row + head * HD; }
  else if (slot < a.H + a.KV) { kind = 1; head = slot - a.H; src = row + QW + head * HD; }
  else { kind = 2; head = slot - a.H - a.KV; src = row + QW + KW + head * HD; }
  const int rh = a.rd >> 1;
  const bool rot = 4 * g < rh;
  const int o1 = rot ? 4 * g : 8 * g;        // first 4 elements
  const int o2 = rot ? 4 * g + rh : o1 + 4;  // second 4 (the rotation partners)

  bf16x4 lo = bf16x4{}, hi = bf16x4{};
  if (live && a.part) {
    // fused K-split reduction: this row's columns c .. c+3 and c-o1+o2 ..
    // summed over the splits in order, plus the segment's bias, rounded as the
    // GEMM epilogue would have stored them
    const int64_t c = (src - row) + o1;
    const int64_t pstride = (a.prows ? a.prows : T_) * a.ld;
    const float* pr = a.part + prow * a.ld + c;
    f32x4 sl = f32x4{0.f, 0.f, 0.f, 0.f}, sh = sl;
    for (int z0 = 0; z0 < a.splits; z0 += 4) {  // 4 splits' loads in flight together
      f32x4 tl[4], th[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* q = pr + min(z0 + u, a.splits - 1) * pstride;
        tl[u] = *reinterpret_cast<const f32x4*>(q);
        th[u] = *reinterpret_cast<const f32x4*>(q + (o2 - o1));
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (z0 + u < a.splits) {
          sl += tl[u];
          sh += th[u];
        }
    }
    const float* bias = a.bias[kind];
    if (bias) {
      const float* bb = bias + head * HD;
      sl += *reinterpret_cast<const f32x4*>(bb + o1);
      sh += *reinterpret_cast<const f32x4*>(bb + o2);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = from_f32<bf16>(sl[e]);
      hi[e] = from_f32<bf16>(sh[e]);
    }
  } else if (live) {
    lo = *reinterpret_cast<const bf16x4*>(src + o1);
    hi = *reinterpret_cast<const bf16x4*>(src + o2);
  }
  const int64_t new_off = (((int64_t)b * a.KV + head) * a.L + t) * HD;
  const bool to_cache = a.kcache && !a.defer_append && (a.window == 0 || t >= a.L - a.window);
  const int cslot = a.window > 0 ? pos % a.window : pos;
  const int64_t cache_off = (((int64_t)b * a.KV + head) * a.cap + cslot) * HD;

  if (kind != 2) {
    float x1[4], x2[4];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x1[e] = to_f32(lo[e]);
      x2[e] = to_f32(hi[e]);
      ss += x1[e] * x1[e] + x2[e] * x2[e];
    }
    const float* nw = kind == 0 ? a.q_norm : a.k_norm;
    if (nw) {  // a head's GH lanes are adjacent and aligned: reduce within them
#pragma unroll
      for (int o = 1; o < GH; o <<= 1) ss += __shfl_xor(ss, o, WAVE);
      const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g1 = a.offset ? 1.0f + nw[o1 + e] : nw[o1 + e];
        const float g2 = a.offset ? 1.0f + nw[o2 + e] : nw[o2 + e];
        x1[e] *= r * g1;
        x2[e] *= r * g2;
      }
    }
    if (rot) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(a.cos_tab + (int64_t)pos * rh + o1);
      const f32x4 s = *reinterpret_cast<const f32x4*>(a.sin_tab + (int64_t)pos * rh + o1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = from_f32<bf16>(x1[e] * c[e] - x2[e] * s[e]);
        hi[e] = from_f32<bf16>(x2[e] * c[e] + x1[e] * s[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = from_f32<bf16>(x1[e]);
        hi[e] = from_f32<bf16>(x2[e]);
      }
    }
  }
  if (!live) return;
  if (kind == 0) {  // q, rotated (in place, or from the fused reduction)
    *reinterpret_cast<bf16x4*>(src + o1) = lo;
    *reinterpret_cast<bf16x4*>(src + o2) = hi;
    return;
  }
  bf16* dn = static_cast<bf16*>(kind == 1 ? a.knew : a.vnew) + new_off;
  *reinterpret_cast<bf16x4*>(dn + o1) = lo;
  *reinterpret_cast<bf16x4*>(dn + o2) = hi;
  if (to_cache) {
    bf16* dc = static_cast<bf16*>(kind == 1 ? a.kcache : a.vcache) + cache_off;
    *reinterpret_cast<bf16x4*>(dc + o1) = lo;
    *reinterpret_cast<bf16x4*>(dc + o2) = hi;
  }
}

// Ring write of the call's keys/values (the deferred form of the append):
// one thread per element of the last min(L, W) positions of each (row, head).
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(RopeArgs a) {
  const int keep = a.window > 0 ? min(a.L, a.window) : a.L;
  const int64_t per = (int64_t)keep * a.hd;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)a.B * a.KV * per) return;
  const int64_t bh = i / per;
  const int b = (int)(bh / a.KV), head = (int)(bh % a.KV);
  const int t = a.L - keep + (int)((i % per) / a.hd), e = (int)(i % a.hd);
  const int pos = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), nullptr) + t;
  const int slot = a.window > 0 ? pos % a.window : pos;
  const int64_t src = (((int64_t)b * a.KV + head) * a.L + t) * a.hd + e;
  const int64_t dst = (((int64_t)b * a.KV + head) * a.cap + slot) * a.hd + e;
  static_cast<T*>(a.kcache)[dst] = static_cast<const T*>(a.knew)[src];
  static_cast<T*>(a.vcache)[dst] = static_cast<const T*>(a.vnew)[src];
}

// The same copy in 16-byte chunks: grid y = (row, kv head), x = blocks of
// chunks of its last `keep` positions (cpr chunks per position).
template <typename T>
__global__ __launch_bounds__(256) void kv_append_vec_kernel(RopeArgs a, int keep, int cpr) {
  const int q = blockIdx.x * 256 + threadIdx.x;
  if (q >= keep * cpr) return;
  const int bh = blockIdx.y;
  const int b = bh / a.KV;
  const int tr = q / cpr, ch = q - tr * cpr;
  const int t = a.L - keep + tr;
  const int pos = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), nullptr) + t;
  const int slot = a.window > 0 ? pos % a.window : pos;
  constexpr int E = 16 / sizeof(T);  // elements per chunk
  const int64_t src = ((int64_t)bh * a.L + t) * a.hd + ch * E;
  const int64_t dst = ((int64_t)bh * a.cap + slot) * a.hd + ch * E;
  *reinterpret_cast<uint4*>(static_cast<T*>(a.kcache) + dst) = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.knew) + src);
  *reinterpret_cast<uint4*>(static_cast<T*>(a.vcache) + dst) = *reinterpret_cast<const uint4*>(static_cast<const T*>(a.vnew) + src);
}

}  // namespace

hipError_t launch_kv_append(const RopeArgs& a, int elem, hipStream_t s) {
  const int keep = a.window > 0 ? (a.L < a.window ? a.L : a.window) : a.L;
  const int64_t n = (int64_t)a.B * a.KV * keep * a.hd;
  if (n == 0 || !a.kcache) return hipSuccess;
  const int es = elem == kBF16 ? 2 : 4;
  const int64_t bh = (int64_t)a.B * a.KV;
  if ((a.hd * es) % 16 == 0 && bh <= 65535 && (int64_t)keep * (a.hd * es / 16) < 0x7fffff00) {
    const int cpr = a.hd * es / 16;
    dim3 vgrid((unsigned)(((int64_t)keep * cpr + 255) / 256), (unsigned)bh);
    if (elem == kBF16)
      hipLaunchKernelGGL(kv_append_vec_kernel<bf16>, vgrid, dim3(256), 0, s, a, keep, cpr);
    else
      hipLaunchKernelGGL(kv_append_vec_kernel<float>, vgrid, dim3(256), 0, s, a, keep, cpr);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((n + 255) / 256));
  if (elem == kBF16)
    hipLaunchKernelGGL(kv_append_kernel<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_vec(const RopeArgs& a, hipStream_t s) {
  const int64_t tokens = (int64_t)a.B * a.L;
  const int per_token = (a.H + 2 * a.KV - (a.skip_q ? a.H : 0)) * (HD / 8);
  if (tokens > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(rope_append_vec_kernel<HD>, dim3((unsigned)tokens, (unsigned)((per_token + 255) / 256)), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

// The vector form (the only one that takes `part`) covers these shapes.
bool rope_append_fuses_reduce(int hd, int rd, int64_t ld, int elem) {
  return elem == kBF16 && ld % 4 == 0 && (hd == 64 || hd == 128 || hd == 256) && rd % 8 == 0 && rd >= 8 &&
         rd <= hd;
}

hipError_t launch_rope_append(const RopeArgs& a, int elem, hipStream_t s) {
  const int64_t waves = (int64_t)a.B * a.L * (a.H + 2 * a.KV);
  if (waves == 0) return hipSuccess;
  if (a.rd < 2 || a.rd > a.hd || a.rd % 2) return hipErrorInvalidValue;
  const bool vec = rope_append_fuses_reduce(a.hd, a.rd, a.ld, elem);
  if (a.part && (!vec || a.splits < 1)) return hipErrorInvalidValue;
  if (a.skip_q && (!vec || a.part)) return hipErrorInvalidValue;
  if (vec) {
    if (a.hd == 64) return launch_vec<64>(a, s);
    if (a.hd == 128) return launch_vec<128>(a, s);
    if (a.hd == 256) return launch_vec<256>(a, s);
  }
  dim3 grid((unsigned)((waves + 3) / 4));
  if (elem == kBF16)
    hipLaunchKernelGGL(rope_append_kernel<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(rope_append_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
