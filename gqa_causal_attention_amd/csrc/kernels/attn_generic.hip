// Grouped-query causal attention, generic form (any head_dim <= 256, any
// group size, float32 or bf16 storage): one wavefront per (row, token, query
// head).  Used for float32 blocks and for shapes the matrix-core kernels do
// not cover.
//
// Semantics (mojolearn TransformerBlock; DantinoX "Core Layers" page, MHA and
// GQA): query head h reads kv head h / G; the query at absolute position p
// attends keys at positions [max(0, p - W + 1), p] (W = 0: [0, p]); scores
// q.k / sqrt(hd), optionally capped to c * tanh(s / c); softmax over those
// keys in float32; weighted sum of values.  Keys of positions produced by the
// same call come from knew/vnew, older ones from the cache (slot p, or p mod W
// for the sliding-window ring).
//
// Each lane owns keys lane, lane + 64, ...: pass 1 keeps a running (max, sum)
// per lane and merges them across the wave; pass 2 recomputes each key's
// weight, broadcasts 64 weights at a time with lane shuffles and accumulates
// the output with lanes owning head dimensions.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

template <typename T>
__device__ __forceinline__ const T* key_row(const AttnArgs& a, const void* fresh, const void* cache, int b,
                                           int j, int start, int kp) {
  if (kp >= start)
    return static_cast<const T*>(fresh) + (((int64_t)b * a.KV + j) * a.L + (kp - start)) * a.hd;
  const int slot = a.window > 0 ? kp % a.window : kp;
  return static_cast<const T*>(cache) + (((int64_t)b * a.KV + j) * a.cap + slot) * a.hd;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_generic_kernel(AttnArgs a) {
  __shared__ float qs[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t gw = (int64_t)blockIdx.x * 4 + w;
  const int64_t total = (int64_t)a.B * a.L * a.H;
  const bool active = gw < total;
  const int64_t tok = active ? gw / a.H : 0;
  const int h = active ? (int)(gw % a.H) : 0;
  const int b = (int)(tok / a.L), t = (int)(tok % a.L);
  const int G = a.H / a.KV, j = h / G, hd = a.hd;
  const int start = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), nullptr);
  const int p = start + t;
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const float scale = 1.0f / sqrtf((float)hd);
  const float cap = a.softcap;

  const T* q = static_cast<const T*>(a.q) + tok * a.ldq + (int64_t)h * hd;
  for (int e = lane; e < hd; e += WAVE) qs[w][e] = to_f32(q[e]);
  __syncthreads();
  if (!active) return;  // no barriers below

  auto score = [&](int kp) {
    const T* kr = key_row<T>(a, a.knew, a.kcache, b, j, start, kp);
    float s = 0.f;
    for (int e = 0; e < hd; ++e) s = fmaf(qs[w][e], to_f32(kr[e]), s);
    s *= scale;
    if (cap > 0.f) s = cap * tanh_exp(s / cap);
    return s;
  };

  // pass 1: running max / sum per lane, merged across the wave
  float m = -INFINITY, l = 0.f;
  for (int kp = lo + lane; kp <= p; kp += WAVE) {
    const float s = score(kp);
    const float mn = fmaxf(m, s);
    l = l * exp2_fast((m - mn) * kLog2e) + exp2_fast((s - mn) * kLog2e);
    m = mn;
  }
  const float M = wave_max(m);
  const float Lsum = wave_sum(m == -INFINITY ? 0.f : l * exp2_fast((m - M) * kLog2e));
  const float inv = 1.0f / Lsum;

  // pass 2: weights broadcast by shuffles, lanes own output dimensions
  constexpr int MAXE = 4;  // hd <= 256
  float o[MAXE] = {0.f, 0.f, 0.f, 0.f};
  for (int kb = lo; kb <= p; kb += WAVE) {
    const int kp = kb + lane;
    const float pw = kp <= p ? exp2_fast((score(kp) - M) * kLog2e) * inv : 0.f;
    const int n = min(WAVE, p - kb + 1);
    for (int i = 0; i < n; ++i) {
      const float wt = __shfl(pw, i, WAVE);
      const T* vr = key_row<T>(a, a.vnew, a.vcache, b, j, start, kb + i);
#pragma unroll
      for (int c = 0; c < MAXE; ++c) {
        const int e = lane + c * WAVE;
        if (e < hd) o[c] = fmaf(wt, to_f32(vr[e]), o[c]);
      }
    }
  }
  T* out = static_cast<T*>(a.ctx) + tok * ((int64_t)a.H * hd) + (int64_t)h * hd;
#pragma unroll
  for (int c = 0; c < MAXE; ++c) {
    const int e = lane + c * WAVE;
    if (e < hd) out[e] = from_f32<T>(o[c]);
  }
}

}  // namespace

hipError_t launch_attention_generic(const AttnArgs& a, int elem, hipStream_t s) {
  const int64_t waves = (int64_t)a.B * a.L * a.H;
  if (waves == 0) return hipSuccess;
  dim3 grid((unsigned)((waves + 3) / 4));
  if (elem == kBF16)
    hipLaunchKernelGGL(attn_generic_kernel<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace gqa
