// Split-K grouped-query decode attention (one new token per row) for bf16
// KV caches, plus the combine of the per-chunk partial results.
//
// The operation is the block's attention at L = 1 (mojolearn
// TransformerBlock.step): the query of row b sits at its own position
// p_b = lengths[b] and attends keys [max(0, p_b - W + 1), p_b].  Decode is
// bound by reading the cache; grouped-query attention stores KV heads
// H / G times fewer than query heads (DantinoX "Core Layers" page, Selection
// guide: 2 * H_kv * d_h bytes per token and layer), and this kernel reads each
// cached key/value exactly once for all G query heads of its group.
//
// Work item = (row b, kv head j, chunk of CH keys).  A workgroup of 256
// threads reads its chunk's key rows with 16-byte coalesced loads (hd/8 lanes
// per row), forms the G scores of each key (lane-shuffle reduction), takes the
// chunk's max and exponentials in float32, then reads the value rows once and
// accumulates the G partial outputs.  It writes (max, sum, output[hd]) per
// (b, query head, chunk); the combine kernel merges the chunks of a row in
// chunk order (deterministic).  Work items past a row's last chunk exit at
// once (rows have different lengths).
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int NT = 256;
constexpr int CH = 512;  // keys per work item

__device__ __forceinline__ const bf16* dec_row(const AttnArgs& a, const void* fresh, const void* cache, int b, int j,
                                              int start, int kp) {
  if (kp >= start)
    return static_cast<const bf16*>(fresh) + (((int64_t)b * a.KV + j) * a.L + (kp - start)) * a.hd;
  const int slot = a.window > 0 ? kp % a.window : kp;
  return static_cast<const bf16*>(cache) + (((int64_t)b * a.KV + j) * a.cap + slot) * a.hd;
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32) with DPP row moves.
template <int N>
__device__ __forceinline__ float row_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of the 8
  if (N >= 16) x += dpp<0x140>(x);  // row_mirror: the other 8 of the 16
  if (N >= 32) x += __shfl_xor(x, 16, WAVE);
  return x;
}

template <int HD, int G>
__global__ __launch_bounds__(NT) void attn_decode_kernel(AttnArgs a) {
  constexpr int LPR = HD / 8;           // lanes per key row (8 bf16 each)
  constexpr int RPI = NT / LPR;         // rows per workgroup iteration
  constexpr int NIT = CH / RPI;         // iterations over the chunk
  constexpr int UNR = NIT >= 8 ? 8 : NIT;
  __shared__ float sc[G][CH];           // scores, then weights
  __shared__ float red[NT / WAVE][G];
  __shared__ float ored[NT / WAVE][G][HD];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunk = blockIdx.x % a.max_chunks;
  const int bj = blockIdx.x / a.max_chunks;
  const int b = bj / a.KV, j = bj % a.KV;
  const int start = a.lengths ? a.lengths[b] : 0;
  const int p = start;                  // the new token's position (L = 1)
  const int klo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int nkeys = p - klo + 1;
  const int nchunks = (nkeys + CH - 1) / CH;
  if (chunk >= nchunks) return;
  const int kc0 = klo + chunk * CH;
  const int kcnt = min(CH, p + 1 - kc0);

  const int rl = tid % LPR;             // lane within the row group: dims 8rl..8rl+7
  const int rg = tid / LPR;             // row group
  const float scale = 1.0f / sqrtf((float)HD);
  const float cap = a.softcap;

  // q values of the G heads for this lane's 8 dims
  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const bf16* qr = static_cast<const bf16*>(a.q) + (int64_t)b * a.ldq + (int64_t)(j * G + g) * HD + rl * 8;
    const u32x4 u = *reinterpret_cast<const u32x4*>(qr);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[g][2 * e] = bf16_lo(u[e]);
      qv[g][2 * e + 1] = bf16_hi(u[e]);
    }
  }

  // ---- phase 1: scores ----
  for (int it0 = 0; it0 < NIT; it0 += UNR) {
    u32x4 kr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kl = (it0 + u) * RPI + rg;
      const int kp = kc0 + min(kl, kcnt - 1);
      kr[u] = *reinterpret_cast<const u32x4*>(dec_row(a, a.knew, a.kcache, b, j, start, kp) + rl * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kl = (it0 + u) * RPI + rg;
      float kf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = bf16_lo(kr[u][e]);
        kf[2 * e + 1] = bf16_hi(kr[u][e]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(qv[g][e], kf[e], s);
        s = row_sum<LPR>(s);
        s *= scale;
        if (cap > 0.f) s = cap * tanh_exp(s / cap);
        if (rl == g % LPR) sc[g][kl] = kl < kcnt ? s : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- phase 2: chunk max, weights, sum (per head) ----
  float mloc[G], lloc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = -INFINITY;
    for (int i = tid; i < CH; i += NT) mx = fmaxf(mx, sc[g][i]);
    mx = wave_max(mx);
    if (lane == 0) red[w][g] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mx = red[0][g];
#pragma unroll
    for (int i = 1; i < NT / WAVE; ++i) mx = fmaxf(mx, red[i][g]);
    mloc[g] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float ls = 0.f;
    for (int i = tid; i < CH; i += NT) {
      const float e = exp2_fast((sc[g][i] - mloc[g]) * kLog2e);
      sc[g][i] = e;
      ls += e;
    }
    ls = wave_sum(ls);
    if (lane == 0) red[w][g] = ls;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) ls += red[i][g];
    lloc[g] = ls;
  }

  // ---- phase 3: weighted values ----
  float ov[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[g][e] = 0.f;
  for (int it0 = 0; it0 < NIT; it0 += UNR) {
    u32x4 vr[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kl = (it0 + u) * RPI + rg;
      const int kp = kc0 + min(kl, kcnt - 1);
      vr[u] = *reinterpret_cast<const u32x4*>(dec_row(a, a.vnew, a.vcache, b, j, start, kp) + rl * 8);
    }
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const int kl = (it0 + u) * RPI + rg;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vr[u][e]);
        vf[2 * e + 1] = bf16_hi(vr[u][e]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = sc[g][kl];  // 0 for keys past the chunk's end
#pragma unroll
        for (int e = 0; e < 8; ++e) ov[g][e] = fmaf(pw, vf[e], ov[g][e]);
      }
    }
  }
  // reduce over the row groups of a wave, then across waves through LDS
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = ov[g][e];
#pragma unroll
      for (int o = LPR; o < WAVE; o <<= 1) v += __shfl_xor(v, o, WAVE);
      ov[g][e] = v;
    }
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) ored[w][g][rl * 8 + e] = ov[g][e];
  }
  __syncthreads();
  // partial record: [B, H, max_chunks, HD + 2] = (out[HD], max, sum)
  for (int i = tid; i < G * HD; i += NT) {
    const int g = i / HD, d = i % HD;
    float s = 0.f;
#pragma unroll
    for (int ww = 0; ww < NT / WAVE; ++ww) s += ored[ww][g][d];
    float* rec = a.part + (((int64_t)b * a.H + j * G + g) * a.max_chunks + chunk) * (HD + 2);
    rec[d] = s;
    if (d == 0) {
      rec[HD] = mloc[g];
      rec[HD + 1] = lloc[g];
    }
  }
}

// One wavefront per (row, query head): merge the row's chunks in order.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= (int64_t)a.B * a.H) return;
  const int b = (int)(gw / a.H), h = (int)(gw % a.H);
  const int p = a.lengths ? a.lengths[b] : 0;
  const int klo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int nchunks = min((p - klo + 1 + CH - 1) / CH, a.max_chunks);
  const float* rec = a.part + ((int64_t)b * a.H + h) * a.max_chunks * (HD + 2);
  float M = -INFINITY;
  for (int c = 0; c < nchunks; ++c) M = fmaxf(M, rec[c * (HD + 2) + HD]);
  constexpr int PE = (HD + 63) / 64;
  float o[PE];
#pragma unroll
  for (int i = 0; i < PE; ++i) o[i] = 0.f;
  float lsum = 0.f;
  for (int c = 0; c < nchunks; ++c) {
    const float* r = rec + c * (HD + 2);
    const float f = exp2_fast((r[HD] - M) * kLog2e);
    lsum += f * r[HD + 1];
#pragma unroll
    for (int i = 0; i < PE; ++i) {
      const int d = lane + i * 64;
      if (d < HD) o[i] += f * r[d];
    }
  }
  const float inv = 1.0f / lsum;
  bf16* out = static_cast<bf16*>(a.ctx) + (int64_t)b * a.H * HD + (int64_t)h * HD;
#pragma unroll
  for (int i = 0; i < PE; ++i) {
    const int d = lane + i * 64;
    if (d < HD) out[d] = from_f32<bf16>(o[i] * inv);
  }
}

template <int HD, int G>
hipError_t launch_hg(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)a.B * a.KV * a.max_chunks));
  hipLaunchKernelGGL((attn_decode_kernel<HD, G>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_h(const AttnArgs& a, hipStream_t s) {
  switch (a.H / a.KV) {
    case 1: return launch_hg<HD, 1>(a, s);
    case 2: return launch_hg<HD, 2>(a, s);
    case 4: return launch_hg<HD, 4>(a, s);
    case 5: return launch_hg<HD, 5>(a, s);
    case 8: return launch_hg<HD, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool attention_decode_bf16_supported(int hd, int G) {
  return (hd == 64 || hd == 128 || hd == 256) && (G == 1 || G == 2 || G == 4 || G == 5 || G == 8);
}

int attention_decode_chunk() { return CH; }

hipError_t launch_attention_decode_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  switch (a.hd) {
    case 64: return launch_h<64>(a, s);
    case 128: return launch_h<128>(a, s);
    case 256: return launch_h<256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa

namespace gqa {

hipError_t launch_attention_decode_combine(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  dim3 g2((unsigned)(((int64_t)a.B * a.H + 3) / 4));
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(attn_combine_kernel<64>, g2, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_combine_kernel<128>, g2, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_combine_kernel<256>, g2, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqa
