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
// Work item = (segment s, kv head j).  The keys all rows attend are laid end
// to end (row b's [klo_b, p_b] after row b-1's) and cut into nseg equal
// contiguous segments, so every workgroup streams the same number of keys
// whatever the mix of row lengths; a segment that spans a row boundary is
// processed as one piece per row, each writing its own partial.  A workgroup
// of 4 waves streams a piece in sub-tiles of 128 keys, 32 per wave; each wave
// issues all of its K and V loads for a sub-tile at once (16 KB in flight per
// wave at hd 128), every load instruction covering whole 256-byte row pieces
// (measured on gfx950, whole-piece loads stream faster than loads shaped as
// MFMA operands, which cover 64 bytes of each of 16 rows); full sub-tiles
// take a short address path:
//  * scores on the matrix cores: S^T[16 keys][16 heads] = K Q^T with
//    v_mfma_f32_16x16x32_bf16, K passed through a per-wave LDS slab into the
//    operand layout (lane -> key lane%16, 16-byte dim pieces), Q^T resident
//    in registers (heads past G are zero columns) — no conversions, no
//    cross-lane sums;
//  * per-wave online softmax in float32 (base 2; the reference max is raised
//    lazily, beyond 2^8), the weights handed through a 16 x G slab of LDS;
//  * values on the vector ALUs: each lane owns 8 dims of one value row and
//    accumulates G outputs with float32 FMAs.
// The four waves are merged once per piece.  A piece of row b in segment s
// writes (output[hd], max, sum) per query head to record s + b (row b's
// segments are consecutive, so rows never share a record); the combine kernel
// merges a row's records in segment order (deterministic).  Cache loads are
// non-temporal: the stream is read once per step.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int NT = 256;
constexpr int NWV = NT / WAVE;
constexpr int kMaxRows = 2048;          // rows whose key-count prefix fits the workgroup's LDS
constexpr int kMaxSeg = 1024;           // segments per kv head (records per row the combine merges)
constexpr float kSlack = 8.0f;          // lazy rescale threshold (log2 units)

// 16 bytes of the cache, read once per step: a non-temporal load, so the
// stream does not evict reused lines from L2 / Infinity Cache.
__device__ __forceinline__ u32x4 stream_load(const bf16* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

template <int HD, int G>
__global__ __launch_bounds__(NT) void attn_decode_kernel(AttnArgs a) {
  constexpr int KPW = 32;               // keys per wave per sub-tile (16 KB of K and V at hd 128)
  constexpr int NKB = KPW / 16;         // 16-key MFMA blocks per wave per sub-tile
  constexpr int SUBK = KPW * NWV;       // keys per sub-tile
  constexpr int NK = HD / 32;           // 16-byte K pieces per lane per 16-key block (= MFMA k-steps)
  constexpr int LPR = HD / 8;           // lanes per V row
  constexpr int RPV = WAVE / LPR;       // V rows per wave load
  constexpr int NV = KPW / RPV;         // V loads per lane per sub-tile
  __shared__ float sp[NWV][KPW][G];     // this sub-tile's weights, per wave
  __shared__ float wm[NWV][G], wl[NWV][G];
  __shared__ float wo[NWV][G][HD];
  __shared__ u32x4 kslab[NWV][KPW * HD / 8];  // each wave's K sub-tile, swizzled 16-byte pieces

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // ---- prefix of the key counts n_b = p_b + 1 - klo_b: pre[b] = sum over rows < b ----
  __shared__ int pre[kMaxRows + 1];
  const int W = a.window;
  if (w == 0) {
    int carry = 0;
    if (lane == 0) pre[0] = 0;
    for (int base = 0; base < a.B; base += WAVE) {
      const int bb = base + lane;
      int v = 0;
      if (bb < a.B) {
        const int pb = guarded_start(a.lengths, bb, 1, position_limit(W, a.cap, a.max_pos), nullptr);
        v = pb + 1 - (W > 0 ? max(0, pb - W + 1) : 0);
      }
#pragma unroll
      for (int o = 1; o < WAVE; o <<= 1) {
        const int t = __shfl_up(v, o, WAVE);
        if (lane >= o) v += t;
      }
      if (bb < a.B) pre[bb + 1] = carry + v;
      carry += __shfl(v, WAVE - 1, WAVE);
    }
  }
  __syncthreads();
  const int j = (int)(blockIdx.x % a.KV), sgm = (int)(blockIdx.x / a.KV);
  const int64_t total = pre[a.B];
  // never more segments than keys (so none is empty): the combine uses the same count
  const int nseg = (int)min((int64_t)a.nseg, total);
  if (blockIdx.x == 0) {
    // row table for the combine: row b's records are fs .. fs + n - 1 (+ b), where
    // fs / ls are the segments of its first / last key (segment of key g: the
    // last s with s * total / nseg <= g)
    int* tab = reinterpret_cast<int*>(a.part + (int64_t)a.H * a.rec_stride * (HD + 2));
    for (int bb = tid; bb < a.B; bb += NT) {
      const int fs = (int)((((int64_t)pre[bb] + 1) * nseg - 1) / total);
      const int ls = (int)((((int64_t)pre[bb + 1]) * nseg - 1) / total);
      tab[2 * bb] = fs;
      tab[2 * bb + 1] = ls - fs + 1;
    }
  }
  if (sgm >= nseg) return;
  const int64_t seg_lo = (int64_t)sgm * total / nseg, seg_hi = (int64_t)(sgm + 1) * total / nseg;
  int b = 0;  // the row holding key seg_lo: the last b with pre[b] <= seg_lo
  {
    int lo = 0, hi = a.B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (pre[mid] <= seg_lo) lo = mid;
      else hi = mid - 1;
    }
    b = lo;
  }
  for (bool first_piece = true; b < a.B && pre[b] < seg_hi; ++b, first_piece = false) {
  if (!first_piece) __syncthreads();  // the previous piece's LDS slabs have been read
  const int start = guarded_start(a.lengths, b, 1, position_limit(W, a.cap, a.max_pos), nullptr);
  const int p = start;                  // the new token's position (L = 1)
  const int klo = W > 0 ? max(0, p - W + 1) : 0;
  const int ks0 = klo + (int)(max(seg_lo, (int64_t)pre[b]) - pre[b]);
  const int kend = klo + (int)(min(seg_hi, (int64_t)pre[b + 1]) - pre[b]);
  const int nsub = (kend - ks0 + SUBK - 1) / SUBK;

  const int64_t bjo = (int64_t)b * a.KV + j;
  const bf16* kfresh = static_cast<const bf16*>(a.knew) + bjo * a.L * HD;
  const bf16* vfresh = static_cast<const bf16*>(a.vnew) + bjo * a.L * HD;
  const bf16* kbase = a.kcache ? static_cast<const bf16*>(a.kcache) + bjo * a.cap * HD : kfresh;
  const bf16* vbase = a.vcache ? static_cast<const bf16*>(a.vcache) + bjo * a.cap * HD : vfresh;
  // row of key position kp (clamped into the split): cache slot kp (or kp mod W), or the fresh row
  auto row = [&](const bf16* fresh, const bf16* base, int kp) {
    kp = min(kp, kend - 1);
    return kp >= start ? fresh + (int64_t)(kp - start) * HD
                       : base + (int64_t)(W > 0 ? kp % W : kp) * HD;
  };

  // K in the MFMA A layout: lane -> key (lane % 16) of each 16-key block, dims 32s + 8(lane / 16)
  // V in rows: lane -> key t*RPV + lane / LPR, dims 8(lane % LPR)
  const int kkey = lane % 16, kdim = 8 * (lane / 16);
  const int vkey = lane / LPR, vdim = 8 * (lane % LPR);

  // Q^T in the MFMA B layout: lane -> head (lane % 16) (zero past G), same dims as K
  const int qh = lane % 16;
  bf16x8 qf[NK];
#pragma unroll
  for (int s2 = 0; s2 < NK; ++s2) {
    if (qh < G) {
      const bf16* qr = static_cast<const bf16*>(a.q) + (int64_t)b * a.ldq + (int64_t)(j * G + qh) * HD + kdim;
      qf[s2] = *reinterpret_cast<const bf16x8*>(qr + 32 * s2);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[s2][e] = from_f32<bf16>(0.f);
    }
  }
  const float cap = a.softcap;
  const float scale = 1.0f / sqrtf((float)HD);

  // per-wave online softmax: m (equal on all lanes of a head), l partial, o[g][8 dims]
  float m_run = -INFINITY, l_run = 0.f;
  float o[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;

  // ---- loads of sub-tile n: all of this wave's K and V at once, each load
  // instruction covering whole 256-byte row pieces (K: keys k0 + 4i + l / 16,
  // 16-byte piece l % 16; V: rows t * RPV + l / LPR, piece l % LPR) ----
  constexpr int KI = KPW * HD * 2 / 1024;           // K load instructions per wave per sub-tile
  constexpr int KRI = 1024 / (HD * 2);              // keys per K load instruction
  constexpr int KPC = HD / 8;                       // 16-byte pieces per key row
  constexpr int KX = KPC < 16 ? KPC : 16;           // XOR range of the slab swizzle
  auto load = [&](int n, u32x4 (&kr)[KI], u32x4 (&vr)[NV]) {
    const int k0 = ks0 + n * SUBK + w * KPW;
    if (W == 0 && k0 + KPW <= min(start, kend)) {   // every row a cache slot = position
#pragma unroll
      for (int i = 0; i < KI; ++i)
        kr[i] = stream_load(kbase + (int64_t)(k0 + KRI * i + lane / KPC) * HD + 8 * (lane % KPC));
#pragma unroll
      for (int t = 0; t < NV; ++t)
        vr[t] = stream_load(vbase + (int64_t)(k0 + t * RPV + vkey) * HD + vdim);
    } else {
#pragma unroll
      for (int i = 0; i < KI; ++i)
        kr[i] = stream_load(row(kfresh, kbase, k0 + KRI * i + lane / KPC) + 8 * (lane % KPC));
#pragma unroll
      for (int t = 0; t < NV; ++t)
        vr[t] = stream_load(row(vfresh, vbase, k0 + t * RPV + vkey) + vdim);
    }
  };

  auto compute = [&](int n, const u32x4 (&kr)[KI], const u32x4 (&vr)[NV]) {
    const int k0 = ks0 + n * SUBK + w * KPW;
    // K through the wave's slab into the MFMA A layout: key row r, piece c at
    // slot r * KPC + (c ^ (r % KX)); lane l reads key 16 h2 + l % 16, pieces
    // 4 s2 + l / 16 (dims 32 s2 + 8 (l / 16), matching Q^T)
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int r = KRI * i + lane / KPC, c = lane % KPC;
      kslab[w][r * KPC + (c ^ (r % KX))] = kr[i];
    }
    // ---- scores: S^T[16 keys][16 heads] per block; lane holds keys 4(lane/16)+e ----
    f32x4 sc[NKB];
#pragma unroll
    for (int h2 = 0; h2 < NKB; ++h2) {
      sc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * h2 + kkey;
#pragma unroll
      for (int s2 = 0; s2 < NK; ++s2) {
        const u32x4 kf = kslab[w][r * KPC + ((4 * s2 + lane / 16) ^ (kkey % KX))];
        sc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf), qf[s2], sc[h2], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int h2 = 0; h2 < NKB; ++h2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float v = cap > 0.f ? cap * kLog2e * tanh_exp(sc[h2][e] * scale / cap) : sc[h2][e] * (scale * kLog2e);
        v = (k0 + 16 * h2 + 4 * (lane / 16) + e < kend) ? v : -INFINITY;
        sc[h2][e] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, xor32(mx));
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float ag = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), g));  // head g's factor
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= ag;
      }
    }
    const float mr = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int h2 = 0; h2 < NKB; ++h2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pw = exp2_fast(sc[h2][e] - mr);
        l_run += pw;
        if (qh < G) sp[w][16 * h2 + 4 * (lane / 16) + e][qh] = pw;
      }
    // the weights go to this wave's LDS slab and come back as per-key broadcasts
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the LDS writes have completed
    __builtin_amdgcn_wave_barrier();

    // ---- values: o[g][dims] += w[key][g] * v[key][dims] ----
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      const int kk = t * RPV + vkey;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_lo(vr[t][e]);
        vf[2 * e + 1] = bf16_hi(vr[t][e]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float pw = sp[w][kk][g];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pw, vf[e], o[g][e]);
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  for (int n = 0; n < nsub; ++n) {
    u32x4 kr[KI], vr[NV];
    load(n, kr, vr);
    compute(n, kr, vr);
  }

  // wave totals: l over the 4 lanes of a head, o over the V row groups
  l_run += __shfl_xor(l_run, 16, WAVE);
  l_run += xor32(l_run);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[g][e];
#pragma unroll
      for (int off = LPR; off < WAVE; off <<= 1) v += __shfl_xor(v, off, WAVE);
      o[g][e] = v;
    }
  if (lane < G) {
    wm[w][lane] = m_run;
    wl[w][lane] = l_run;
  }
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) wo[w][g][vdim + e] = o[g][e];
  }
  __syncthreads();
  // partial record of this piece: (out[HD], max (base 2), sum) per query head
  for (int i = tid; i < G * HD; i += NT) {
    const int g = i / HD, d = i % HD;
    float M = wm[0][g];
#pragma unroll
    for (int ww = 1; ww < NWV; ++ww) M = fmaxf(M, wm[ww][g]);
    float s2 = 0.f, ls = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) {
      const float f = wm[ww][g] == -INFINITY ? 0.f : exp2_fast(wm[ww][g] - M);
      s2 += wo[ww][g][d] * f;
      ls += wl[ww][g] * f;
    }
    float* rec = a.part + ((int64_t)(j * G + g) * a.rec_stride + sgm + b) * (HD + 2);
    rec[d] = s2;
    if (d == 0) {
      rec[HD] = M;
      rec[HD + 1] = ls;
    }
  }
  }  // piece
}

// One workgroup per (row, query head): merge the row's records in segment order.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  constexpr int DG = 256 / HD;          // record groups summed in parallel (2 for hd=128)
  __shared__ float fw[kMaxSeg];
  __shared__ float red[8];
  __shared__ float osum[DG][HD];
  const int tid = threadIdx.x;
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int* tab = reinterpret_cast<const int*>(a.part + (int64_t)a.H * a.rec_stride * (HD + 2));
  const int fs = tab[2 * b], nrec = tab[2 * b + 1];
  const float* rec = a.part + ((int64_t)h * a.rec_stride + fs + b) * (HD + 2);
  float m = -INFINITY;
  for (int c = tid; c < nrec; c += 256) m = fmaxf(m, rec[c * (HD + 2) + HD]);
  m = wave_max(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float l = 0.f;
  for (int c = tid; c < nrec; c += 256) {
    const float f = exp2_fast(rec[c * (HD + 2) + HD] - M);
    fw[c] = f;
    l += f * rec[c * (HD + 2) + HD + 1];
  }
  l = wave_sum(l);
  if ((tid & 63) == 0) red[4 + (tid >> 6)] = l;
  __syncthreads();
  const float lsum = red[4] + red[5] + red[6] + red[7];
  const int d = tid % HD, cg = tid / HD;
  float o = 0.f;
#pragma unroll 4
  for (int c = cg; c < nrec; c += DG) o = fmaf(fw[c], rec[c * (HD + 2) + d], o);
  osum[cg][d] = o;
  __syncthreads();
  if (tid < HD) {
    float t = 0.f;
#pragma unroll
    for (int g = 0; g < DG; ++g) t += osum[g][tid];
    static_cast<bf16*>(a.ctx)[(int64_t)b * a.H * HD + (int64_t)h * HD + tid] = from_f32<bf16>(t / lsum);
  }
}

template <int HD, int G>
hipError_t launch_hg(const AttnArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((int64_t)a.nseg * a.KV));
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
  return (hd == 64 || hd == 128 || hd == 256) && (G == 1 || G == 2 || G == 4 || G == 5 || G == 8);  // G <= 16
}

int attention_decode_max_rows() { return kMaxRows; }

// Segments per kv head for `total` attended keys: about `keys_per_seg` keys
// each, at most kMaxSeg, never more than the keys.
int attention_decode_segments(int64_t total, int keys_per_seg) {
  int64_t s = (total + keys_per_seg / 2) / keys_per_seg;
  if (s > kMaxSeg) s = kMaxSeg;
  if (s > total) s = total;
  return s < 1 ? 1 : (int)s;
}
int attention_decode_max_segments() { return kMaxSeg; }

hipError_t launch_attention_decode_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.B > kMaxRows || a.nseg < 1 || a.nseg > kMaxSeg || a.rec_stride < a.nseg + a.B) return hipErrorInvalidValue;
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
  dim3 g2((unsigned)((int64_t)a.B * a.H));
  switch (a.hd) {
    case 64: hipLaunchKernelGGL(attn_combine_kernel<64>, g2, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL(attn_combine_kernel<128>, g2, dim3(256), 0, s, a); break;
    case 256: hipLaunchKernelGGL(attn_combine_kernel<256>, g2, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqa
