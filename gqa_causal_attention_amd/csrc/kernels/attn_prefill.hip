// Flash-style grouped-query causal attention for bf16 activations on gfx950
// matrix cores (prefill and chunked continuation).
//
// What is computed is the plain attention of the block (mojolearn
// TransformerBlock; DantinoX "Core Layers" page, MHA and GQA / Flash
// Attention): for query head h (kv head j = h / G) at position p, softmax over
// keys [max(0, p - W + 1), p] of q.k / sqrt(hd) (optionally c * tanh(s / c)),
// times the values.  The DantinoX page's flash path (exact attention without
// an O(T^2) score matrix in HBM) is the idea kept; the kernel is written for
// CDNA4:
//
//  * One workgroup per (row b, kv head j, block of BQ query positions); its
//    waves cover all G query heads of the group, so every K/V tile staged in
//    LDS is read from HBM once for the whole group.  Blocks are issued
//    longest-first (the causal triangle's last query blocks first); for a
//    small causal grid a workgroup takes the pair of blocks p and nqb-1-p,
//    so all workgroups have equal work.
//  * Each wave owns 32 query positions of one head.  Transposed products
//    S^T = K Q^T and O^T += V^T P^T with v_mfma_f32_32x32x16_bf16: each lane
//    then owns one query column, so softmax statistics are per-lane scalars,
//    and the P^T operand of the second product is the lane's own S^T
//    accumulator converted to bf16 — provided V^T's keys are stored in the
//    same order, which the transposing LDS write arranges.
//  * Q^T fragments live in registers; K tiles are [key][hd] and V^T tiles
//    [hd][key] in LDS, padded rows, double-buffered (global -> registers ->
//    LDS, one barrier per tile).  A tile is two 32-key sub-tiles whose score
//    products are both issued before the first softmax, so the exponentials
//    of one overlap the matrix work of the other.
//  * Softmax in float32 (dew CausalTransformer force_fp32_for_softmax) with
//    base-2 exponentials; the scale is folded into one FMA.  The running
//    reference max is raised lazily: the output is rescaled only when a
//    column's max exceeds its reference by more than 2^8 (the weights stay
//    <= 256, harmless in float32/bf16), which after the first tiles is rare.
//  * Masks only on tiles that cross the diagonal or the window edge; tiles a
//    wave cannot see are skipped.
#include "common.h"
#include "launch.h"

#include <cstdlib>

namespace gqa {
namespace {

template <int HD>
struct PrefillCfg {
  static constexpr int BKV = 64;                    // keys per LDS tile (two 32-key sub-tiles)
  static constexpr int KS = HD / 16;                // 16-deep MFMA steps over hd
  static constexpr int RT = HD / 32;                // 32-row tiles of O^T
  static constexpr int KLD = HD + 8;                // K tile row (bf16)
  static constexpr int VLD = BKV + 8;               // V^T tile row (bf16)
  static constexpr int STAGE = BKV * KLD + HD * VLD;
};

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazily rescale beyond 2^8

__device__ __forceinline__ const bf16* kv_row(const AttnArgs& a, const void* fresh, const void* cache, int b, int j,
                                             int start, int kp) {
  if (kp >= start)
    return static_cast<const bf16*>(fresh) + (((int64_t)b * a.KV + j) * a.L + (kp - start)) * a.hd;
  const int slot = a.window > 0 ? kp % a.window : kp;
  return static_cast<const bf16*>(cache) + (((int64_t)b * a.KV + j) * a.cap + slot) * a.hd;
}

// Logical key (within a tile) of physical V^T slot e of 8-key chunk g: each
// 16-key group is stored as keys [0..3, 8..11, 4..7, 12..15], the order in
// which one lane's S^T accumulator holds them.
__device__ __forceinline__ int vt_key(int g, int e) {
  return (g >> 1) * 16 + (e < 4 ? (g & 1) * 4 + e : 8 + (g & 1) * 4 + (e - 4));
}

template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_prefill_kernel(AttnArgs a, int nqb, int paired) {
  using C = PrefillCfg<HD>;
  constexpr int NT = NW * 64, BKV = C::BKV, KS = C::KS, RT = C::RT;
  constexpr int KCH = (BKV * HD / 8 + NT - 1) / NT;    // 16-byte K chunks per thread
  constexpr int VUN = (BKV * HD / 32 + NT - 1) / NT;   // (8 keys x 4 dims) V units per thread
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.H / a.KV;
  const int wph = NW / G;          // waves per head
  const int BQ = 32 * wph;         // query positions per workgroup

  // Query blocks: unpaired, one per workgroup, longest first; paired (causal,
  // no window), workgroup p takes blocks nqb-1-p and p in turn, so every
  // workgroup has the same number of key tiles.
  const int bkv = a.B * a.KV;
  const int slot = (int)(blockIdx.x / bkv);
  const int bj = blockIdx.x % bkv;
  const int b = bj / a.KV, j = bj % a.KV;
  const int start = a.lengths ? a.lengths[b] : 0;
  const int L = a.L, W = a.window;
  const int npass = paired && slot < nqb - 1 - slot ? 2 : 1;

  for (int pass = 0; pass < npass; ++pass) {
  if (pass > 0) __syncthreads();  // the previous block's last LDS reads are done
  const int qb = pass == 0 ? nqb - 1 - slot : slot;
  const int q0 = qb * BQ;
  const int hh = w / wph, sub = w % wph;
  const int h = j * G + hh;
  const int qt0 = q0 + sub * 32;                     // first token of this wave
  const int qp_lo = start + qt0;                     // its position
  const int qp_hi = start + min(qt0 + 32, L) - 1;    // last valid position of this wave
  const int my_qp = start + qt0 + (lane & 31);       // this lane's query position

  const int blk_lo = start + q0, blk_hi = start + min(q0 + BQ, L) - 1;
  int klo = W > 0 ? max(0, blk_lo - W + 1) : 0;
  klo = klo / BKV * BKV;
  const int khi = blk_hi + 1;
  const int ntiles = (khi - klo + BKV - 1) / BKV;

  // ---- Q^T fragments: column = query token, 8 consecutive dims per lane ----
  bf16x8 qf[KS];
  {
    const int tok = min(qt0 + (lane & 31), L - 1);
    const bf16* qr = static_cast<const bf16*>(a.q) + ((int64_t)b * L + tok) * a.ldq + (int64_t)h * HD +
                     (lane >> 5) * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qr + ks * 16);
  }

  // ---- staging of one K/V tile ----
  u32x4 kreg[KCH];
  u32x2 vreg[VUN][8];
  auto gload = [&](int t) {
    const int kb = klo + t * BKV;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT;
      if (c < BKV * HD / 8) {
        const int r = c / (HD / 8), ch = c % (HD / 8);
        const int kp = min(kb + r, khi - 1);
        kreg[i] = *reinterpret_cast<const u32x4*>(kv_row(a, a.knew, a.kcache, b, j, start, kp) + ch * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT;
      if (u < BKV * HD / 32) {
        const int g = u % (BKV / 8), dg = u / (BKV / 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int kp = min(kb + vt_key(g, e), khi - 1);
          vreg[i][e] = *reinterpret_cast<const u32x2*>(kv_row(a, a.vnew, a.vcache, b, j, start, kp) + dg * 4);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    bf16* sK = smem + buf * C::STAGE;
    bf16* sV = sK + BKV * C::KLD;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * NT;
      if (c < BKV * HD / 8) {
        const int r = c / (HD / 8), ch = c % (HD / 8);
        *reinterpret_cast<u32x4*>(sK + r * C::KLD + ch * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VUN; ++i) {
      const int u = tid + i * NT;
      if (u < BKV * HD / 32) {
        const int g = u % (BKV / 8), dg = u / (BKV / 8);
        // vreg[i][e] holds dims 4dg..4dg+3 of key vt_key(g, e): transpose into 4 rows of V^T
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          u32x4 row;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const uint32_t x0 = vreg[i][2 * e2][r / 2], x1 = vreg[i][2 * e2 + 1][r / 2];
            const uint32_t h0 = (r & 1) ? (x0 >> 16) : (x0 & 0xffffu);
            const uint32_t h1 = (r & 1) ? (x1 >> 16) : (x1 & 0xffffu);
            row[e2] = h0 | (h1 << 16);
          }
          *reinterpret_cast<u32x4*>(sV + (dg * 4 + r) * C::VLD + g * 8) = row;
        }
      }
    }
  };

  // ---- accumulators and softmax state (per lane = per query column) ----
  f32x16 o[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[r][e] = 0.f;
  float m_ref = -INFINITY;   // reference max (log2 units) the weights are taken against
  float l_run = 0.f;         // this lane's share of the softmax denominator

  const float scale = 1.0f / sqrtf((float)HD);
  const float cap = a.softcap;
  const float s_log2 = scale * kLog2e;           // no softcap: t = s * scale * log2e
  const float cap_log2 = cap * kLog2e;           // softcap: t = cap * log2e * tanh(s * scale / cap)
  const float inv_cap = cap > 0.f ? scale / cap : 0.f;
  const bool wave_valid = qt0 < L;

  // scores of one 32-key sub-tile: S^T[32 keys][32 queries]
  auto qk = [&](const bf16* sK, int sb) {
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sK + (sb * 32 + (lane & 31)) * C::KLD + ks * 16 +
                                                        (lane >> 5) * 8);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
    }
    return s;
  };
  // softmax update for a sub-tile starting at key position k32; returns P^T (bf16) in s
  auto softmax = [&](f32x16& s, int k32) {
    const bool need_mask = (k32 + 31 > qp_lo) || (W > 0 && k32 < qp_hi - W + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = cap > 0.f ? cap_log2 * tanh_exp(s[e] * inv_cap) : s[e] * s_log2;
      if (need_mask) {
        const int kp = k32 + (e / 4) * 8 + (lane >> 5) * 4 + (e % 4);
        const bool ok = kp <= my_qp && (W == 0 || kp > my_qp - W);
        v = ok ? v : -INFINITY;
      }
      s[e] = v;
      mx = fmaxf(mx, v);
    }
    // raise the reference only when some column's max outgrew it by the slack
    if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, fmaxf(mx, xor32(mx)));
      const float alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[r][e] *= alpha;
    }
    const float mr = m_ref == -INFINITY ? 0.f : m_ref;
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = exp2_fast(s[e] - mr);
      s[e] = p;
      ls += p;
    }
    l_run += ls;
  };
  auto pv = [&](const bf16* sV, const f32x16& p, int sb) {
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = from_f32<bf16>(p[k16 * 8 + e]);
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sV + (r * 32 + (lane & 31)) * C::VLD + sb * 32 +
                                                          k16 * 16 + (lane >> 5) * 8);
        o[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[r], 0, 0, 0);
      }
    }
  };

  if (ntiles > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const bf16* sK = smem + buf * C::STAGE;
    const bf16* sV = sK + BKV * C::KLD;
    const int kb = klo + t * BKV;
    // which of the two sub-tiles this wave can see
    bool use[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int k32 = kb + sb * 32;
      use[sb] = wave_valid && !(k32 > qp_hi) && !(W > 0 && k32 + 31 < qp_lo - W + 1);
    }
    f32x16 s0, s1;
    if (use[0]) s0 = qk(sK, 0);
    if (use[1]) s1 = qk(sK, 1);
    if (use[0]) {
      softmax(s0, kb);
      pv(sV, s0, 0);
    }
    if (use[1]) {
      softmax(s1, kb + 32);
      pv(sV, s1, 1);
    }
    if (t + 1 < ntiles) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write ctx[token, h*HD + d] ----
  const int tok = qt0 + (lane & 31);
  const float lt = l_run + xor32(l_run);
  if (wave_valid && tok < L) {
    const float inv = 1.0f / lt;
    bf16* out = static_cast<bf16*>(a.ctx) + ((int64_t)b * L + tok) * ((int64_t)a.H * HD) + (int64_t)h * HD;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = r * 32 + e4 * 8 + (lane >> 5) * 4;
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = from_f32<bf16>(o[r][e4 * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(out + d) = v;
      }
  }
  }  // pass
}

// Waves per workgroup for group size G: G heads x floor(8 / G) waves of 32
// positions each (one wave per head when G >= 5).  head_dim 256 keeps 4 waves
// (one per SIMD, so each wave may hold its 256-row O^T and Q^T in registers).
int waves_for(int hd, int G) {
  if (hd == 256) return G * (G >= 4 ? 1 : 4 / G);
  return G * (G >= 5 ? 1 : 8 / G);
}

// Pairing evens out the causal triangle when the grid is small; with many
// workgroups (or a window, whose blocks have near-equal work) longest-first
// ordering balances well by itself.  GQA_ATTN_PAIR=0/1 overrides (tuning).
bool pair_blocks(const AttnArgs& a, int nqb) {
  static const int forced = [] {
    const char* e = getenv("GQA_ATTN_PAIR");
    return e ? atoi(e) : -1;
  }();
  if (forced >= 0) return forced != 0 && a.window == 0;
  return a.window == 0 && (int64_t)nqb * a.B * a.KV <= 4096;
}

template <int HD, int NW>
hipError_t launch_hd_nw(const AttnArgs& a, hipStream_t s) {
  const int G = a.H / a.KV;
  const int BQ = 32 * (NW / G);
  const int nqb = (a.L + BQ - 1) / BQ;
  const int paired = pair_blocks(a, nqb) ? 1 : 0;
  const int slots = paired ? (nqb + 1) / 2 : nqb;
  dim3 grid((unsigned)(slots * a.B * a.KV));
  hipLaunchKernelGGL((attn_prefill_kernel<HD, NW>), grid, dim3(NW * 64), 0, s, a, nqb, paired);
  return hipGetLastError();
}

template <int HD>
hipError_t launch_hd(const AttnArgs& a, hipStream_t s) {
  switch (waves_for(HD, a.H / a.KV)) {
    case 4: return launch_hd_nw<HD, 4>(a, s);
    case 5: return launch_hd_nw<HD, 5>(a, s);
    case 6: return launch_hd_nw<HD, 6>(a, s);
    case 8: return launch_hd_nw<HD, 8>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool attention_prefill_bf16_supported(int hd, int G) {
  const int nw = waves_for(hd, G);
  return (hd == 64 || hd == 128 || hd == 256) && (nw == 4 || nw == 5 || nw == 6 || nw == 8);
}

hipError_t launch_attention_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  if (a.B * a.L == 0) return hipSuccess;
  switch (a.hd) {
    case 64: return launch_hd<64>(a, s);
    case 128: return launch_hd<128>(a, s);
    case 256: return launch_hd<256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
