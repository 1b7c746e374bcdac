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
//    accumulator converted to bf16.  The MFMA's inner (key) index may be
//    permuted freely as long as both operands agree, so V^T is fetched in the
//    key order in which a lane's accumulator holds P^T.
//  * K and V tiles of 64 keys stream from global memory straight into LDS
//    (global_load_lds_dwordx4, no register staging), row-major as stored,
//    double-buffered with one barrier per tile.  K fragments are plain
//    16-byte reads; V^T fragments come from the transposing read
//    ds_read_b64_tr_b16 (within a 16-lane group, lane i receives element i % 4
//    of the 8-byte pieces addressed by lanes 4e + i / 4), 4 keys x 1 dim per
//    lane per read.  Both tiles are XOR-swizzled on 16-byte chunks (chosen
//    through the global address each lane fetches) so that the fragment reads
//    of 16 consecutive rows, or the 8 rows x 64 bytes of a transposing read,
//    spread over all LDS banks.
//  * With whole-head RoPE, q arrives as the projection left it: the kernel
//    applies the per-head q norm and the rotation to its Q^T fragments in
//    registers (each lane holds both halves of every rotation pair), once
//    the first K/V tile's loads are in flight, which saves the RoPE kernel a
//    read and a write of every query.
//  * Softmax in float32 (dew CausalTransformer force_fp32_for_softmax) with
//    base-2 exponentials; the scale is folded into one multiply.  The running
//    reference max is raised lazily: the output is rescaled only when a
//    column's max exceeds its reference by more than 2^8 (the weights stay
//    <= 256, harmless in float32/bf16), which after the first tiles is rare.
//    The softcap variant is a separate instantiation; masks are selects on
//    tiles that cross the diagonal or the window edge only (wave-uniform
//    tests), and tiles a wave cannot see are skipped.
#include "attn_tile.h"
#include "common.h"
#include "launch.h"

#include <cstdlib>

namespace gqa {
namespace {

template <int HD>
struct PrefillCfg {
  static constexpr int BKV = 64;                      // keys per LDS tile (two 32-key sub-tiles)
  static constexpr int RB = HD * 2;                   // bytes per K / V row
  static constexpr int CR = HD / 8;                   // 16-byte chunks per row
  static constexpr int RP = RB >= 256 ? 1 : 256 / RB; // rows per 256 bytes of LDS
  static constexpr int RPI = 1024 / RB;               // rows per load instruction (64 lanes x 16 B)
  static constexpr int TILE = BKV * RB;               // bytes of a K (or V) tile
  static constexpr int NI = TILE / 1024;              // load instructions per K (or V) tile
  static constexpr int STAGE = 2 * TILE;              // K tile + V tile
  static constexpr int KS = HD / 16;                  // 16-deep MFMA steps over hd
  static constexpr int RT = HD / 32;                  // 32-row tiles of O^T
  static constexpr int XK = CR < 16 ? CR : 16;        // XOR range of the swizzles
  // K: 16 consecutive rows read one chunk each -> distinct bank groups
  static __device__ __forceinline__ int kkey(int r) { return (r / RP) % XK; }
  // V: a transposing read covers 8 rows x 4 chunks -> each bank group twice
  static __device__ __forceinline__ int vkey(int r) { return 4 * ((r / RP) % (XK / 4)); }
};

constexpr float kRescaleSlack = 8.0f;  // log2 units: lazily rescale beyond 2^8

// tanh(x) = 1 - 2 / (e^{2x} + 1) with the hardware reciprocal.
__device__ __forceinline__ float tanh_rcp(float x) {
  const float e = exp2_fast(2.0f * kLog2e * x);
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(e + 1.0f);
}

// q norm and RoPE of a lane's Q^T fragments (8 dims ks * 16 + khi * 8 .. + 7
// per step ks), for the whole-head rotation (rope_dim = head_dim): the
// rotate-half partner of step ks < KS/2 is step ks + KS/2 of the same lane.
// Same float32 arithmetic as the RoPE kernel; the head's sum of squares meets
// the other half of its dims in lane ^ 32.  Applied after the first K/V
// tile's loads are issued, so the cos / sin (and norm weight) loads wait
// alongside them.
template <int HD>
__device__ __forceinline__ void rope_q_frags(bf16x8 (&qf)[HD / 16], const AttnArgs& a, int pos, int khi) {
  constexpr int KS = HD / 16, HK = KS / 2, RH = HD / 2;
  const float* ct = a.cos_tab + (int64_t)pos * RH + khi * 8;
  const float* st = a.sin_tab + (int64_t)pos * RH + khi * 8;
  float x[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) x[ks][e] = to_f32(qf[ks][e]);
  if (a.q_norm) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += x[ks][e] * x[ks][e];
    ss += xor32(ss);
    const float r = 1.0f / sqrtf(ss / (float)HD + a.eps);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = a.q_norm[ks * 16 + khi * 8 + e];
        x[ks][e] *= r * (a.offset ? 1.0f + w : w);
      }
  }
#pragma unroll
  for (int ks = 0; ks < HK; ++ks) {
    const f32x4 c0 = *reinterpret_cast<const f32x4*>(ct + ks * 16), c1 = *reinterpret_cast<const f32x4*>(ct + ks * 16 + 4);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(st + ks * 16), s1 = *reinterpret_cast<const f32x4*>(st + ks * 16 + 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = e < 4 ? c0[e & 3] : c1[e & 3], sn = e < 4 ? s0[e & 3] : s1[e & 3];
      const float x1 = x[ks][e], x2 = x[ks + HK][e];
      qf[ks][e] = from_f32<bf16>(x1 * c - x2 * sn);
      qf[ks + HK][e] = from_f32<bf16>(x2 * c + x1 * sn);
    }
  }
}

__device__ __forceinline__ const bf16* kv_row(const AttnArgs& a, const void* fresh, const void* cache, int b, int j,
                                             int start, int kp) {
  if (kp >= start)
    return static_cast<const bf16*>(fresh) + (((int64_t)b * a.KV + j) * a.L + (kp - start)) * a.hd;
  const int slot = a.window > 0 ? kp % a.window : kp;
  return static_cast<const bf16*>(cache) + (((int64_t)b * a.KV + j) * a.cap + slot) * a.hd;
}

template <int HD, int NW, bool CAP>
__global__ __launch_bounds__(NW * 64, 1) void attn_prefill_kernel(AttnArgs a, int nqb, int paired) {
  using C = PrefillCfg<HD>;
  constexpr int BKV = C::BKV, KS = C::KS, RT = C::RT, RB = C::RB;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (scalar)
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
  const int start = guarded_start(a.lengths, b, a.L, position_limit(a.window, a.cap, a.max_pos), nullptr);
  // this row's tokens (a packed ragged row: its own length; row of token t in q / ctx)
  const int L = a.row_len ? a.row_len[b] : a.L, W = a.window;
  const int64_t row0 = a.row_start ? (int64_t)a.row_start[b] : (int64_t)b * a.L;
  const int npass = paired && slot < nqb - 1 - slot ? 2 : 1;

  // per-lane constants of the fragment reads
  const int kfrag = (lane & 31) * RB + 16 * 0;                   // K row lane % 32 of a 32-key sub-tile
  const int khi = lane >> 5;                                     // K chunk within a 16-deep step
  const int kkey = C::kkey(lane & 31);
  const int g16 = lane >> 4, i16 = lane & 15;                    // transposing reads: group, lane in group
  const int vrow = 4 * (g16 >> 1) + (i16 >> 2);                  // V row (key) offset of this lane's piece
  const int vdim = 16 * (g16 & 1) + 4 * (i16 & 3);               // V dim offset of this lane's piece
  const int vkey = C::vkey(vrow);                                // (rows +8, +16, ... share the key)

  const float scale = 1.0f / sqrtf((float)HD);
  const float s_log2 = scale * kLog2e;           // no softcap: t = s * scale * log2e
  const float cap_log2 = a.softcap * kLog2e;     // softcap: t = cap * log2e * tanh(s * scale / cap)
  const float inv_cap = CAP ? scale / a.softcap : 0.f;

  for (int pass = 0; pass < npass; ++pass) {
  if (pass > 0) __syncthreads();  // the previous block's last LDS reads are done
  const int qb = pass == 0 ? nqb - 1 - slot : slot;
  const int q0 = qb * BQ;
  if (q0 >= L) continue;  // past a ragged row's end (uniform over the workgroup)
  const int hh = w / wph, sub = w % wph;
  const int h = j * G + hh;
  const int qt0 = q0 + sub * 32;                     // first token of this wave
  const int qp_lo = start + qt0;                     // its position
  const int qp_hi = start + min(qt0 + 32, L) - 1;    // last valid position of this wave
  const int my_qp = start + qt0 + (lane & 31);       // this lane's query position
  const bool wave_valid = qt0 < L;

  const int blk_lo = start + q0, blk_hi = start + min(q0 + BQ, L) - 1;
  int klo = W > 0 ? max(0, blk_lo - W + 1) : 0;
  klo = klo / BKV * BKV;
  const int kend = blk_hi + 1;
  const int ntiles = (kend - klo + BKV - 1) / BKV;

  // ---- Q^T fragments: column = query token, 8 consecutive dims per lane ----
  bf16x8 qf[KS];
  int qpos;  // this lane's query position (clamped to the row's last token)
  {
    const int tok = min(qt0 + (lane & 31), L - 1);
    const bf16* qr = static_cast<const bf16*>(a.q) + (row0 + tok) * a.ldq + (int64_t)h * HD + khi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(qr + ks * 16);
    qpos = start + tok;
  }

  // ---- one K/V tile: C::NI load instructions each, spread over the waves.
  // A tile wholly of this call's keys (the usual case) takes per-lane offsets
  // fixed per pass plus one add; tiles reaching into the cache or past the
  // last key take the general row lookup. ----
  constexpr int MI = (C::NI + NW - 1) / NW;  // load instructions per wave per operand
  constexpr int MK = MI <= 2 ? MI : 1;       // offsets kept in registers (else formed per load)
  auto k_off = [&](int i) {
    const int r = i * C::RPI + lane / C::CR;
    return r * HD + ((lane % C::CR) ^ C::kkey(r)) * 8;
  };
  auto v_off = [&](int i) {
    const int r = i * C::RPI + lane / C::CR;
    return r * HD + ((lane % C::CR) ^ C::vkey(r)) * 8;
  };
  int koffs[MK], voffs[MK];
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    koffs[m] = k_off(w + NW * m);
    voffs[m] = v_off(w + NW * m);
  }
  // row kp of this call's keys / values is at fresh + kp * HD (kp >= start)
  const int64_t fresh_row0 = ((int64_t)b * a.KV + j) * a.L - start;
  const bf16* kfresh = static_cast<const bf16*>(a.knew) + fresh_row0 * HD;
  const bf16* vfresh = static_cast<const bf16*>(a.vnew) + fresh_row0 * HD;
  auto issue = [&](int t, int stage) {
    const int kb = klo + t * BKV;
    char* sK = smem + stage * C::STAGE;
    char* sV = sK + C::TILE;
    if (kb >= start && kb + BKV <= kend) {
#pragma unroll
      for (int m = 0; m < MI; ++m) {
        const int i = w + NW * m;
        if (MI * NW == C::NI || i < C::NI) {
          const int ko = MI <= 2 ? koffs[m % MK] : k_off(i), vo = MI <= 2 ? voffs[m % MK] : v_off(i);
          load_lds16(kfresh + (int64_t)kb * HD + ko, sK + i * 1024);
          load_lds16(vfresh + (int64_t)kb * HD + vo, sV + i * 1024);
        }
      }
      return;
    }
    for (int i = w; i < C::NI; i += NW) {
      const int r = i * C::RPI + lane / C::CR, sl = lane % C::CR;
      const int kp = min(kb + r, kend - 1);
      load_lds16(kv_row(a, a.knew, a.kcache, b, j, start, kp) + (sl ^ C::kkey(r)) * 8, sK + i * 1024);
      load_lds16(kv_row(a, a.vnew, a.vcache, b, j, start, kp) + (sl ^ C::vkey(r)) * 8, sV + i * 1024);
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

  // scores of one 32-key sub-tile: S^T[32 keys][32 queries]
  auto qk = [&](const char* sK, int sb) {
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    const char* base = sK + sb * 32 * RB + kfrag;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(base + (((2 * ks + khi) ^ kkey) * 16));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
    }
    return s;
  };
  // softmax update for a sub-tile starting at key position k32; leaves P^T in s
  auto softmax = [&](f32x16& s, int k32) {
    const bool need_mask = (k32 + 31 > qp_lo) || (W > 0 && k32 < qp_hi - W + 1);
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float v = CAP ? cap_log2 * tanh_rcp(s[e] * inv_cap) : s[e] * s_log2;
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
  // O^T += V^T P^T for a sub-tile: 16-key step k16 uses the lane's P^T values
  // 8 k16 .. 8 k16 + 7 (keys 16 k16 + {0..3, 8..11} + 4 (lane / 32)), so the
  // V^T fragment takes the same keys: two transposing reads of 4 keys each.
  auto pv = [&](const char* sV, const f32x16& p, int sb) {
#pragma unroll
    for (int k16 = 0; k16 < 2; ++k16) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = from_f32<bf16>(p[k16 * 8 + e]);
      const int row = sb * 32 + k16 * 16 + vrow;
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const int d = r * 32 + vdim;
        const int off = ((d >> 3) ^ vkey) * 16 + (d & 7) * 2;
        const s16x4 lo = lds_read_tr16(sV + row * RB + off);
        const s16x4 hi = lds_read_tr16(sV + (row + 8) * RB + off);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[r], 0, 0, 0);
      }
    }
  };

  // ---- interior tiles (every key visible to every query of the wave):
  // the two sub-tiles' matrix products overlap the other sub-tile's softmax.
  // QK(1) is issued step by step with P(0) = exp2 of sub-tile 0's scores
  // spread between its MFMAs; PV(0) likewise carries P(1).  The MFMAs run in
  // the matrix pipe while the same wave issues the independent VALU work.
  // Maxima are taken on the raw scores (the scale, and tanh of the softcap,
  // are increasing), and the scale folds into the exponent's fma. ----
  constexpr int EPS = 16 / KS;  // elements of the previous sub-tile per QK step
  const float s_k2 = 2.0f * kLog2e * inv_cap;       // softcap: tanh argument, times 2 log2e
  // scaled score of a raw maximum (log2 units)
  auto scaled = [&](float mx) {
    return CAP ? cap_log2 * (1.0f - 2.0f * __builtin_amdgcn_rcpf(exp2_fast(mx * s_k2) + 1.0f)) : mx * s_log2;
  };
  // exp2(scaled(s) - m) with nm = -m
  auto prob = [&](float sv, float nm) {
    if constexpr (CAP) {
      const float r = __builtin_amdgcn_rcpf(exp2_fast(sv * s_k2) + 1.0f);
      return exp2_fast(__builtin_fmaf(r, -2.0f * cap_log2, cap_log2 + nm));
    } else {
      return exp2_fast(__builtin_fmaf(sv, s_log2, nm));
    }
  };
  auto max16 = [&](const f32x16& v) {
    float m0 = fmaxf(fmaxf(v[0], v[1]), v[2]), m1 = fmaxf(fmaxf(v[3], v[4]), v[5]);
    float m2 = fmaxf(fmaxf(v[6], v[7]), v[8]), m3 = fmaxf(fmaxf(v[9], v[10]), v[11]);
    float m4 = fmaxf(fmaxf(v[12], v[13]), v[14]);
    return fmaxf(fmaxf(fmaxf(m0, m1), fmaxf(m2, m3)), fmaxf(m4, v[15]));
  };
  // raise the reference when a column's max outgrew it by the slack; returns
  // the factor the accumulated output was multiplied by (1 if unchanged)
  auto raise_ref = [&](float mxs) {
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(mxs > m_ref + kRescaleSlack)) {
      const float m_new = fmaxf(m_ref, fmaxf(mxs, xor32(mxs)));
      alpha = m_ref == -INFINITY ? 1.f : exp2_fast(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[r][e] *= alpha;
    }
    return alpha;
  };
  // V^T fragment pair of 16-key step k16 of sub-tile sb, output rows r*32..: two
  // transposing reads of 4 keys each
  auto vfrag = [&](const char* sV, int sb, int k16, int r) {
    const int row = sb * 32 + k16 * 16 + vrow;
    const int d = r * 32 + vdim;
    const int off = ((d >> 3) ^ vkey) * 16 + (d & 7) * 2;
    const s16x4 lo = lds_read_tr16(sV + row * RB + off);
    const s16x4 hi = lds_read_tr16(sV + (row + 8) * RB + off);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // One interior tile.  Fragment reads run two MFMA steps ahead: K fragments
  // (2 KS steps of QK(0) and QK(1)) through a two-slot ring of ordinary LDS
  // reads; V^T fragment pairs (4 RT steps of PV(0) and PV(1)) through a
  // three-slot ring of transposing reads issued as inline asm with explicit
  // lgkmcnt waits -- the builtin form would make the compiler wait for every
  // global load in flight first (vmcnt 0), i.e. for the next tile's
  // direct-to-LDS loads in the middle of this tile.  A V^T slot is refilled
  // one step after the MFMA that read it.  Each step is pinned as "MFMA, its
  // reads, its VALU share".
  auto tile_fast = [&](const char* sK, const char* sV) __attribute__((always_inline)) {
    const char* kb0 = sK + kfrag;
    auto kread = [&](int i) {  // K fragment i of 2 KS: sub-tile i / KS, step i % KS
      const char* base = kb0 + (i / KS) * 32 * RB;
      return *reinterpret_cast<const bf16x8*>(base + (((2 * (i % KS) + khi) ^ kkey) * 16));
    };
    s16x4 vlo[3], vhi[3];
    auto vissue = [&](int v) {  // V^T fragment v of 4 RT: sub-tile v / (2 RT), k16, r
      const int sb = v / (2 * RT), j = v % (2 * RT), k16 = j / RT, r = j % RT;
      const int row = sb * 32 + k16 * 16 + vrow;
      const int d = r * 32 + vdim;
      const char* p = sV + row * RB + ((d >> 3) ^ vkey) * 16 + (d & 7) * 2;
      vlo[v % 3] = lds_read_tr16_nowait(p);
      vhi[v % 3] = lds_read_tr16_nowait(p + 8 * RB);
    };
    constexpr int NK = 2 * KS, NV = 4 * RT;
    // V^T fragment v for its MFMA: every LDS operation issued after its two
    // reads is the next fragment's pair (issued one step earlier), if any
    auto vtake = [&](int v) {
      if (v + 1 < NV) lgkm_wait<2>();
      else lgkm_wait<0>();
      tie(vlo[v % 3]);
      tie(vhi[v % 3]);
      const bf16x8 f = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vlo[v % 3], vhi[v % 3], 0, 1, 2, 3, 4, 5, 6, 7));
      if (v + 2 < NV) vissue(v + 2);
      return f;
    };
    bf16x8 kring[2];
    kring[0] = kread(0);
    kring[1] = kread(1);
    auto ktake = [&](int i) {  // K fragment i; refills its slot with i + 2 (past the K steps: V^T 0, 1)
      const bf16x8 f = kring[i & 1];
      if (i + 2 < NK) kring[i & 1] = kread(i + 2);
      else vissue(i + 2 - NK);
      return f;
    };
    // stage 1: S0 = K0 Q^T
    f32x16 s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) s0[e] = s1[e] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktake(ks), qf[ks], s0, 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first MFMA of QK(1) goes ahead of sub-tile 0's statistics
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktake(KS), qf[0], s1, 0, 0, 0);
    raise_ref(scaled(max16(s0)));
    float nm = -m_ref;
    // stage 2: the rest of S1 = K1 Q^T, with P0 = exp2(scaled(S0) - m) between its MFMAs
    float ls = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks > 0) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ktake(KS + ks), qf[ks], s1, 0, 0, 0);
#pragma unroll
      for (int e = ks * EPS; e < (ks + 1) * EPS; ++e) {
        s0[e] = prob(s0[e], nm);  // in place: sub-tile 0's probabilities
        ls += s0[e];
      }
      if (ks > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, 4 * EPS, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += ls;
    bf16x8 p0[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 8; ++e) p0[h2][e] = from_f32<bf16>(s0[h2 * 8 + e]);
    // sub-tile 1's maximum; a raised reference also scales P0 (not yet added)
    const float alpha = raise_ref(scaled(max16(s1)));
    if (alpha != 1.f) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) p0[h2][e] = from_f32<bf16>(static_cast<float>(p0[h2][e]) * alpha);
    }
    nm = -m_ref;
    // stage 3: O += V0 P0, with P1 between its MFMAs
    ls = 0.f;
    constexpr int PER = 16 / (2 * RT);
#pragma unroll
    for (int j = 0; j < 2 * RT; ++j) {
      o[j % RT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vtake(j), p0[j / RT], o[j % RT], 0, 0, 0);
#pragma unroll
      for (int e = j * PER; e < (j + 1) * PER; ++e) {
        s1[e] = prob(s1[e], nm);
        ls += s1[e];
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 4 * PER, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += ls;
    // stage 4: O += V1 P1
    bf16x8 p1[2];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
      for (int e = 0; e < 8; ++e) p1[h2][e] = from_f32<bf16>(s1[h2 * 8 + e]);
#pragma unroll
    for (int j = 0; j < 2 * RT; ++j) {
      o[j % RT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vtake(2 * RT + j), p1[j / RT], o[j % RT], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- pipeline: tile t + 1 is in flight while tile t is multiplied.  Each
  // wave walks its tiles in three runs -- tiles at the window's lower edge
  // (masked), interior tiles (every key visible to every query of the wave:
  // tile_fast), tiles crossing the diagonal (masked) -- with one barrier per
  // tile in every run, so all waves stay in step.  (Separate loops keep the
  // two paths' registers apart.) ----
  if (ntiles > 0) issue(0, 0);
  if constexpr (HD <= 128)  // (head_dim 256 has no registers to spare: q rotated by the RoPE kernel)
    if (a.rope_q) rope_q_frags<HD>(qf, a, qpos, khi);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of tile 0 (and Q) are done
  lds_sync();
  if (ntiles > 1) issue(1, 1);
  auto next_tile = [&](int t) {
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): this wave's loads of tile t + 1 are done
      lds_sync();                          // ... everyone's; and stage t & 1 is free
      if (t + 2 < ntiles) issue(t + 2, t & 1);
    }
  };
  auto tile_masked = [&](int t) {
    const int stage = t & 1;
    const char* sK = smem + stage * C::STAGE;
    const char* sV = sK + C::TILE;
    const int kb = klo + t * BKV;
    // which of the two sub-tiles this wave can see (wave-uniform)
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
  };
  // interior run [t_lo, t_hi): tile t's keys klo + 64 t .. + 63 are all at or
  // below the wave's first query and (windowed) inside its last query's window
  int t_lo = 0, t_hi = 0;
  if (wave_valid) {
    if (W > 0) t_lo = max(0, (qp_hi - W + 1 - klo + BKV - 1) / BKV);
    t_hi = qp_lo - (BKV - 1) - klo >= 0 ? (qp_lo - (BKV - 1) - klo) / BKV + 1 : 0;
    t_lo = min(t_lo, ntiles);
    t_hi = min(max(t_hi, t_lo), ntiles);
  }
  int t = 0;
  for (; t < t_lo; ++t) {
    tile_masked(t);
    next_tile(t);
  }
  for (; t < t_hi; ++t) {
    const char* sK = smem + (t & 1) * C::STAGE;
    tile_fast(sK, sK + C::TILE);
    next_tile(t);
  }
  for (; t < ntiles; ++t) {
    tile_masked(t);
    next_tile(t);
  }

  // ---- normalise and write ctx[token, h*HD + d] (and, when asked, the row's
  // log-sum-exp of the scaled scores in base 2, for the backward) ----
  const int tok = qt0 + (lane & 31);
  const float lt = l_run + xor32(l_run);
  if (a.lse && wave_valid && tok < L && lane < 32)
    a.lse[((int64_t)b * a.H + h) * ((a.L + 3) & ~3) + tok] = m_ref + __log2f(lt);
  if (wave_valid && tok < L) {
    const float inv = 1.0f / lt;
    bf16* out = static_cast<bf16*>(a.ctx) + (row0 + tok) * ((int64_t)a.H * HD) + (int64_t)h * HD;
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
  if (forced >= 0) return forced != 0 && a.window == 0 && !a.row_len;
  // (packed ragged rows: a block's work depends on its position only, so the
  // longest-first order balances rows of any length; pairing by the padded
  // index would not)
  return a.window == 0 && !a.row_len && (int64_t)nqb * a.B * a.KV <= 4096;
}

template <int HD, int NW>
hipError_t launch_hd_nw(const AttnArgs& a, hipStream_t s) {
  const int G = a.H / a.KV;
  const int BQ = 32 * (NW / G);
  const int nqb = (a.L + BQ - 1) / BQ;
  const int paired = pair_blocks(a, nqb) ? 1 : 0;
  const int slots = paired ? (nqb + 1) / 2 : nqb;
  dim3 grid((unsigned)(slots * a.B * a.KV));
  if (a.softcap > 0.f)
    hipLaunchKernelGGL((attn_prefill_kernel<HD, NW, true>), grid, dim3(NW * 64), 0, s, a, nqb, paired);
  else
    hipLaunchKernelGGL((attn_prefill_kernel<HD, NW, false>), grid, dim3(NW * 64), 0, s, a, nqb, paired);
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
  if (a.rope_q && (a.rd != a.hd || a.hd > 128 || !a.cos_tab || !a.sin_tab)) return hipErrorInvalidValue;
  switch (a.hd) {
    case 64: return launch_hd<64>(a, s);
    case 128: return launch_hd<128>(a, s);
    case 256: return launch_hd<256>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
