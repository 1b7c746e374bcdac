// Matrix-core backward of grouped-query causal attention (bf16 activations,
// head_dim 64 or 128) for the block's backward of a zero-state prefill.
//
// The softmax backward of the DantinoX "Core Layers" page's attention, with the
// flash idea of that page (recompute the probabilities from the row's
// log-sum-exp instead of storing them): with S = q k^T / sqrt(hd) (masked),
// P = exp(S - lse), dP = dO v^T, D = rowsum(dO * O):
//   dS = P * (dP - D),  dq = dS k / sqrt(hd),  dk = dS^T q / sqrt(hd),  dv = P^T dO.
// The forward kernel leaves lse (base 2) per (row, head, token) with each
// head's tokens contiguous; a prep kernel forms D in the same layout and a bf16
// copy of dO.
//
// Both kernels use the forward kernel's product shapes on
// v_mfma_f32_32x32x16_bf16 and its LDS conventions (direct-to-LDS tile loads,
// XOR-swizzled 16-byte chunks, transposing ds_read_b64_tr_b16 reads):
//  * "rows x columns": rows of a 32-row LDS tile (A operand) times 32 columns
//    held in registers (B operand): out[e] is tile row (e/4)*8 + (lane/32)*4 +
//    e%4, column lane%32.
//  * "transposed accumulate": acc^T[d][column] += sum over the tile's 32 rows
//    of tile[row][d] * w[row][column], w in the layout above converted to
//    bf16, the tile read transposed.
// attn_bwd_dq_kernel: a wave owns 32 queries of one head (as in the forward):
//   S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T over the key tiles.
// attn_bwd_dkv_kernel: a wave owns 32 keys; a workgroup (4 waves, 128 keys) one
//   query head of the group: S = Q K^T, dP = dO V^T, dS; dV^T += dO^T P,
//   dK^T += Q^T dS over the query tiles; the group's heads are summed later
//   (the per-head partials, in head order, by the RoPE-backward pack).
// Each LDS tile is staged twice when it is read both ways (row-swizzled for
// the A operand, column-swizzled for the transposing reads).
#include "attn_tile.h"
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

template <int HD>
struct BwdTile {
  static constexpr int ROWS = 32;                     // keys or queries per LDS tile
  static constexpr int RB = HD * 2;                   // bytes per row
  static constexpr int CR = HD / 8;                   // 16-byte chunks per row
  static constexpr int RP = RB >= 256 ? 1 : 256 / RB; // rows per 256 bytes of LDS
  static constexpr int RPI = 1024 / RB;               // rows per load instruction
  static constexpr int TILE = ROWS * RB;
  static constexpr int NI = TILE / 1024;              // load instructions per tile copy
  static constexpr int KS = HD / 16;                  // 16-deep MFMA steps over hd
  static constexpr int RT = HD / 32;                  // 32-row blocks of an accumulator^T
  static constexpr int XK = CR < 16 ? CR : 16;
  static __device__ __forceinline__ int kkey(int r) { return (r / RP) % XK; }
  static __device__ __forceinline__ int vkey(int r) { return 4 * ((r / RP) % (XK / 4)); }
};

__device__ __forceinline__ int acc_row(int e, int lane) { return (e / 4) * 8 + (lane >> 5) * 4 + (e % 4); }

template <int HD>
__device__ __forceinline__ f32x16 rows_x_cols(const char* tile, const bf16x8 (&bf)[BwdTile<HD>::KS], int lane) {
  using C = BwdTile<HD>;
  f32x16 s;
#pragma unroll
  for (int e = 0; e < 16; ++e) s[e] = 0.f;
  const char* base = tile + (lane & 31) * C::RB;
  const int khi = lane >> 5, key = C::kkey(lane & 31);
#pragma unroll
  for (int ks = 0; ks < C::KS; ++ks) {
    const bf16x8 af = *reinterpret_cast<const bf16x8*>(base + (((2 * ks + khi) ^ key) * 16));
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf[ks], s, 0, 0, 0);
  }
  return s;
}

// NOWAIT: the transposing reads go through inline asm (no compiler wait for
// outstanding global loads), waited for explicitly before each 16-key step.
template <int HD, bool NOWAIT = false>
__device__ __forceinline__ void tr_acc(const char* tile, const f32x16& w, f32x16 (&acc)[BwdTile<HD>::RT],
                                       int lane) {
  using C = BwdTile<HD>;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vrow = 4 * (g16 >> 1) + (i16 >> 2);
  const int vdim = 16 * (g16 & 1) + 4 * (i16 & 3);
  const int vk = C::vkey(vrow);  // rows vrow + 8 i share the swizzle
#pragma unroll
  for (int k16 = 0; k16 < 2; ++k16) {
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = from_f32<bf16>(w[k16 * 8 + e]);
    const int row = k16 * 16 + vrow;
    if constexpr (NOWAIT) {
      s16x4 lo[C::RT], hi[C::RT];
#pragma unroll
      for (int r = 0; r < C::RT; ++r) {
        const int d = r * 32 + vdim;
        const int off = ((d >> 3) ^ vk) * 16 + (d & 7) * 2;
        lo[r] = lds_read_tr16_nowait(tile + row * C::RB + off);
        hi[r] = lds_read_tr16_nowait(tile + (row + 8) * C::RB + off);
      }
      lgkm_wait<0>();
#pragma unroll
      for (int r = 0; r < C::RT; ++r) {
        tie(lo[r]);
        tie(hi[r]);
      }
#pragma unroll
      for (int r = 0; r < C::RT; ++r) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[r], hi[r], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[r], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int r = 0; r < C::RT; ++r) {
        const int d = r * 32 + vdim;
        const int off = ((d >> 3) ^ vk) * 16 + (d & 7) * 2;
        const s16x4 lo = lds_read_tr16(tile + row * C::RB + off);
        const s16x4 hi = lds_read_tr16(tile + (row + 8) * C::RB + off);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[r], 0, 0, 0);
      }
    }
  }
}

// ---- dq: a wave per 32 queries of one head, workgroups as the forward's ----
template <int HD, int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_bwd_dq_kernel(BwdAttnArgs a, const bf16* __restrict__ dob,
                                                                int nqb) {
  using C = BwdTile<HD>;
  constexpr int KS = C::KS, RT = C::RT;
  constexpr int STAGE = 3 * C::TILE;  // K (row swizzle), V (row swizzle), K (column swizzle)
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.H / a.KV, wph = NW / G, BQ = 32 * wph;
  const int bkv = a.B * a.KV;
  const int slot = (int)(blockIdx.x / bkv), bj = blockIdx.x % bkv;
  const int b = bj / a.KV, j = bj % a.KV;
  const int L = a.L, W = a.window;
  const int qb = nqb - 1 - slot;  // longest first
  const int q0 = qb * BQ;
  const int h = j * G + w / wph;
  const int qt0 = q0 + (w % wph) * 32;
  const int my_q = qt0 + (lane & 31);
  const bool wave_valid = qt0 < L;
  const int qp_lo = qt0, qp_hi = min(qt0 + 32, L) - 1;
  const int blk_lo = q0, blk_hi = min(q0 + BQ, L) - 1;
  int klo = W > 0 ? max(0, blk_lo - W + 1) : 0;
  klo = klo / 32 * 32;
  const int kend = blk_hi + 1;
  const int ntiles = (kend - klo + 31) / 32;
  const float s_log2 = a.scale * kLog2e;

  const int tokc = min(my_q, L - 1);
  const int64_t trow = (int64_t)b * L + tokc;
  const int khi = lane >> 5;
  bf16x8 qf[KS], df[KS];
  {
    const bf16* qr = static_cast<const bf16*>(a.q) + trow * a.ldq + (int64_t)h * HD + khi * 8;
    const bf16* dr = dob + trow * a.ldo + (int64_t)h * HD + khi * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *reinterpret_cast<const bf16x8*>(qr + ks * 16);
      df[ks] = *reinterpret_cast<const bf16x8*>(dr + ks * 16);
    }
  }
  const int64_t hrow = ((int64_t)b * a.H + h) * a.lse_ld + tokc;  // [B, H, lse_ld]
  const float lse2 = a.lse[hrow];
  const float dsum = a.dsum[hrow];
  const bf16* kbase = static_cast<const bf16*>(a.k) + ((int64_t)b * a.KV + j) * L * HD;
  const bf16* vbase = static_cast<const bf16*>(a.v) + ((int64_t)b * a.KV + j) * L * HD;

  auto issue = [&](int t, int stage) {
    const int kb = klo + t * 32;
    char* sK = smem + stage * STAGE;
    for (int i = w; i < C::NI; i += NW) {
      const int r = i * C::RPI + lane / C::CR, sl = lane % C::CR;
      const int kp = min(kb + r, kend - 1);
      const bf16* kr = kbase + (int64_t)kp * HD;
      const bf16* vr = vbase + (int64_t)kp * HD;
      load_lds16(kr + (sl ^ C::kkey(r)) * 8, sK + i * 1024);
      load_lds16(vr + (sl ^ C::kkey(r)) * 8, sK + C::TILE + i * 1024);
      load_lds16(kr + (sl ^ C::vkey(r)) * 8, sK + 2 * C::TILE + i * 1024);
    }
  };

  f32x16 acc[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[r][e] = 0.f;

  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
  lds_sync();
  if (ntiles > 1) issue(1, 1);
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    const char* sK = smem + stage * STAGE;
    const int kb = klo + t * 32;
    const bool use = wave_valid && !(kb > qp_hi) && !(W > 0 && kb + 31 < qp_lo - W + 1);
    if (use) {
      const f32x16 s = rows_x_cols<HD>(sK, qf, lane);              // S^T [keys][queries]
      const f32x16 dp = rows_x_cols<HD>(sK + C::TILE, df, lane);   // dP^T
      f32x16 ds;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int kp = kb + acc_row(e, lane);
        const bool ok = kp <= my_q && (W == 0 || kp > my_q - W);
        const float p = ok ? exp2_fast(s[e] * s_log2 - lse2) : 0.f;
        ds[e] = p * (dp[e] - dsum);
      }
      tr_acc<HD, true>(sK + 2 * C::TILE, ds, acc, lane);            // dQ^T += K^T dS^T
    }
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      lds_sync();
      if (t + 2 < ntiles) issue(t + 2, stage);
    }
  }
  if (wave_valid && my_q < L) {
    float* out = a.dq + (((int64_t)b * L + my_q) * a.H + h) * HD;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = r * 32 + e4 * 8 + (lane >> 5) * 4;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[r][e4 * 4 + e] * a.scale;
        *reinterpret_cast<f32x4*>(out + d) = v;
      }
  }
}

// ---- dk, dv: a wave per 32 keys, a workgroup per (128 keys, query head) ----
// Two workgroups per CU (64 KB of LDS each): the register budget of 256 per
// lane spills a few values at head_dim 128 and still runs faster (measured
// 0.85 vs 1.11 ms for the 4k prefill's attention backward) than one workgroup
// per CU without spills.
template <int HD>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkv_kernel(BwdAttnArgs a, const bf16* __restrict__ dob,
                                                             float* __restrict__ dkp, float* __restrict__ dvp) {
  using C = BwdTile<HD>;
  constexpr int NW = 4, KS = C::KS, RT = C::RT;
  // Q (row swizzle), dO (row), Q (column), dO (column), then the tile's 32
  // log-sum-exp and 32 D values (float32)
  constexpr int STAGE = 4 * C::TILE + 256;
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int G = a.H / a.KV;
  const int per = a.B * a.KV * G;
  const int kblk = (int)(blockIdx.x / per);  // key blocks from the first: longest first
  const int rest = blockIdx.x % per;
  const int b = rest / (a.KV * G), j = (rest / G) % a.KV, g = rest % G;
  const int h = j * G + g;
  const int L = a.L, W = a.window;
  const int k0 = kblk * 128;
  const int kw0 = k0 + w * 32;
  const int my_k = kw0 + (lane & 31);
  const bool wave_valid = kw0 < L;
  const int kw_hi = min(kw0 + 32, L) - 1;
  const int k_hi = min(k0 + 128, L) - 1;
  const int qlo = k0;
  const int qend = W > 0 ? min(L, k_hi + W) : L;
  const int ntiles = (qend - qlo + 31) / 32;
  const float s_log2 = a.scale * kLog2e;

  const int kc = min(my_k, L - 1);
  const int khi = lane >> 5;
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t o = (((int64_t)b * a.KV + j) * L + kc) * HD + khi * 8;
    const bf16* kr = static_cast<const bf16*>(a.k) + o;
    const bf16* vr = static_cast<const bf16*>(a.v) + o;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *reinterpret_cast<const bf16x8*>(kr + ks * 16);
      vf[ks] = *reinterpret_cast<const bf16x8*>(vr + ks * 16);
    }
  }
  const bf16* qbase = static_cast<const bf16*>(a.q) + (int64_t)b * L * a.ldq + (int64_t)h * HD;
  const bf16* dbase = dob + (int64_t)b * L * a.ldo + (int64_t)h * HD;
  const float* lse = a.lse + ((int64_t)b * a.H + h) * a.lse_ld;  // this head's queries contiguous
  const float* dsm = a.dsum + ((int64_t)b * a.H + h) * a.lse_ld;

  auto issue = [&](int t, int stage) {
    const int qb = qlo + t * 32;
    char* sQ = smem + stage * STAGE;
    for (int i = w; i < C::NI; i += NW) {
      const int r = i * C::RPI + lane / C::CR, sl = lane % C::CR;
      const int qp = min(qb + r, qend - 1);
      const bf16* qr = qbase + (int64_t)qp * a.ldq;
      const bf16* dr = dbase + (int64_t)qp * a.ldo;
      load_lds16(qr + (sl ^ C::kkey(r)) * 8, sQ + i * 1024);
      load_lds16(dr + (sl ^ C::kkey(r)) * 8, sQ + C::TILE + i * 1024);
      load_lds16(qr + (sl ^ C::vkey(r)) * 8, sQ + 2 * C::TILE + i * 1024);
      load_lds16(dr + (sl ^ C::vkey(r)) * 8, sQ + 3 * C::TILE + i * 1024);
    }
    // lanes 0-7 of wave 0: lse[qb .. qb + 31], lanes 8-15: D (16 bytes each;
    // starts past the padded row clamp back, their entries only feed masked rows)
    if (w == 0 && lane < 16) {
      const float* src = (lane < 8 ? lse : dsm) + min(qb + 4 * (lane & 7), a.lse_ld - 4);
      load_lds16(src, sQ + 4 * C::TILE);
    }
  };

  f32x16 dk[RT], dv[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int e = 0; e < 16; ++e) dk[r][e] = dv[r][e] = 0.f;

  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0f70);
  lds_sync();
  if (ntiles > 1) issue(1, 1);
  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    const char* sQ = smem + stage * STAGE;
    const int qb = qlo + t * 32;
    // some query of the tile sees some key of the wave
    const bool use = wave_valid && qb + 31 >= kw0 && !(W > 0 && qb > kw_hi + W - 1);
    if (use) {
      // this lane's rows are 4 runs of 4 consecutive queries: (e/4)*8 + (lane/32)*4 + e%4;
      // their lse / D entries are 16-byte reads of the tile's copies in LDS (entries
      // past L only feed masked rows)
      const float* sl = reinterpret_cast<const float*>(sQ + 4 * C::TILE);  // lse, then D at + 32
      auto q4 = [&](int e4) { return e4 * 8 + (lane >> 5) * 4; };
      f32x16 p = rows_x_cols<HD>(sQ, kf, lane);                     // S [queries][keys] -> P
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(sl + q4(e4));
#pragma unroll
        for (int e = 4 * e4; e < 4 * e4 + 4; ++e) {
          const int q = qb + acc_row(e, lane);
          const bool ok = q < L && q >= my_k && (W == 0 || q - my_k < W);
          p[e] = ok ? exp2_fast(p[e] * s_log2 - l4[e % 4]) : 0.f;
        }
      }
      tr_acc<HD, true>(sQ + 3 * C::TILE, p, dv, lane);              // dV^T += dO^T P
      f32x16 ds = rows_x_cols<HD>(sQ + C::TILE, vf, lane);          // dP -> dS
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(sl + 32 + q4(e4));
#pragma unroll
        for (int e = 4 * e4; e < 4 * e4 + 4; ++e)  // (p = 0 on masked rows; D's padding is unwritten)
          ds[e] = p[e] != 0.f ? p[e] * (ds[e] - d4[e % 4]) : 0.f;
      }
      tr_acc<HD, true>(sQ + 2 * C::TILE, ds, dk, lane);             // dK^T += Q^T dS
    }
    if (t + 1 < ntiles) {
      __builtin_amdgcn_s_waitcnt(0x0f70);
      lds_sync();
      if (t + 2 < ntiles) issue(t + 2, stage);
    }
  }
  if (wave_valid && my_k < L) {
    const int64_t o = (int64_t)g * a.kv_part_stride + (((int64_t)b * a.KV + j) * L + my_k) * HD;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = r * 32 + e4 * 8 + (lane >> 5) * 4;
        f32x4 x, y;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[e] = dk[r][e4 * 4 + e] * a.scale;
          y[e] = dv[r][e4 * 4 + e];
        }
        *reinterpret_cast<f32x4*>(dkp + o + d) = x;
        *reinterpret_cast<f32x4*>(dvp + o + d) = y;
      }
  }
}

// D = rowsum(dO * O) per (token, head) and dO in bf16: a wave per (token, head).
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(BwdAttnArgs a, bf16* __restrict__ dob) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)a.B * a.L * a.H) return;
  const int64_t tok = wid / a.H;
  const int h = (int)(wid % a.H);
  const float* dr = a.dout + tok * a.ldo + (int64_t)h * a.hd;
  const bf16* orow = static_cast<const bf16*>(a.o) + tok * a.ldo + (int64_t)h * a.hd;
  bf16* db = dob + tok * a.ldo + (int64_t)h * a.hd;
  float s = 0.f;
  for (int e = lane; e < a.hd; e += WAVE) {
    const float d = dr[e];
    s += d * to_f32(orow[e]);
    db[e] = from_f32<bf16>(d);
  }
  s = wave_sum(s);
  const int64_t b = tok / a.L, t = tok % a.L;
  if (lane == 0) a.dsum[(b * a.H + h) * a.lse_ld + t] = s;
}

// The same for head_dim 64 / 128: 16 lanes per (token, head), hd / 16
// consecutive dims per lane (16-byte loads and stores), group-of-16 sum.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_prep_vec_kernel(BwdAttnArgs a, bf16* __restrict__ dob) {
  constexpr int DPL = HD / 16;
  const int sub = threadIdx.x & 15;
  const int64_t n = (int64_t)a.B * a.L * a.H;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const bool ok = pair < n;
  const int64_t pc = ok ? pair : n - 1;  // every lane stays in the group sum
  const int64_t tok = pc / a.H;
  const int h = (int)(pc % a.H);
  const int64_t off = tok * a.ldo + (int64_t)h * HD + sub * DPL;
  const float* dr = a.dout + off;
  const bf16* orow = static_cast<const bf16*>(a.o) + off;
  float s = 0.f;
  bf16 ob[DPL];
#pragma unroll
  for (int c = 0; c < DPL / 4; ++c) {
    const f32x4 d4 = reinterpret_cast<const f32x4*>(dr)[c];
    const bf16x4 o4 = reinterpret_cast<const bf16x4*>(orow)[c];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s += d4[e] * to_f32(o4[e]);
      ob[4 * c + e] = from_f32<bf16>(d4[e]);
    }
  }
  if (ok) {
#pragma unroll
    for (int c = 0; c < DPL / 4; ++c) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = ob[4 * c + e];
      reinterpret_cast<bf16x4*>(dob + off)[c] = v;
    }
  }
  s += __shfl_xor(s, 1, WAVE);
  s += __shfl_xor(s, 2, WAVE);
  s += __shfl_xor(s, 4, WAVE);
  s += __shfl_xor(s, 8, WAVE);
  const int64_t b = tok / a.L, t = tok % a.L;
  if (ok && sub == 0) a.dsum[(b * a.H + h) * a.lse_ld + t] = s;
}

int dq_waves(int G) { return G * (G >= 5 ? 1 : 8 / G); }  // as the forward: G heads x 32-query waves

template <int HD>
hipError_t launch_hd(const BwdAttnArgs& a, bf16* dob, float* dkp, float* dvp, hipStream_t s) {
  const int G = a.H / a.KV;
  const int nw = dq_waves(G);
  const int BQ = 32 * (nw / G);
  const int nqb = (a.L + BQ - 1) / BQ;
  dim3 gq((unsigned)(nqb * a.B * a.KV));
  switch (nw) {
    case 4: hipLaunchKernelGGL((attn_bwd_dq_kernel<HD, 4>), gq, dim3(256), 0, s, a, dob, nqb); break;
    case 5: hipLaunchKernelGGL((attn_bwd_dq_kernel<HD, 5>), gq, dim3(320), 0, s, a, dob, nqb); break;
    case 6: hipLaunchKernelGGL((attn_bwd_dq_kernel<HD, 6>), gq, dim3(384), 0, s, a, dob, nqb); break;
    case 8: hipLaunchKernelGGL((attn_bwd_dq_kernel<HD, 8>), gq, dim3(512), 0, s, a, dob, nqb); break;
    default: return hipErrorInvalidValue;
  }
  const int nkb = (a.L + 127) / 128;
  dim3 gk((unsigned)(nkb * a.B * a.KV * G));
  hipLaunchKernelGGL(attn_bwd_dkv_kernel<HD>, gk, dim3(256), 0, s, a, dob, dkp, dvp);
  return hipGetLastError();
}

}  // namespace

bool attention_bwd_mfma_supported(int hd, int G) {
  const int nw = dq_waves(G);
  return (hd == 64 || hd == 128) && (nw == 4 || nw == 5 || nw == 6 || nw == 8);
}

hipError_t launch_attention_bwd_mfma(const BwdAttnArgs& a, void* dob, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.L * a.H;
  if (n == 0) return hipSuccess;
  if (!attention_bwd_mfma_supported(a.hd, a.H / a.KV) || a.kv_parts != a.H / a.KV || !a.lse)
    return hipErrorInvalidValue;
  if (a.ldo % 8 == 0 && (uintptr_t)a.dout % 16 == 0 && (uintptr_t)a.o % 16 == 0 && (uintptr_t)dob % 16 == 0) {
    const dim3 g((unsigned)((n + 15) / 16));
    if (a.hd == 64)
      hipLaunchKernelGGL(attn_bwd_prep_vec_kernel<64>, g, dim3(256), 0, s, a, static_cast<bf16*>(dob));
    else
      hipLaunchKernelGGL(attn_bwd_prep_vec_kernel<128>, g, dim3(256), 0, s, a, static_cast<bf16*>(dob));
  } else {
    hipLaunchKernelGGL(attn_bwd_prep_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, a,
                       static_cast<bf16*>(dob));
  }
  if (a.hd == 64) return launch_hd<64>(a, static_cast<bf16*>(dob), a.dk, a.dv, s);
  return launch_hd<128>(a, static_cast<bf16*>(dob), a.dk, a.dv, s);
}

}  // namespace gqa
