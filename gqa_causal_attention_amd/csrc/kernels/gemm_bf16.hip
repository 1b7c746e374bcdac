// bf16 "TN" GEMM on gfx950 matrix cores: C[m, n] = sum_k A[m, k] * W[n, k],
// A = activations [M, K] and W = a Hugging Face [out, in] weight, both
// K-contiguous, so every MFMA operand is one 16-byte row chunk.
//
// The block's projections (mojolearn TransformerBlock: q/k/v, o_proj,
// gate/up, down) are all of this form.  Fused epilogues:
//   kEpiStore  : q/k/v from three weight segments in one launch, + bias
//   kEpiResid  : o_proj / down_proj plus the float32 residual stream
//   kEpiGated  : gate/up pair, act(gate) * up (SiLU or tanh-GELU)
//   kEpiPartial: float32 partial sums of one K split (decode-sized M)
//
// Structure: a workgroup owns a BM x BN tile; K advances in steps of 64
// through two LDS buffers (global -> registers -> LDS, one barrier per step);
// each wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16.  LDS rows are padded to 72 elements so the 16-byte
// fragment reads of 32 consecutive rows hit distinct banks.
#include "common.h"
#include "launch.h"

#include <cstdlib>

namespace gqa {
namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // padded LDS row (bf16 elements)

__device__ __forceinline__ int seg_of(const GemmArgs& a, int64_t n) {
  return n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
}

// Pointer to the start of B-tile row r (global K offset k0) for tile column tn.
// Gated mode: each wave's WTN B rows are WTN/2 gate rows then the WTN/2 up
// rows of the same output columns, so one lane holds both accumulators.
template <int MODE, int BN, int WTN>
__device__ __forceinline__ const bf16* b_row(const GemmArgs& a, int tn, int r, int k0) {
  if (MODE == kModeGated) {
    const int blk = r / WTN, w = r % WTN;
    int col = tn * (BN / 2) + blk * (WTN / 2) + (w % (WTN / 2));
    col = min(col, a.N - 1);
    const bf16* base = static_cast<const bf16*>(w < WTN / 2 ? a.B[0] : a.B[1]);
    return base + (int64_t)col * a.K + k0;
  } else {
    int64_t n = min((int64_t)tn * BN + r, (int64_t)a.N - 1);
    const int s = seg_of(a, n);
    const int64_t start = s == 0 ? 0 : a.seg_end[s - 1];
    return static_cast<const bf16*>(a.B[s]) + (n - start) * a.K + k0;
  }
}

template <int BM, int BN, int WGM, int WGN, int MODE, int EPI, int WPOS>
__global__ __launch_bounds__(WGM* WGN * 64, 1) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int CPR = BK / 8;  // 16-byte chunks per row
  constexpr int CH_A = BM * CPR / NT, CH_B = BN * CPR / NT;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile loads must divide evenly");
  static_assert(MODE != kModeGated || FN % 2 == 0, "gated wave tiles hold gate and up halves");
  constexpr int STAGE = (BM + BN) * LDK;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.bump_n; i += NT) a.bump[i] += a.bump_by;

  // ---- tile order: XCD-contiguous, then groups of 4 M-tiles across N ----
  const int cols_per_tile = MODE == kModeGated ? BN / 2 : BN;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + cols_per_tile - 1) / cols_per_tile;
  const int total = gridDim.x;
  int pid = blockIdx.x;
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  constexpr int GROUP_M = 4;
  const int group = pid / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int rem = pid % (GROUP_M * tiles_n);
  const int tm = first_m + rem % gsize;
  const int tn = rem / gsize;
  const int m0 = tm * BM;

  const int kbeg = blockIdx.y * a.k_split;
  const int nk = (min(a.K, kbeg + a.k_split) - kbeg) / BK;

  // ---- per-thread global row pointers (rows past M / N are clamped) ----
  const int kc = tid % CPR;
  const bf16* ap[CH_A];
  const bf16* bp[CH_B];
  const bf16* A = static_cast<const bf16*>(a.A);
#pragma unroll
  for (int i = 0; i < CH_A; ++i) {
    const int row = tid / CPR + i * (NT / CPR);
    const int m = min(m0 + row, a.M - 1);
    ap[i] = A + (int64_t)m * a.lda + kbeg + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < CH_B; ++i) {
    const int row = tid / CPR + i * (NT / CPR);
    bp[i] = b_row<MODE, BN, WTN>(a, tn, row, kbeg) + kc * 8;
  }

  u32x4 ra[CH_A], rb[CH_B];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < CH_A; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < CH_B; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + kt * BK);
  };
  auto sstore = [&](int buf) {
    bf16* sA = smem + buf * STAGE;
    bf16* sB = sA + BM * LDK;
#pragma unroll
    for (int i = 0; i < CH_A; ++i) {
      const int row = tid / CPR + i * (NT / CPR);
      *reinterpret_cast<u32x4*>(sA + row * LDK + kc * 8) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CH_B; ++i) {
      const int row = tid / CPR + i * (NT / CPR);
      *reinterpret_cast<u32x4*>(sB + row * LDK + kc * 8) = rb[i];
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Fragment registers are double-buffered across the 16-deep k-steps of a
  // tile (the reads for step ks+1 are in flight while step ks's MFMAs issue),
  // and the next tile's LDS write is issued after step WPOS-1 so that only
  // the barrier is left at the end of the tile.
  constexpr int KS = BK / 16;
  const int frag_row = lane & 31, frag_k = (lane >> 5) * 8;
  bf16x8 fa[2][FM], fb[2][FN];
  auto lfrag = [&](int buf, int ks, int slot) {
    const bf16* sA = smem + buf * STAGE;
    const bf16* sB = sA + BM * LDK;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      fa[slot][i] = *reinterpret_cast<const bf16x8*>(sA + (wm * WTM + i * 32 + frag_row) * LDK + ks * 16 + frag_k);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      fb[slot][j] = *reinterpret_cast<const bf16x8*>(sB + (wn * WTN + j * 32 + frag_row) * LDK + ks * 16 + frag_k);
  };

  if (nk > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();
  if (nk > 0) lfrag(0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) lfrag(buf, ks + 1, cur ^ 1);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
      if (ks == WPOS - 1 && more) sstore(buf ^ 1);
    }
    __syncthreads();
    if (more) lfrag(buf ^ 1, 0, 0);
  }

  // ---- epilogue: accumulator (i, lane) holds row (i/4)*8 + (lane/32)*4 + i%4, column lane%32 ----
  // (the activation is resolved once: one compiled loop per activation)
  with_act(EPI == kEpiGated || EPI == kEpiStore ? a.act : (int)kActNone, [&](auto act_c) {
  constexpr int ACT = decltype(act_c)::value;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = m0 + wm * WTM + i * 32 + (e / 4) * 8 + (lane >> 5) * 4 + (e % 4);
      if (m >= a.M) continue;
      if constexpr (EPI == kEpiGated) {
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int n = tn * (BN / 2) + wn * (WTN / 2) + j * 32 + (lane & 31);
          if (n < a.N) {
            const float g = acc[i][j][e] + (a.bias[0] ? a.bias[0][n] : 0.f);
            const float u = acc[i][j + FN / 2][e] + (a.bias[1] ? a.bias[1][n] : 0.f);
            static_cast<bf16*>(a.C)[(int64_t)m * a.ldc + n] = from_f32<bf16>(act_t<ACT>(g) * u);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int cb = wn * WTN + j * 32 + (lane & 31);  // B row within the tile
          const float v = acc[i][j][e];
          if (EPI == kEpiPartial) {
            int64_t nb;
            int64_t NB;
            if (MODE == kModeGated) {
              const int blk = cb / WTN, w = cb % WTN;
              const int col = tn * (BN / 2) + blk * (WTN / 2) + (w % (WTN / 2));
              if (col >= a.N) continue;
              nb = (w < WTN / 2 ? 0 : a.N) + col;
              NB = 2 * (int64_t)a.N;
            } else {
              nb = (int64_t)tn * BN + cb;
              if (nb >= a.N) continue;
              NB = a.N;
            }
            a.partial[((int64_t)blockIdx.y * a.M + m) * NB + nb] = v;
          } else {
            const int64_t n = (int64_t)tn * BN + cb;
            if (n >= a.N) continue;
            if (EPI == kEpiResid) {
              const float t = v + (a.bias[0] ? a.bias[0][n] : 0.f);
              static_cast<float*>(a.C)[(int64_t)m * a.ldc + n] = a.resid ? a.resid[(int64_t)m * a.ldr + n] + t : t;
            } else {  // kEpiStore
              const int s = seg_of(a, n);
              const float b = a.bias[s] ? a.bias[s][n - (s == 0 ? 0 : a.seg_end[s - 1])] : 0.f;
              const float t = v + b;
              static_cast<bf16*>(a.C)[(int64_t)m * a.ldc + n] = from_f32<bf16>(act_t<ACT>(t));
            }
          }
        }
      }
    }
  }
  });
}

// Sum of the K-split partials in split order, then the epilogue.
template <typename OutT, int MODE, int EPI>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs a, int rows_in_y) {
  const int64_t N4 = a.N / 4;
  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.bump_n; i += 256) a.bump[i] += a.bump_by;
  // rows_in_y: grid y = row, x = blocks of 4-column groups (no 64-bit division);
  // else a 1-D grid over row x group
  int64_t m, n;
  if (rows_in_y) {
    const int q = blockIdx.x * 256 + threadIdx.x;
    if (q >= N4) return;
    m = blockIdx.y;
    n = (int64_t)q * 4;
  } else {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)a.M * N4) return;
    m = idx / N4;
    n = (idx % N4) * 4;
  }
  const int64_t NB = MODE == kModeGated ? 2 * (int64_t)a.N : a.N;
  f32x4 s = {0.f, 0.f, 0.f, 0.f}, su = {0.f, 0.f, 0.f, 0.f};
  // (unrolled so the splits' loads are in flight together; the adds stay in split order)
#pragma unroll 8
  for (int z = 0; z < a.splits; ++z) {
    const float* p = a.partial + ((int64_t)z * a.M + m) * NB;
    s += *reinterpret_cast<const f32x4*>(p + n);
    if (MODE == kModeGated) su += *reinterpret_cast<const f32x4*>(p + a.N + n);
  }
  if (EPI == kEpiResid) {
    if (a.bias[0]) s += *reinterpret_cast<const f32x4*>(a.bias[0] + n);
    if (a.resid) s = *reinterpret_cast<const f32x4*>(a.resid + m * a.ldr + n) + s;
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.C) + m * a.ldc + n) = s;
  } else {
    OutT* c = static_cast<OutT*>(a.C) + m * a.ldc + n;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v;
      if (EPI == kEpiGated) {
        const float g = s[e] + (a.bias[0] ? a.bias[0][n + e] : 0.f);
        const float u = su[e] + (a.bias[1] ? a.bias[1][n + e] : 0.f);
        v = act_fn(a.act, g) * u;
      } else {
        const int64_t col = n + e;
        const int sg = seg_of(a, col);
        v = s[e] + (a.bias[sg] ? a.bias[sg][col - (sg == 0 ? 0 : a.seg_end[sg - 1])] : 0.f);
        if (a.act != kActNone) v = act_fn(a.act, v);
      }
      c[e] = from_f32<OutT>(v);
    }
  }
}

int g_wpos = -1;  // LDS write position override (tuning), read once from GQA_GEMM_WPOS

template <int BM, int BN, int WGM, int WGN, int MODE, int EPI>
hipError_t launch_tile(const GemmArgs& a, hipStream_t s) {
  const int cols = MODE == kModeGated ? BN / 2 : BN;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + cols - 1) / cols);
  dim3 grid(tiles, a.splits);
  if (g_wpos < 0) {
    const char* e = getenv("GQA_GEMM_WPOS");
    g_wpos = e ? atoi(e) : 3;
  }
  switch (g_wpos) {
    case 2: hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, MODE, EPI, 2>), grid, dim3(WGM * WGN * 64), 0, s, a); break;
    case 4: hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, MODE, EPI, 4>), grid, dim3(WGM * WGN * 64), 0, s, a); break;
    default: hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, MODE, EPI, 3>), grid, dim3(WGM * WGN * 64), 0, s, a); break;
  }
  return hipGetLastError();
}

template <int MODE, int EPI>
hipError_t dispatch_tile(const GemmArgs& a, int tile, hipStream_t s) {
  switch (tile) {
    case kTile256x256: return launch_tile<256, 256, 2, 4, MODE, EPI>(a, s);
    case kTile256x256w4: return launch_tile<256, 256, 2, 2, MODE, EPI>(a, s);
    case kTile256x192:
      if constexpr (MODE == kModeGated) return hipErrorInvalidValue;
      else return launch_tile<256, 192, 4, 2, MODE, EPI>(a, s);
    case kTile128x128: return launch_tile<128, 128, 2, 2, MODE, EPI>(a, s);
    case kTile64x128: return launch_tile<64, 128, 1, 2, MODE, EPI>(a, s);
    case kTile64x64: return launch_tile<64, 64, 2, 1, MODE, EPI>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& a, int mode, int epi, int tile, hipStream_t s) {
  if (tile == kTileSkinny) return launch_gemm_skinny(a, mode, epi, s);
  if (gemm_dma_tile(tile)) return launch_gemm_dma(a, mode, epi, tile, s);
  if (mode == kModeGated) {
    if (epi == kEpiGated) return dispatch_tile<kModeGated, kEpiGated>(a, tile, s);
    if (epi == kEpiPartial) return dispatch_tile<kModeGated, kEpiPartial>(a, tile, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case kEpiStore: return dispatch_tile<kModeSeg, kEpiStore>(a, tile, s);
    case kEpiResid: return dispatch_tile<kModeSeg, kEpiResid>(a, tile, s);
    case kEpiPartial: return dispatch_tile<kModeSeg, kEpiPartial>(a, tile, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_splitk_reduce(const GemmArgs& a, int mode, int epi, int out_type, hipStream_t s) {
  const int64_t work = (int64_t)a.M * (a.N / 4);
  const int rows_in_y = a.M <= 65535 ? 1 : 0;
  dim3 grid = rows_in_y ? dim3((unsigned)((a.N / 4 + 255) / 256), (unsigned)a.M) : dim3((unsigned)((work + 255) / 256));
  if (mode == kModeGated) {
    if (epi != kEpiGated) return hipErrorInvalidValue;
    if (out_type == kBF16)
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16, kModeGated, kEpiGated>), grid, dim3(256), 0, s, a, rows_in_y);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<float, kModeGated, kEpiGated>), grid, dim3(256), 0, s, a, rows_in_y);
  } else if (epi == kEpiResid) {
    hipLaunchKernelGGL((splitk_reduce_kernel<float, kModeSeg, kEpiResid>), grid, dim3(256), 0, s, a, rows_in_y);
  } else if (epi == kEpiStore) {
    if (out_type == kBF16)
      hipLaunchKernelGGL((splitk_reduce_kernel<bf16, kModeSeg, kEpiStore>), grid, dim3(256), 0, s, a, rows_in_y);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<float, kModeSeg, kEpiStore>), grid, dim3(256), 0, s, a, rows_in_y);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gqa
