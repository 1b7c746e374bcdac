// Decode-sized bf16 "TN" GEMM (M <= 64 activation rows):
//   C[m, n] = sum_k A[m, k] * W[n, k]
// for the block's projections during single-token decode (mojolearn
// TransformerBlock: q/k/v, o_proj, gate/up, down), where every weight byte is
// used by at most 64 rows and the kernel is bound by streaming W from HBM.
//
// Streaming W at full HBM bandwidth is a question of how the loads are shaped
// and spread (measured on gfx950 with M = 64):
//  * loads straight into LDS (global_load_lds) top out near 3.5 TB/s, plain
//    register loads reach 5-6 TB/s;
//  * loads shaped as MFMA operands (64 bytes of each of 16 rows per
//    instruction) stream ~15 % slower than loads covering whole 256-byte row
//    pieces (4 rows x 256 bytes per instruction);
//  * every CU should stream the same number of bytes with several
//    independent waves: 256 workgroups of 7 waves, one 16-row weight group
//    each, beat 224 workgroups of 4 waves x 32 rows on the same matrix.
// So the work is cut into (16-row weight group, K split) tasks, one per wave;
// a workgroup holds `wg_waves` tasks of one K split, and the host picks the
// split count and the waves per workgroup so that the grid is (close to) one
// workgroup per CU.  Each wave streams its rows in whole-piece loads into a
// register ring of SK_D 128-deep chunks; a chunk coming due goes through the
// wave's private LDS slab (XOR-swizzled on 16-byte pieces) into the MFMA
// A-operand layout (lane l: row l % 16, 8 consecutive k at 8 (l / 16) of each
// 32-deep step) -- only the wave itself touches its slab, so no barrier is
// involved.  The activations (at most 64 rows, reused by every weight row) are
// shared through LDS in B-operand fragment order, a 256-deep super-chunk at a
// time, double-buffered: each thread loads its share of super-chunk s + 1
// (whole row pieces again) into registers while super-chunk s is multiplied
// and writes it to LDS before the one barrier per super-chunk.  That barrier
// has no memory fence, so the weight loads stay in flight across it.
//
// Gated mode (gate/up with act(gate) * up): a 16-row group is 8 gate rows and
// the 8 up rows of the same 8 output columns, so the gate and up results of a
// column sit in lanes l and l + 32 of one wave and meet through a lane swap.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int SK_KX = 128;           // k per chunk (256 bytes of a row)
constexpr int SK_SC = 2;             // chunks per super-chunk (one LDS activation buffer)
constexpr int SK_D = 2;              // weight chunks in flight per wave (register ring)
constexpr int SK_KS = SK_KX / 32;    // MFMA k-steps per chunk
constexpr int SK_MINW = 4, SK_MAXW = 8;  // waves per workgroup

__device__ __forceinline__ int seg_index(const GemmArgs& a, int64_t n) {
  return n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
}

// Workgroup-wide barrier that publishes this wave's LDS writes (lgkmcnt 0).  No
// memory fence: a workgroup-scope release fence would also wait for every
// outstanding global load (vmcnt 0) and drain the weight stream at each
// barrier.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16-byte load through the global address space: a generic (flat) load would
// count on both wait counters, and the compiler then waits for every
// outstanding load (vmcnt 0) before using its result.
__device__ __forceinline__ bf16x8 load_global16(const bf16* p) {
  return *(const __attribute__((address_space(1))) bf16x8*)p;
}

// Global row of row r (0..15) of weight group g.
template <int MODE>
__device__ __forceinline__ const bf16* group_row(const GemmArgs& a, int64_t g, int r) {
  if (MODE == kModeGated) {  // rows 0-7: gate columns 8g .., rows 8-15: up, same columns
    const int64_t col = min(8 * g + (r & 7), (int64_t)a.N - 1);
    return static_cast<const bf16*>(a.B[r >> 3]) + col * a.K;
  }
  const int64_t n = min(16 * g + r, (int64_t)a.N - 1);
  const int sg = seg_index(a, n);
  return static_cast<const bf16*>(a.B[sg]) + (n - (sg == 0 ? 0 : a.seg_end[sg - 1])) * a.K;
}

template <int MT, int NWV, int MODE, int EPI>
__global__ __launch_bounds__(NWV * 64, 1) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NT = NWV * 64;
  constexpr int XF = SK_SC * SK_KS * MT;         // activation fragments (1 KB each) per super-chunk
  constexpr int XP = XF * 64;                    // 16-byte activation pieces per super-chunk
  constexpr int XT = (XP + NT - 1) / NT;         // pieces per thread (the last may be a repeat)
  __shared__ __attribute__((aligned(1024))) bf16x8 xs[2][XF][64];
  __shared__ __attribute__((aligned(1024))) bf16x8 wslab[NWV][16 * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int z = blockIdx.y;
  const int64_t g = (int64_t)blockIdx.x * NWV + wave;   // this wave's 16-row weight group
  const int64_t kb = (int64_t)z * a.k_split;
  const int nchunks = a.k_split / SK_KX;

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.bump_n; i += NT) a.bump[i] += a.bump_by;

  // ---- weights: load instruction q moves rows 4 q .. 4 q + 3 of the group,
  // lane l: row 4 q + l / 16, 16-byte piece l % 16 of the chunk's 256 bytes ----
  const bf16* wp[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) wp[q] = group_row<MODE>(a, g, 4 * q + lg) + kb + 8 * lr;
  bf16x8 wr[SK_D][4];
  auto load_w = [&](int c, bf16x8 (&dst)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dst[q] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(wp[q] + c * SK_KX));
  };
  // slab slot of (row r, 16-byte piece p): r * 16 + (p ^ r)
  bf16x8* slab = wslab[wave];

  // ---- activations: a super-chunk is MT*16 rows x 256 k = 32 pieces of 16
  // bytes per row; this thread loads pieces tid + NT i (row p / 32, piece
  // p % 32; rows past M repeat row M-1; a piece index past the super-chunk
  // repeats the last piece and is not stored) and stores piece kp of row m at
  // fragment (kp / 4) * MT + m / 16, lane m % 16 + 16 (kp % 4) ----
  const bf16* xbase = static_cast<const bf16*>(a.A) + kb;
  // Slot of operand lane l in a fragment of k-step group g (fragment index / MT):
  // lane l ^ (2 (l / 16) + g % 2).  Eight consecutive writer lanes hold the
  // eight 16-byte pieces kp of one row -- lanes 16 (kp % 4) + row of two
  // fragment groups -- and land in eight distinct 16-byte bank groups; eight
  // consecutive reader lanes (l / 16 fixed) stay eight distinct slots.
  auto xslot = [](int l, int g) { return l ^ ((((l >> 4) & 3) << 1) | (g & 1)); };
  bf16x8 xr[XT];
  auto load_x = [&](int sc) {
#pragma unroll
    for (int i = 0; i < XT; ++i) {
      const int p = min((int)threadIdx.x + NT * i, XP - 1);
      const int m = min(p / 32, a.M - 1);
      const int k = min(sc * (SK_SC * SK_KX) + (p % 32) * 8, a.k_split - 8);  // past the end: never read
      xr[i] = load_global16(xbase + (int64_t)m * a.lda + k);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XT; ++i) {
      const int p = threadIdx.x + NT * i;
      if (XP % NT == 0 || p < XP) {
        const int m = p / 32, kp = p % 32;
        xs[buf][(kp / 4) * MT + m / 16][xslot((m % 16) + 16 * (kp % 4), kp / 4)] = xr[i];
      }
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, const bf16x8 (&w)[4]) {
    // the chunk through the wave's slab, from whole row pieces to A-operand layout
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * q + lg;
      slab[r * 16 + (lr ^ r)] = w[q];
    }
    const int buf = (c / SK_SC) & 1, cl = c % SK_SC;
#pragma unroll
    for (int ks = 0; ks < SK_KS; ++ks) {
      const bf16x8 wf = slab[lr * 16 + ((4 * ks + lg) ^ lr)];
      bf16x8 xf[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) xf[t] = xs[buf][(cl * SK_KS + ks) * MT + t][xslot(lane, cl * SK_KS + ks)];
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[t], acc[t], 0, 0, 0);
    }
  };

  // ---- pipeline (nchunks is a multiple of SK_D = SK_SC).  Chunk c's weights
  // are loaded SK_D chunks ahead into ring slot c % SK_D (the loop is unrolled
  // by SK_D so the slots are registers).  Super-chunk s + 1's activations are
  // loaded into registers while super-chunk s is multiplied and written to LDS
  // buffer (s + 1) & 1 after it: that buffer was last read in super-chunk
  // s - 1, which every wave finished before the barrier that closed it.  Every
  // load is unconditional (indices clamp), and loads and stores of one
  // activation super-chunk fall in one loop iteration, so the compiler's waits
  // stay exact and never drain the weight stream; sched_barrier pins the
  // issue order (the waits derived for the loop must hold for the prologue's
  // order as well). ----
  static_assert(SK_D == SK_SC, "one activation super-chunk per loop iteration");
  load_x(0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < SK_D; ++u) {
    load_w(u, wr[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  store_x(0);
  lds_barrier();
  for (int c0 = 0; c0 < nchunks; c0 += SK_D) {
    load_x(c0 / SK_SC + 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < SK_D; ++u) {
      const int c = c0 + u;
      compute(c, wr[u]);
      load_w(min(c + SK_D, nchunks - 1), wr[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x((c0 / SK_SC + 1) & 1);
    lds_barrier();
  }

  // ---- epilogue: acc[t] element e is weight row 4 lg + e of the group and
  // activation row 16 t + lr ----
  if constexpr (MODE == kModeGated && EPI == kEpiGated) {
    // gate rows 4 lg + e (lanes 0-31) and up rows 8 + 4 (lg - 2) + e (lanes
    // 32-63) are the same columns 8 g + 4 (lg & 1) + e: bring up to the gate lanes
    with_act(a.act, [&](auto act_c) {
    constexpr int ACT = decltype(act_c)::value;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4 up;
#pragma unroll
      for (int e = 0; e < 4; ++e) up[e] = xor32(acc[t][e]);
      const int m = 16 * t + lr;
      const int64_t col = 8 * g + 4 * (lg & 1);
      if (lane < 32 && m < a.M && col < a.N) {
        f32x4 gv = acc[t];
        if (a.bias[0]) gv += *reinterpret_cast<const f32x4*>(a.bias[0] + col);
        if (a.bias[1]) up += *reinterpret_cast<const f32x4*>(a.bias[1] + col);
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<bf16>(act_t<ACT>(gv[e]) * up[e]);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + col) = o;
      }
    }
    });
    return;
  }
  with_act(EPI == kEpiStore ? a.act : (int)kActNone, [&](auto act_c) {
  constexpr int ACT = decltype(act_c)::value;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + lr;
    if (m >= a.M) continue;
    const f32x4 v = acc[t];
    if constexpr (MODE == kModeGated) {  // kEpiPartial: gate at column col, up at N + col
      const int64_t col = 8 * g + 4 * (lg & 1);
      if (col >= a.N) continue;
      float* p = a.partial + ((int64_t)z * a.M + m) * (2 * (int64_t)a.N);
      *reinterpret_cast<f32x4*>(p + (lg >= 2 ? a.N : 0) + col) = v;
    } else {
      const int64_t n = 16 * g + 4 * lg;
      if (n >= a.N) continue;
      if constexpr (EPI == kEpiPartial) {
        *reinterpret_cast<f32x4*>(a.partial + ((int64_t)z * a.M + m) * a.N + n) = v;
      } else if constexpr (EPI == kEpiResid) {
        f32x4 r = v;
        if (a.bias[0]) r += *reinterpret_cast<const f32x4*>(a.bias[0] + n);
        if (a.resid) r = *reinterpret_cast<const f32x4*>(a.resid + (int64_t)m * a.ldr + n) + r;
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.C) + (int64_t)m * a.ldc + n) = r;
      } else {  // kEpiStore (+ bias, act); a segment boundary may fall inside the 4 columns
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t col = n + e;
          const int s = seg_index(a, col);
          const float b = a.bias[s] ? a.bias[s][col - (s == 0 ? 0 : a.seg_end[s - 1])] : 0.f;
          const float x = v[e] + b;
          o[e] = from_f32<bf16>(act_t<ACT>(x));
        }
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + n) = o;
      }
    }
  }
  });
}

template <int MT, int MODE, int EPI>
hipError_t launch_w(const GemmArgs& a, dim3 grid, hipStream_t s) {
  switch (a.wg_waves) {
    case 4: hipLaunchKernelGGL((gemm_skinny_kernel<MT, 4, MODE, EPI>), grid, dim3(4 * 64), 0, s, a); break;
    case 5: hipLaunchKernelGGL((gemm_skinny_kernel<MT, 5, MODE, EPI>), grid, dim3(5 * 64), 0, s, a); break;
    case 6: hipLaunchKernelGGL((gemm_skinny_kernel<MT, 6, MODE, EPI>), grid, dim3(6 * 64), 0, s, a); break;
    case 7: hipLaunchKernelGGL((gemm_skinny_kernel<MT, 7, MODE, EPI>), grid, dim3(7 * 64), 0, s, a); break;
    case 8: hipLaunchKernelGGL((gemm_skinny_kernel<MT, 8, MODE, EPI>), grid, dim3(8 * 64), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MODE, int EPI>
hipError_t launch_mt(const GemmArgs& a, hipStream_t s) {
  const int64_t groups = gemm_skinny_groups(a.N, MODE == kModeGated);
  dim3 grid((unsigned)(groups / a.wg_waves), a.splits);
  if (a.M <= 16) return launch_w<1, MODE, EPI>(a, grid, s);
  if (a.M <= 32) return launch_w<2, MODE, EPI>(a, grid, s);
  return launch_w<4, MODE, EPI>(a, grid, s);
}

}  // namespace

int64_t gemm_skinny_groups(int N, bool gated) { return gated ? ((int64_t)N + 7) / 8 : ((int64_t)N + 15) / 16; }

bool gemm_skinny_supported(int M, int N, int K, int k_split, int waves, bool gated) {
  // whole super-chunks (an even number of 128-deep chunks) per split, and the
  // weight groups split evenly over the workgroups
  return M >= 1 && M <= 64 && N % 4 == 0 && K % 8 == 0 && k_split >= SK_SC * SK_KX &&
         k_split % (SK_SC * SK_KX) == 0 && waves >= SK_MINW && waves <= SK_MAXW &&
         gemm_skinny_groups(N, gated) % waves == 0;
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int mode, int epi, hipStream_t s) {
  if (!gemm_skinny_supported(a.M, a.N, a.K, a.k_split, a.wg_waves, mode == kModeGated) || a.splits < 1 ||
      (int64_t)a.k_split * a.splits != a.K)
    return hipErrorInvalidValue;
  if (mode == kModeGated) {
    if (epi == kEpiGated) return launch_mt<kModeGated, kEpiGated>(a, s);
    if (epi == kEpiPartial) return launch_mt<kModeGated, kEpiPartial>(a, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case kEpiStore: return launch_mt<kModeSeg, kEpiStore>(a, s);
    case kEpiResid: return launch_mt<kModeSeg, kEpiResid>(a, s);
    case kEpiPartial: return launch_mt<kModeSeg, kEpiPartial>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
