// Decode-sized bf16 "TN" GEMM (M <= 64 activation rows):
//   C[m, n] = sum_k A[m, k] * W[n, k]
// for the block's projections during single-token decode (mojolearn
// TransformerBlock: q/k/v, o_proj, gate/up, down), where every weight byte is
// used by at most 64 rows and the kernel is bound by streaming W from HBM.
//
// Streaming W at full HBM bandwidth is a question of how the loads are shaped
// (measured on gfx950 with this kernel's geometry, 4 waves x 32 rows per
// workgroup, M = 64): loads straight into LDS (global_load_lds) top out near
// 3.5 TB/s; register loads in MFMA operand layout (each instruction 64 bytes of
// 16 rows) near 4.3 TB/s; register loads that cover whole 256-byte row pieces
// (each instruction 4 rows x 256 bytes) near 5.3 TB/s.  So each wave streams
// its 32 weight rows in that whole-piece shape into a register ring of SK_D
// 128-deep chunks, and when a chunk comes due writes it to a private LDS slab
// (XOR-swizzled on 16-byte pieces) and reads it back in A-operand layout (lane
// l: row l % 16 of a 16-row group, 8 consecutive k at 8 (l / 16) of each
// 32-deep step); only the wave itself touches its slab, so no barrier is
// involved.  The activations (at most 64 rows, reused by every weight row) are
// shared through LDS in B-operand fragment order a 256-deep super-chunk at a
// time, double-buffered: each thread loads its share of super-chunk s + 1
// (whole row pieces again) into registers while super-chunk s is multiplied
// and writes it to LDS before the one barrier per super-chunk.  That barrier
// has no memory fence, so the weight loads stay in flight across it.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int SK_KX = 128;           // k per chunk (256 bytes of a row)
constexpr int SK_SC = 2;             // chunks per super-chunk (one LDS activation buffer)
constexpr int SK_D = 2;              // weight chunks in flight per wave (register ring)
constexpr int SK_KS = SK_KX / 32;    // MFMA k-steps per chunk
constexpr int SK_NW = 4;             // waves per workgroup
constexpr int SK_RG = 2;             // 16-row weight groups per wave
constexpr int SK_ROWS = SK_NW * SK_RG * 16;
constexpr int SK_WI = SK_RG * 4;     // weight load instructions per wave per chunk (4 rows each)

__device__ __forceinline__ float act_of(int act, float g) {
  return act == kActGeluTanh ? gelu_tanh(g) : silu(g);
}

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

template <int MT, int MODE, int EPI>
__global__ __launch_bounds__(SK_NW * 64, 1) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int WROWS = SK_RG * 16;              // weight rows per wave (32)
  constexpr int XF = SK_SC * SK_KS * MT;         // activation fragments (1 KB each) per super-chunk
  constexpr int XT = XF / SK_NW;                 // 16-byte activation pieces per thread per super-chunk
  static_assert(XF % SK_NW == 0, "activation pieces split evenly over the threads");
  __shared__ __attribute__((aligned(1024))) bf16x8 xs[2][XF][64];
  __shared__ __attribute__((aligned(1024))) bf16x8 wslab[SK_NW][WROWS * 16];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int z = blockIdx.y;
  const int64_t kb = (int64_t)z * a.k_split;
  const int nchunks = a.k_split / SK_KX;

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.bump_n; i += SK_NW * 64) a.bump[i] += a.bump_by;

  // ---- weights: load instruction q moves rows 4 q .. 4 q + 3 of the wave's 32
  // (rows 0-15 row group 0, 16-31 group 1), lane l: row 4 q + l / 16, 16-byte
  // piece l % 16 of the chunk's 256 bytes ----
  const bf16* wp[SK_WI];
#pragma unroll
  for (int q = 0; q < SK_WI; ++q) {
    const int wr = 4 * q + (lane >> 4);          // row within the wave's 32
    const bf16* row;
    if (MODE == kModeGated) {                    // group 0 gate, group 1 up, same 16 columns
      const int col = min(blockIdx.x * (SK_ROWS / 2) + wave * 16 + (wr & 15), a.N - 1);
      row = static_cast<const bf16*>(a.B[wr >> 4]) + (int64_t)col * a.K;
    } else {
      const int64_t n = min((int64_t)blockIdx.x * SK_ROWS + wave * WROWS + wr, (int64_t)a.N - 1);
      const int sg = seg_index(a, n);
      row = static_cast<const bf16*>(a.B[sg]) + (n - (sg == 0 ? 0 : a.seg_end[sg - 1])) * a.K;
    }
    wp[q] = row + kb + 8 * (lane & 15);
  }
  bf16x8 wr[SK_D][SK_WI];
  auto load_w = [&](int c, bf16x8 (&dst)[SK_WI]) {
#pragma unroll
    for (int q = 0; q < SK_WI; ++q)
      dst[q] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(wp[q] + c * SK_KX));
  };
  // slab slot of (row r of the wave's 32, 16-byte piece p): r * 16 + (p ^ (r % 16))
  bf16x8* slab = wslab[wave];

  // ---- activations: a super-chunk is MT*16 rows x 256 k = 32 pieces of 16 bytes
  // per row; this thread loads pieces tid + 256 i (row p / 32, piece p % 32;
  // rows past M repeat row M-1) and stores piece kp of row m at fragment
  // (kp / 4) * MT + m / 16, lane m % 16 + 16 (kp % 4) (B-operand order) ----
  const bf16* xbase = static_cast<const bf16*>(a.A) + kb;
  bf16x8 xr[XT];
  auto load_x = [&](int sc) {
#pragma unroll
    for (int i = 0; i < XT; ++i) {
      const int p = threadIdx.x + SK_NW * 64 * i;
      const int m = min(p / 32, a.M - 1);
      const int k = min(sc * (SK_SC * SK_KX) + (p % 32) * 8, a.k_split - 8);  // past the end: never read
      xr[i] = load_global16(xbase + (int64_t)m * a.lda + k);
    }
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int i = 0; i < XT; ++i) {
      const int p = threadIdx.x + SK_NW * 64 * i;
      const int m = p / 32, kp = p % 32;
      xs[buf][(kp / 4) * MT + m / 16][(m % 16) + 16 * (kp % 4)] = xr[i];
    }
  };

  f32x4 acc[SK_RG][MT];
#pragma unroll
  for (int r = 0; r < SK_RG; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, const bf16x8 (&w)[SK_WI]) {
    // the chunk through the wave's slab, from whole row pieces to A-operand layout
#pragma unroll
    for (int q = 0; q < SK_WI; ++q) {
      const int r = 4 * q + (lane >> 4), p = lane & 15;
      slab[r * 16 + (p ^ (r & 15))] = w[q];
    }
    const int buf = (c / SK_SC) & 1, cl = c % SK_SC;
#pragma unroll
    for (int ks = 0; ks < SK_KS; ++ks) {
      bf16x8 wf[SK_RG], xf[MT];
#pragma unroll
      for (int r = 0; r < SK_RG; ++r) {
        const int row = 16 * r + lr;
        wf[r] = slab[row * 16 + ((4 * ks + lg) ^ lr)];
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) xf[t] = xs[buf][(cl * SK_KS + ks) * MT + t][lane];
#pragma unroll
      for (int r = 0; r < SK_RG; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[r], xf[t], acc[r][t], 0, 0, 0);
    }
  };

  // ---- pipeline (nchunks is a multiple of SK_D = SK_SC).  Chunk c's weights
  // are loaded SK_D chunks ahead into ring slot c % SK_D (the loop is unrolled
  // by SK_D so the slots are registers).  Super-chunk s + 1's activations are
  // loaded into registers while super-chunk s is multiplied and written to LDS
  // buffer (s + 1) & 1 after it: that buffer was last read in super-chunk
  // s - 1, which every wave finished before the barrier that closed it.  Every
  // load is unconditional (indices clamp to the last chunk), and loads and
  // stores of one activation super-chunk fall in one loop iteration, so the
  // compiler's waits stay exact and never drain the weight stream. ----
  static_assert(SK_D == SK_SC, "one activation super-chunk per loop iteration");
  // (sched_barrier pins the issue order: the waits the compiler derives for
  // the loop must hold for the prologue's order as well)
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
      // keep the issue order: the scheduler would otherwise sink these loads
      // below the activation stores and the waits would cover them
      __builtin_amdgcn_sched_barrier(0);
    }
    store_x((c0 / SK_SC + 1) & 1);
    lds_barrier();
  }

  // Epilogue: acc[r][t] element e is weight row 4*lg + e of row group r and
  // activation row 16*t + lr, so each lane owns 4 consecutive output columns.
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + lr;
    if (m >= a.M) continue;
    if constexpr (MODE == kModeGated) {
      const int col = blockIdx.x * (SK_ROWS / 2) + wave * 16 + 4 * lg;
      if (col >= a.N) continue;
      if constexpr (EPI == kEpiPartial) {
        float* p = a.partial + ((int64_t)z * a.M + m) * (2 * (int64_t)a.N);
        *reinterpret_cast<f32x4*>(p + col) = acc[0][t];
        *reinterpret_cast<f32x4*>(p + a.N + col) = acc[1][t];
      } else {  // kEpiGated
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<bf16>(act_of(a.act, acc[0][t][e]) * acc[1][t][e]);
        *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + col) = o;
      }
    } else {
#pragma unroll
      for (int r = 0; r < SK_RG; ++r) {
        const int64_t n = (int64_t)blockIdx.x * SK_ROWS + wave * (SK_RG * 16) + r * 16 + 4 * lg;
        if (n >= a.N) continue;
        const f32x4 v = acc[r][t];
        if constexpr (EPI == kEpiPartial) {
          *reinterpret_cast<f32x4*>(a.partial + ((int64_t)z * a.M + m) * a.N + n) = v;
        } else if constexpr (EPI == kEpiResid) {
          const f32x4 rv = *reinterpret_cast<const f32x4*>(a.resid + (int64_t)m * a.ldr + n);
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.C) + (int64_t)m * a.ldc + n) = rv + v;
        } else {  // kEpiStore (+ bias); a segment boundary may fall inside the 4 columns
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t col = n + e;
            const int s = seg_index(a, col);
            const float b = a.bias[s] ? a.bias[s][col - (s == 0 ? 0 : a.seg_end[s - 1])] : 0.f;
            o[e] = from_f32<bf16>(v[e] + b);
          }
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + n) = o;
        }
      }
    }
  }
}

template <int MODE, int EPI>
hipError_t launch_mt(const GemmArgs& a, hipStream_t s) {
  const int64_t rows = MODE == kModeGated ? 2 * (int64_t)a.N : a.N;
  dim3 grid((unsigned)((rows + SK_ROWS - 1) / SK_ROWS), a.splits);
  dim3 block(SK_NW * 64);
  if (a.M <= 16) hipLaunchKernelGGL((gemm_skinny_kernel<1, MODE, EPI>), grid, block, 0, s, a);
  else if (a.M <= 32) hipLaunchKernelGGL((gemm_skinny_kernel<2, MODE, EPI>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((gemm_skinny_kernel<4, MODE, EPI>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool gemm_skinny_supported(int M, int N, int K, int k_split) {
  // whole super-chunks (an even number of 128-deep chunks) per split
  return M >= 1 && M <= 64 && N % 4 == 0 && K % 8 == 0 && k_split >= SK_SC * SK_KX && k_split % (SK_SC * SK_KX) == 0;
}

hipError_t launch_gemm_skinny(const GemmArgs& a, int mode, int epi, hipStream_t s) {
  if (!gemm_skinny_supported(a.M, a.N, a.K, a.k_split) || a.splits < 1 ||
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
