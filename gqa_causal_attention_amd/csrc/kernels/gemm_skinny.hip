// Decode-sized bf16 "TN" GEMM (M <= 64 activation rows):
//   C[m, n] = sum_k A[m, k] * W[n, k]
// for the block's projections during single-token decode (mojolearn
// TransformerBlock: q/k/v, o_proj, gate/up, down), where every weight byte is
// used by at most 64 rows and the kernel is bound by streaming W from HBM.
//
// What bounds it is bytes in flight, not arithmetic: a CU must keep tens of KB
// of weight loads outstanding to cover HBM latency.  So W never goes through
// LDS: each lane loads its 16-byte weight chunks straight into registers in
// the A-operand layout of v_mfma_f32_16x16x32_bf16 (lane l: weight row l%16,
// k-slots 8*(l/16)..+7 of a 32-deep k-step), a whole 128-deep chunk ahead of
// the MFMAs that consume it.  The activations are the part reused across
// weight rows; a workgroup stages each 128-deep chunk of them once in LDS, in
// B-operand fragment order (1 KB per 16 rows x 32 k, lane l at byte 16*l), so
// every fragment read is one conflict-free ds_read_b128.
//
// Workgroup: 4 waves x 2 row groups x 16 weight rows = 128 weight rows (gated
// mode: 64 output columns, each wave holding 16 gate rows and the 16 up rows
// of the same columns so act(gate) * up is formed in-lane), over one K split.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int SK_KX = 128;           // k per chunk (one LDS buffer)
constexpr int SK_KS = SK_KX / 32;    // MFMA k-steps per chunk
constexpr int SK_NW = 4;             // waves per workgroup
constexpr int SK_RG = 2;             // 16-row weight groups per wave
constexpr int SK_ROWS = SK_NW * SK_RG * 16;

__device__ __forceinline__ float act_of(int act, float g) {
  return act == kActGeluTanh ? gelu_tanh(g) : silu(g);
}

__device__ __forceinline__ int seg_index(const GemmArgs& a, int64_t n) {
  return n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
}

// Workgroup-wide barrier for the LDS staging: the LDS writes are complete
// (lgkmcnt 0) before the barrier; outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int MT, int MODE, int EPI>
__global__ __launch_bounds__(SK_NW * 64, 2) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int XF = MT * SK_KS;     // activation fragments per chunk
  constexpr int XPW = XF / SK_NW;    // fragments each wave stages per chunk
  static_assert(XF % SK_NW == 0, "activation fragments split evenly over the waves");
  __shared__ bf16x8 xs[2][XF][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int z = blockIdx.y;
  const int64_t kb = (int64_t)z * a.k_split;
  const int nchunks = a.k_split / SK_KX;

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.bump_n; i += SK_NW * 64) a.bump[i] += a.bump_by;

  // This lane's weight rows (one per row group), advanced to its k-slots.
  const bf16* wp[SK_RG];
#pragma unroll
  for (int r = 0; r < SK_RG; ++r) {
    if (MODE == kModeGated) {
      const int col = min(blockIdx.x * (SK_ROWS / 2) + wave * 16 + lr, a.N - 1);
      wp[r] = static_cast<const bf16*>(a.B[r]) + (int64_t)col * a.K;
    } else {
      const int64_t n = min((int64_t)blockIdx.x * SK_ROWS + wave * (SK_RG * 16) + r * 16 + lr, (int64_t)a.N - 1);
      const int s = seg_index(a, n);
      wp[r] = static_cast<const bf16*>(a.B[s]) + (n - (s == 0 ? 0 : a.seg_end[s - 1])) * a.K;
    }
    wp[r] += kb + 8 * lg;
  }
  // The activation fragments this wave stages: f = wave * XPW + j holds k-step
  // f / MT and rows 16 * (f % MT) + (0..15); rows past M repeat row M-1.
  const bf16* xp[XPW];
#pragma unroll
  for (int j = 0; j < XPW; ++j) {
    const int f = wave * XPW + j;
    const int m = min(16 * (f % MT) + lr, a.M - 1);
    xp[j] = static_cast<const bf16*>(a.A) + (int64_t)m * a.lda + kb + 32 * (f / MT) + 8 * lg;
  }

  f32x4 acc[SK_RG][MT];
#pragma unroll
  for (int r = 0; r < SK_RG; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bf16x8 wb0[SK_KS][SK_RG], wb1[SK_KS][SK_RG], xst[XPW];
  auto load_w = [&](bf16x8 (&w)[SK_KS][SK_RG], int c) {
#pragma unroll
    for (int s = 0; s < SK_KS; ++s)
#pragma unroll
      for (int r = 0; r < SK_RG; ++r)
        w[s][r] = *reinterpret_cast<const bf16x8*>(wp[r] + c * SK_KX + 32 * s);
    // keep the prefetch ahead of the MFMAs that follow (the scheduler would
    // otherwise sink the loads next to their first use)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto load_x = [&](int c) {
#pragma unroll
    for (int j = 0; j < XPW; ++j) xst[j] = *reinterpret_cast<const bf16x8*>(xp[j] + c * SK_KX);
  };
  auto store_x = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XPW; ++j) xs[buf][wave * XPW + j][lane] = xst[j];
  };
  auto compute = [&](const bf16x8 (&w)[SK_KS][SK_RG], int buf) {
#pragma unroll
    for (int s = 0; s < SK_KS; ++s) {
      bf16x8 xf[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) xf[t] = xs[buf][s * MT + t][lane];
#pragma unroll
      for (int r = 0; r < SK_RG; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[s][r], xf[t], acc[r][t], 0, 0, 0);
    }
  };

  // Two chunks per trip (registers wb0 / wb1, LDS buffers 0 / 1); every load
  // in the loop body is unconditional so the wait before each compute only
  // covers the chunk it consumes.
  load_x(0);
  load_w(wb0, 0);
  store_x(0);
  lds_barrier();
  int c = 0;
  for (; c + 2 < nchunks; c += 2) {
    load_x(c + 1);
    load_w(wb1, c + 1);
    compute(wb0, 0);
    store_x(1);
    lds_barrier();
    load_x(c + 2);
    load_w(wb0, c + 2);
    compute(wb1, 1);
    store_x(0);
    lds_barrier();
  }
  if (nchunks - c == 2) {
    load_x(c + 1);
    load_w(wb1, c + 1);
    compute(wb0, 0);
    store_x(1);
    lds_barrier();
    compute(wb1, 1);
  } else {
    compute(wb0, 0);
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
  return M >= 1 && M <= 64 && N % 4 == 0 && K % 8 == 0 && k_split >= SK_KX && k_split % SK_KX == 0;
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
