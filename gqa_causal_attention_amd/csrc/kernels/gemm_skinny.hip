// Decode-sized bf16 "TN" GEMM (M <= 64 activation rows):
//   C[m, n] = sum_k A[m, k] * W[n, k]
// for the block's projections during single-token decode (mojolearn
// TransformerBlock: q/k/v, o_proj, gate/up, down), where every weight byte is
// used by at most 64 rows and the kernel is bound by streaming W from HBM.
//
// What bounds it is streaming W at full HBM bandwidth, and two things hold
// that back: partial-line loads, and waves waiting on each other (a
// workgroup barrier per chunk holds every wave to the slowest one's HBM
// latency).  So each wave streams its own 32 weight rows into a private ring
// of 3 LDS stages with global_load_lds_dwordx4, two chunks ahead: one
// instruction moves 4 rows x 256 bytes (a 128-deep chunk of each row, whole
// lines), XOR-swizzled on 16-byte chunks (chunk c of row r at slot
// c ^ (r % 16)) so the MFMA operand reads of 16 rows hit distinct banks.  A
// wave waits only on its own weight loads.  The activations (at most 64 rows,
// reused by every weight row) are shared: fetched the same way in B-operand
// fragment order (1 KB per 16 rows x 32 k) a 256-deep super-chunk at a time,
// double-buffered, with one barrier per super-chunk that waits only on
// activation loads issued a chunk before the weights in flight.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

constexpr int SK_KX = 128;           // k per chunk
constexpr int SK_SC = 2;             // chunks per super-chunk (one LDS activation buffer)
constexpr int SK_WST = 3;            // weight ring stages per wave (two chunks in flight)
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

// 16 bytes per lane from global memory straight into LDS at lds + 16 * lane
// (lds is wave-uniform).  The builtin only exists for the device pass.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int MT, int MODE, int EPI>
__global__ __launch_bounds__(SK_NW * 64, 1) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int RB = SK_KX * 2;                  // bytes of a row's chunk (256)
  constexpr int WROWS = SK_RG * 16;              // weight rows per wave (32)
  constexpr int W_WAVE = WROWS * RB;             // a wave's weight chunk (8 KB)
  constexpr int WI = W_WAVE / 1024;              // its load instructions per chunk (8)
  constexpr int XF = MT * SK_KS;                 // activation fragments per chunk
  constexpr int XS = SK_SC * XF;                 // per super-chunk
  constexpr int XI = XS / SK_NW;                 // fragments each wave loads per super-chunk
  static_assert(XS % SK_NW == 0, "activation fragments split evenly over the waves");
  static_assert(SK_SC == 2 && SK_WST == 3, "the wait counts below assume these depths");
  constexpr int W_RING = SK_NW * SK_WST * W_WAVE;
  __shared__ __attribute__((aligned(1024))) char smem[W_RING + 2 * XS * 1024];
  bf16x8 (*xs)[XS][64] = reinterpret_cast<bf16x8 (*)[XS][64]>(smem + W_RING);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int z = blockIdx.y;
  const int64_t kb = (int64_t)z * a.k_split;
  const int nchunks = a.k_split / SK_KX;
  const int nsc = (nchunks + SK_SC - 1) / SK_SC;
  char* ring = smem + wave * (SK_WST * W_WAVE);

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < a.bump_n; i += SK_NW * 64) a.bump[i] += a.bump_by;

  // ---- weights: load instruction jj moves the wave's rows 4jj .. 4jj+3 (lane l:
  // row 4jj + l/16, 16-byte chunk (l % 16) ^ (row % 16)) ----
  const bf16* gW[WI];
#pragma unroll
  for (int jj = 0; jj < WI; ++jj) {
    const int wr = 4 * jj + (lane >> 4);         // row within the wave's 32
    const bf16* row;
    if (MODE == kModeGated) {                    // rows 0-15 gate, 16-31 up, same 16 columns
      const int col = min(blockIdx.x * (SK_ROWS / 2) + wave * 16 + (wr & 15), a.N - 1);
      row = static_cast<const bf16*>(a.B[wr >> 4]) + (int64_t)col * a.K;
    } else {
      const int64_t n = min((int64_t)blockIdx.x * SK_ROWS + wave * WROWS + wr, (int64_t)a.N - 1);
      const int sg = seg_index(a, n);
      row = static_cast<const bf16*>(a.B[sg]) + (n - (sg == 0 ? 0 : a.seg_end[sg - 1])) * a.K;
    }
    gW[jj] = row + kb + 8 * ((lane & 15) ^ (wr & 15));
  }
  auto issue_w = [&](int c) {
    char* dst = ring + (c % SK_WST) * W_WAVE;
#pragma unroll
    for (int jj = 0; jj < WI; ++jj) load_lds16(gW[jj] + (int64_t)c * SK_KX, dst + jj * 1024);
  };
  // ---- activations: fragment f of a super-chunk (k-step f / MT, rows 16 (f % MT)
  // + (0..15), rows past M repeating row M-1) is one load instruction into a 1 KB
  // slot in B-operand order; wave w loads fragments w XI .. w XI + XI - 1 ----
  const bf16* xrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xrow[t] = static_cast<const bf16*>(a.A) + (int64_t)min(16 * t + lr, a.M - 1) * a.lda + kb + 8 * lg;
  auto issue_x = [&](int sc) {
#pragma unroll
    for (int j = 0; j < XI; ++j) {
      const int f = wave * XI + j;
      const int kstep = min(sc * SK_SC * SK_KS + f / MT, nchunks * SK_KS - 1);  // past the end: never read
      load_lds16(xrow[f % MT] + 32 * kstep, &xs[sc & 1][f][0]);
    }
  };

  f32x4 acc[SK_RG][MT];
#pragma unroll
  for (int r = 0; r < SK_RG; ++r)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // chunk c: weights from the wave's ring (row lr of each 16-row group, chunk
  // 4 ks + lg, swizzled by lr), activations from super-chunk buffer (c / 2) & 1
  auto compute = [&](int c) {
    const char* sW = ring + (c % SK_WST) * W_WAVE + lr * RB;
    const int buf = (c / SK_SC) & 1, cl = c % SK_SC;
#pragma unroll
    for (int ks = 0; ks < SK_KS; ++ks) {
      const int off = ((4 * ks + lg) ^ lr) * 16;
      bf16x8 wf[SK_RG], xf[MT];
#pragma unroll
      for (int r = 0; r < SK_RG; ++r) wf[r] = *reinterpret_cast<const bf16x8*>(sW + r * 16 * RB + off);
#pragma unroll
      for (int t = 0; t < MT; ++t) xf[t] = xs[buf][(cl * SK_KS + ks) * MT + t][lane];
#pragma unroll
      for (int r = 0; r < SK_RG; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[r], xf[t], acc[r][t], 0, 0, 0);
    }
  };

  // ---- pipeline.  Issue order: x0 w0 w1 | x1 w2 | w3 | x2 w4 | w5 | ... (iteration
  // c issues super-chunk c/2 + 1's activations when c is even, then chunk c + 2's
  // weights).  Chunk c is ready once at most the later issues are pending:
  // w(c+1), w(c+2) and x(c/2 + 1), whichever exist.  The one barrier per
  // super-chunk waits only on activations issued before w(c), i.e. on loads
  // that are normally long complete; the weight stream stays in flight. ----
  issue_x(0);
  issue_w(0);
  if (nchunks > 1) issue_w(1);
  for (int c = 0; c < nchunks; ++c) {
    if (c % SK_SC == 0) {
      // this super-chunk's activations: issued before w(c) (and w(c+1))
      if (c + 1 < nchunks) wait_vmcnt<2 * WI>();
      else wait_vmcnt<WI>();
      lds_barrier();  // published; and every wave is done with the other buffer
      if (c / SK_SC + 1 < nsc) issue_x(c / SK_SC + 1);
    }
    if (c + 2 < nchunks) issue_w(c + 2);  // into the slot chunk c - 1 used
    // chunk c's weights
    const int later = (c + 1 < nchunks ? WI : 0) + (c + 2 < nchunks ? WI : 0) + (c / SK_SC + 1 < nsc ? XI : 0);
    if (later == 2 * WI + XI) wait_vmcnt<2 * WI + XI>();
    else if (later == 2 * WI) wait_vmcnt<2 * WI>();
    else if (later == WI + XI) wait_vmcnt<WI + XI>();
    else if (later == WI) wait_vmcnt<WI>();
    else if (later == XI) wait_vmcnt<XI>();
    else wait_vmcnt<0>();
    compute(c);
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
