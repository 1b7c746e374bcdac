// bf16 "TN" GEMM for prefill-sized M on gfx950 matrix cores:
//   C[m, n] = sum_k A[m, k] * W[n, k]
// A = activations [M, K], W = a Hugging Face [out, in] weight (mojolearn
// TransformerBlock weight table: q/k/v, o_proj, gate/up, down), both
// K-contiguous.  Same epilogues as the register-staged kernel (q/k/v segments
// + bias, residual add, act(gate) * up, split-K partials).
//
// Tiles stream from global memory straight into LDS with
// global_load_lds_dwordx4 (no register round trip, no LDS write
// instructions), through a ring of ST stages of BK-deep k-slices.  One
// barrier per slice, placed after the last fragment reads of slice kt and
// before that k-step's MFMAs: it publishes slice kt + 1 (every wave has waited
// for its own loads of it) and frees slice kt's stage, which is refilled with
// slice kt + ST; the MFMAs of the last k-step then overlap the first
// fragment reads of slice kt + 1.  The refill's load instructions are spread
// over that k-step, one group after the first MFMA of each row of MFMAs,
// rather than issued in one burst: a wave issues in order, and while the L1's
// queue of outstanding L2 requests is full (misses to the Infinity Cache or
// HBM hold their entries for hundreds of cycles) a burst of loads keeps the
// wave -- and, with every wave released by the same barrier, the SIMD -- from
// issuing MFMAs (measured on the 4k-token prefill: gate/up 0.83 -> 0.78 ms;
// spreading them over two k-steps leaves the later loads too little time to
// land and is slower than the burst).
//
// A load instruction writes 64 lanes x 16 bytes contiguously into LDS, so the
// LDS layout is chosen through the global address each lane reads: lane l of
// load instruction i fetches row i * RPI + l / CPR (CPR = 16-byte chunks per
// row), chunk (l % CPR) ^ swz(row).  Each instruction therefore reads whole
// rows (full cache lines), and an MFMA fragment read (32 consecutive rows, one
// chunk) hits 16 distinct 16-byte bank groups in every 16-lane phase: the XOR
// key swz(row) = (row / RP) % CPR, with RP rows per 256 bytes of LDS, gives
// each of 16 consecutive rows its own (row % RP, slot) pair.
//
// Each wave owns a (BM/WGM) x (BN/WGN) sub-tile of 32x32 accumulators fed by
// v_mfma_f32_32x32x16_bf16; fragment registers are double-buffered across the
// 16-deep k-steps of a slice.
//
// Transposed operands (TR bit 0: A, bit 1: B; 256-wide tiles, 16x16x32 MFMA):
// the operand is stored K-major, X^T[k][x] (a weight [out, in] read as the
// product's right operand along `out`, or activations [tokens, features] read
// along the token axis), so the backward's products need no transposed copies.
// Its slice is staged as BK rows of 256 consecutive x (512 bytes; a load
// instruction moves two rows), XOR-swizzled on 16-byte chunks with a key of
// the row, and the MFMA operand (8 consecutive k of one x per lane) comes from
// two transposing reads ds_read_b64_tr_b16 (within a 16-lane group lane i
// receives element i % 4 of the 8-byte pieces addressed by lanes 4e + i / 4,
// e = 0..3, i.e. 4 consecutive k of one x).  Those reads are issued through
// inline asm (the builtin makes the compiler wait for every outstanding global
// load first, the next slice's direct-to-LDS loads included), and their
// results are waited for explicitly with counts derived from the fixed issue
// order below.
#include "common.h"
#include "launch.h"

namespace gqa {
namespace {

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
  // s_waitcnt: vmcnt = N (bits 3:0 and 15:14), expcnt 7 and lgkmcnt 15 = no wait
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `later` slices (NLD loads each) of this wave are pending.
template <int NLD, int L>
__device__ __forceinline__ void wait_slices(int later) {
  if constexpr (L <= 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= L) wait_vmcnt<L * NLD>();
    else wait_slices<NLD, L - 1>(later);
  }
}

// Workgroup barrier that orders LDS accesses only: this wave's LDS reads are
// complete (lgkmcnt 0) and the caller has waited (vmcnt) for the slices it
// publishes.  No memory fence: a workgroup-scope release fence also covers the
// direct-to-LDS loads still in flight and would wait for all of them
// (vmcnt 0), which would cut a ring deeper than two stages to one slice of
// lookahead.  The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0) only
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int seg_of(const GemmArgs& a, int64_t n) {
  return n < a.seg_end[0] ? 0 : (n < a.seg_end[1] ? 1 : 2);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
// ds_read_b64_tr_b16 at LDS byte address addr + OFF.  The result is not
// tracked by the compiler's wait-count insertion: wait (lgkm_wait) and tie()
// it before use.
template <int OFF>
__device__ __forceinline__ s16x4 lds_read_tr16_at(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset is 16 bits");
  s16x4 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
// Wait until at most N LDS / scalar-memory operations of this wave are
// outstanding (LDS operations complete in issue order).
template <int N>
__device__ __forceinline__ void lgkm_wait() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// Makes v look redefined here, so its uses stay behind a preceding lgkm_wait.
__device__ __forceinline__ void tie(bf16x8& v) { asm volatile("" : "+v"(v)); }

// XOR key (in 16-byte chunks) of k-row r of a transposed slice: rows r and
// r + 1..3, r + 8 land in different 32-byte slots of 256 bytes.
__device__ __forceinline__ int tkey(int r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); }

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<I + 1, N>(f);
  }
}


// Global row pointer of B-tile row r (K offset k0) for tile column tn.  Gated
// mode: each wave's WTN B rows are WTN/2 gate rows then the WTN/2 up rows of
// the same output columns, so one lane holds both accumulators of a column.
template <int MODE, int BN, int WTN>
__device__ __forceinline__ const bf16* b_row_ptr(const GemmArgs& a, int tn, int r, int64_t k0) {
  if (MODE == kModeGated) {
    const int blk = r / WTN, w = r % WTN;
    int col = tn * (BN / 2) + blk * (WTN / 2) + (w % (WTN / 2));
    col = min(col, a.N - 1);
    const bf16* base = static_cast<const bf16*>(w < WTN / 2 ? a.B[0] : a.B[1]);
    return base + (int64_t)col * a.K + k0;
  } else {
    const int64_t n = min((int64_t)tn * BN + r, (int64_t)a.N - 1);
    const int s = seg_of(a, n);
    const int64_t start = s == 0 ? 0 : a.seg_end[s - 1];
    return static_cast<const bf16*>(a.B[s]) + (n - start) * a.K + k0;
  }
}

// MFMA shapes: MF = 32 -> v_mfma_f32_32x32x16_bf16 (16 accumulators per lane),
// MF = 16 -> v_mfma_f32_16x16x32_bf16 (4 per lane).  The A/B operand of lane l
// is 8 consecutive k of row l % MF, at k offset 8 * (l / MF) within the step.
template <int MF> struct Mfma;
template <> struct Mfma<32> {
  typedef f32x16 acc_t;
  static constexpr int KD = 16;  // k per instruction
  __device__ static acc_t run(bf16x8 a, bf16x8 b, acc_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }
  // accumulator element e of lane l: row (e / 4) * 8 + (l / 32) * 4 + e % 4, column l % 32
  __device__ static int row(int e, int lane) { return (e / 4) * 8 + (lane >> 5) * 4 + (e % 4); }
};
template <> struct Mfma<16> {
  typedef f32x4 acc_t;
  static constexpr int KD = 32;
  __device__ static acc_t run(bf16x8 a, bf16x8 b, acc_t c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }
  // accumulator element e of lane l: row (l / 16) * 4 + e, column l % 16
  __device__ static int row(int e, int lane) { return (lane >> 4) * 4 + e; }
};

// SCHED 0: fragments double-buffered, two reads of the next k-step after each
//          of the first MFMAs of a step;
// SCHED 1: B fragments double-buffered (read one or two per A row), each A
//          fragment re-read for the next k-step as soon as its row of MFMAs
//          has issued (fewer live registers, reads spread over the step).
template <int BM, int BN, int BK, int ST, int WGM, int WGN, int MF, int SCHED, int MODE, int EPI, int TR>
__global__ __launch_bounds__(WGM* WGN * 64, 1) void gemm_dma_kernel(GemmArgs a) {
  typedef Mfma<MF> MM;
  typedef typename MM::acc_t acc_t;
  constexpr int NACC = sizeof(acc_t) / sizeof(float);
  constexpr int NW = WGM * WGN, NT = NW * 64;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int CPR = BK / 8;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;          // rows per load instruction
  constexpr int RP = 128 / BK;           // rows per 256 bytes of LDS
  constexpr bool TA = (TR & 1) != 0, TB = (TR & 2) != 0;
  constexpr int RBA = BM * 2, RBB = BN * 2;         // bytes per k-row of a transposed slice
  constexpr int TPR = 1024 / RBA;                   // k-rows per load instruction (transposed)
  // load instructions per wave per slice
  constexpr int IA = TA ? BK / TPR / NW : BM / RPI / NW, IB = TB ? BK / TPR / NW : BN / RPI / NW;
  constexpr int NLD = IA + IB;
  constexpr int A_BYTES = BM * BK * 2, STAGE_BYTES = (BM + BN) * BK * 2;
  constexpr int KS = BK / MM::KD;        // MFMA k-steps per slice
  constexpr int CPF = MM::KD / 8;        // 16-byte chunks per fragment row per k-step
  constexpr int BPR = (FN + FM - 1) / FM;  // SCHED 1: B reads per A row
  static_assert(BK == 32 || BK == 64 || BK == 128, "slice depth");
  static_assert(RP * CPR == 16, "swizzle period is 16 rows");
  static_assert((BM / RPI) % NW == 0 && (BN / RPI) % NW == 0, "load instructions split evenly over waves");
  static_assert(WTM % MF == 0 && WTN % MF == 0, "wave tile must be a multiple of the MFMA size");
  static_assert(MODE != kModeGated || FN % 2 == 0, "gated wave tiles hold gate and up halves");
  static_assert(ST >= 2 && ST <= 6 && (ST - 1) * NLD < 64, "pipeline depth");
  static_assert(KS % 2 == 0 || SCHED == 1, "fragment slots alternate across slices");
  static_assert(TR == 0 || (MF == 16 && SCHED == 1 && MODE == kModeSeg && BM == 256 && BN == 256 && BK == 64 &&
                            (BK / TPR) % NW == 0),
                "transposed operands: 256x256 tiles, 64-deep slices, 16x16x32 MFMA, A re-read schedule");
  __shared__ __attribute__((aligned(1024))) char smem[ST * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;

  if (a.bump && blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.bump_n; i += NT) a.bump[i] += a.bump_by;

  // ---- tile order (order 0, the default): consecutive workgroup ids go
  // round-robin to the 8 XCDs, so give each XCD a contiguous run of the tile
  // order, then walk groups of GM M-tiles across N so tiles running together
  // on an XCD share A and B panels in its L2.  Orders 1 (row-major, no remap)
  // and 2 (groups of 4, no XCD remap) are kept for tuning. ----
  const int cols_per_tile = MODE == kModeGated ? BN / 2 : BN;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = (a.N + cols_per_tile - 1) / cols_per_tile;
  const int total = gridDim.x;
  int pid = blockIdx.x, tm, tn;
  if (a.order == 1) {
    tm = pid / tiles_n;
    tn = pid % tiles_n;
  } else {
    if (a.order == 0 && total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
    const int GM = a.order == 3 ? 8 : 4;
    const int group = pid / (GM * tiles_n);
    const int first_m = group * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int rem = pid % (GM * tiles_n);
    tm = first_m + rem % gsize;
    tn = rem / gsize;
  }
  const int m0 = tm * BM;

  const int64_t kbeg = (int64_t)blockIdx.y * a.k_split;
  const int nk = (int)((min((int64_t)a.K, kbeg + a.k_split) - kbeg) / BK);

  // ---- this lane's global source of every load instruction it issues ----
  // (transposed: lane l of instruction i fetches k-row i * TPR + l / 32, 16-byte
  // chunk (l % 32) ^ tkey(row); columns past M or N clamp to the last whole
  // chunk, whose products land in discarded outputs)
  const int lrow = lane / CPR, lslot = lane % CPR;
  const int trw = lane / (64 / TPR), tsl = lane % (64 / TPR);
  const bf16* gA[IA];
  const bf16* gB[IB];
  {
    const bf16* A = static_cast<const bf16*>(a.A);
#pragma unroll
    for (int j = 0; j < IA; ++j) {
      if constexpr (TA) {
        const int r = (wave + NW * j) * TPR + trw;
        const int m = min(m0 + (tsl ^ tkey(r)) * 8, a.M - 8);
        gA[j] = A + (kbeg + r) * a.lda + m;
      } else {
        const int r = (wave + NW * j) * RPI + lrow;
        const int chunk = lslot ^ ((r / RP) % CPR);
        const int m = min(m0 + r, a.M - 1);
        gA[j] = A + (int64_t)m * a.lda + kbeg + chunk * 8;
      }
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      if constexpr (TB) {
        gB[j] = nullptr;  // per slice, from the K segment (issue)
      } else {
        const int r = (wave + NW * j) * RPI + lrow;
        const int chunk = lslot ^ ((r / RP) % CPR);
        gB[j] = b_row_ptr<MODE, BN, WTN>(a, tn, r, kbeg) + chunk * 8;
      }
    }
  }
  // The segment table as the first entry plus increments: a choice between
  // two captured values becomes a data-dependent offset into the lambda's
  // captures, which keeps every captured variable in scratch memory; adding
  // an increment or zero does not.
  const uint64_t tb_u0 = (uint64_t)(uintptr_t)a.B[0];
  const uint64_t tb_d1 = (uint64_t)(uintptr_t)a.B[1] - tb_u0, tb_d2 = (uint64_t)(uintptr_t)a.B[2] - (uint64_t)(uintptr_t)a.B[1];
  const int64_t tb_e0 = a.seg_end[0], tb_g1 = a.seg_end[1] - a.seg_end[0], tb_g2 = a.seg_end[2] - a.seg_end[1];
  auto issue = [&](int kt, int stage) __attribute__((always_inline)) {
    char* sA = smem + stage * STAGE_BYTES;
    char* sB = sA + A_BYTES;
    const int64_t kk = kbeg + (int64_t)kt * BK;
#pragma unroll
    for (int j = 0; j < IA; ++j)
      load_lds16(gA[j] + (TA ? kk - kbeg : 0) * a.lda + (TA ? 0 : (int64_t)kt * BK), sA + (wave + NW * j) * 1024);
    if constexpr (TB) {
      // B^T rows come from up to three segments along K (slice-aligned
      // boundaries); rows past the last one (K padding) repeat it
      const int64_t e1 = tb_e0 + tb_g1, e2 = e1 + tb_g2;
      const int64_t kq = min(kk, e2 - 1);
      const bool past0 = kq >= tb_e0, past1 = kq >= e1;
      const int64_t start = (past0 ? tb_e0 : 0) + (past1 ? tb_g1 : 0);
      const int64_t avail = tb_e0 + (past0 ? tb_g1 : 0) + (past1 ? tb_g2 : 0) - kk;  // rows of the slice in the segment
      const uint64_t base = tb_u0 + (past0 ? tb_d1 : 0) + (past1 ? tb_d2 : 0);
      const bf16* Bs = reinterpret_cast<const bf16*>((uintptr_t)base) + (kk - start) * a.ldb;
      const int last = (int)min(avail, (int64_t)BK) - 1;
#pragma unroll
      for (int j = 0; j < IB; ++j) {
        const int r = (wave + NW * j) * TPR + trw;
        const int col = min(tn * BN + (tsl ^ tkey(r)) * 8, a.N - 8);
        load_lds16(Bs + (min(r, last) * (int)a.ldb + col), sB + (wave + NW * j) * 1024);
      }
    } else {
#pragma unroll
      for (int j = 0; j < IB; ++j)
        load_lds16(gB[j] + (int64_t)kt * BK, sB + (wave + NW * j) * 1024);
    }
  };

  // Load instruction j of slice kt into `stage` (A's first), for the spread
  // refill (non-transposed operands, A re-read schedule): LPR per row of MFMAs.
  constexpr bool SPREAD = TR == 0 && SCHED == 1;
  constexpr int LPR = (NLD + FM - 1) / FM;
  auto issue_one = [&](int kt, int stage, int j) __attribute__((always_inline)) {
    char* sA = smem + stage * STAGE_BYTES;
    char* sB = sA + A_BYTES;
    if (j < IA) load_lds16(gA[j] + (int64_t)kt * BK, sA + (wave + NW * j) * 1024);
    else load_lds16(gB[j - IA] + (int64_t)kt * BK, sB + (wave + NW * (j - IA)) * 1024);
  };

  // ---- fragment addressing: row lane % MF of an MF-row block, chunk CPF ks + lane / MF ----
  // (MF-row blocks start at multiples of 16 rows, so the XOR key is a function of lane % MF)
  const int frow = lane % MF, fhi = lane / MF;
  const int fsw = (frow / RP) % CPR;
  const int a_off = (wm * WTM + frow) * (BK * 2);
  const int b_off = A_BYTES + (wn * WTN + frow) * (BK * 2);
  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = ((CPF * ks + fhi) ^ fsw) * 16;
  // transposed fragments (16x16x32): lane l of group g = l / 16, j = l % 16
  // addresses k-row 8 g + j / 4 (+ 4 for the second read) and the 8 bytes of
  // columns xb + 4 (j % 4) .. + 3 of its 16-column block xb
  const int tg = lane >> 4, tj = lane & 15;
  const int tkl = 2 * ((tj >> 2) + 4 * (tg & 1));  // = tkey of every row this lane reads
  const int trow = 8 * tg + (tj >> 2);
  uint32_t ta_off[TA ? FM : 1], tb_off[TB ? FN : 1];
#pragma unroll
  for (int i = 0; i < (TA ? FM : 0); ++i) {
    const int xb = wm * WTM + i * 16;
    ta_off[i] = trow * RBA + ((((xb >> 3) ^ tkl) | ((tj & 3) >> 1)) * 16) + (tj & 1) * 8;
  }
#pragma unroll
  for (int j = 0; j < (TB ? FN : 0); ++j) {
    const int xb = wn * WTN + j * 16;
    tb_off[j] = A_BYTES + trow * RBB + ((((xb >> 3) ^ tkl) | ((tj & 3) >> 1)) * 16) + (tj & 1) * 8;
  }
  const uint32_t smem_lds = lds_addr(smem);

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < NACC; ++e) acc[i][j][e] = 0.f;

  // Fragment registers: see SCHED.  `cur` is the slot the MFMAs of a k-step
  // read; the reads of the next k-step (possibly of the next slice) go to the
  // other slot (SCHED 0) or, for A under SCHED 1, to slot 0 after its row.
  bf16x8 fa[2][FM], fb[2][FN];
  auto rd_tr = [&](uint32_t ad, auto ks_c, int rb) __attribute__((always_inline)) {
    constexpr int KSN = decltype(ks_c)::value;
    s16x4 lo, hi;
    if (rb == RBA) {
      lo = lds_read_tr16_at<KSN * 32 * RBA>(ad);
      hi = lds_read_tr16_at<KSN * 32 * RBA + 4 * RBA>(ad);
    } else {
      lo = lds_read_tr16_at<KSN * 32 * RBB>(ad);
      hi = lds_read_tr16_at<KSN * 32 * RBB + 4 * RBB>(ad);
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto rd = [&](int stage, auto ks_c, int slot, int r) __attribute__((always_inline)) {
    constexpr int KSN = decltype(ks_c)::value;
    const char* s = smem + stage * STAGE_BYTES + koff[KSN];
    if (r < FM) {
      if constexpr (TA) fa[slot][r] = rd_tr(smem_lds + stage * STAGE_BYTES + ta_off[r], ks_c, RBA);
      else fa[slot][r] = *reinterpret_cast<const bf16x8*>(s + a_off + r * MF * (BK * 2));
    } else {
      if constexpr (TB) fb[slot][r - FM] = rd_tr(smem_lds + stage * STAGE_BYTES + tb_off[r - FM], ks_c, RBB);
      else fb[slot][r - FM] = *reinterpret_cast<const bf16x8*>(s + b_off + (r - FM) * MF * (BK * 2));
    }
  };
  // Waits for the asm reads (TR != 0), from the issue order of a step (A
  // re-read schedule): row r issues its MFMAs, after the first one the next
  // step's B fragment r (r < FN), and after the row the next step's A
  // fragment r; a fragment read takes NA / NB instructions.  A fragment r is
  // therefore followed by P - ops(r) instructions when row r of the next
  // step starts, and the last B fragment by NA * (FM - FN + 1) when row 0
  // starts.  (After the prologue and after each barrier nothing is pending.)
  constexpr int NA = TA ? 2 : 1, NB = TB ? 2 : 1;
  constexpr int P_OPS = FM * NA + (FN < FM ? FN : FM) * NB;
  auto row_wait = [&](auto i_c) {
    constexpr int I = decltype(i_c)::value;
    constexpr int OPS_I = NA + (I < FN ? NB : 0);
    constexpr int NW_A = TA ? P_OPS - OPS_I : 64;
    constexpr int NW_B = (TB && I == 0) ? NA * (FM - FN + 1) : 64;
    constexpr int NWT = NW_A < NW_B ? NW_A : NW_B;
    if constexpr (NWT < 64) lgkm_wait<(NWT < 15 ? NWT : 15)>();
  };
  // ldkt >= 0: spread the loads of slice ldkt into stage ldstage over this step
  auto step = [&](int cur, int stage, auto ks, int ldkt = -1, int ldstage = 0) __attribute__((always_inline)) {
    if constexpr (SCHED == 1) {
      static_for<0, FM>([&](auto i_c) {
        constexpr int i = decltype(i_c)::value;
        if constexpr (TR != 0) {
          row_wait(i_c);
          if constexpr (TA) tie(fa[0][i]);
          if constexpr (TB && i == 0) {
#pragma unroll
            for (int j = 0; j < FN; ++j) tie(fb[cur][j]);
          }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          acc[i][j] = MM::run(fa[0][i], fb[cur][j], acc[i][j]);
          if (j < BPR && i * BPR + j < FN) rd(stage, ks, cur ^ 1, FM + i * BPR + j);
          if constexpr (SPREAD) {
            if (j == 0 && ldkt >= 0) {
#pragma unroll
              for (int q = i * LPR; q < (i + 1) * LPR && q < NLD; ++q) issue_one(ldkt, ldstage, q);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        rd(stage, ks, 0, i);
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
#pragma unroll
      for (int t = 0; t < FM * FN; ++t) {
        acc[t / FN][t % FN] = MM::run(fa[cur][t / FN], fb[cur][t % FN], acc[t / FN][t % FN]);
#pragma unroll
        for (int r = 2 * t; r < 2 * t + 2; ++r)
          if (r < FM + FN) rd(stage, ks, cur ^ 1, r);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- pipeline: all ST stages in flight from the start; a stage is refilled
  // (ST slices ahead) as soon as every wave has read its last fragments ----
#pragma unroll
  for (int s = 0; s < ST; ++s)
    if (s < nk) issue(s, s);
  if (nk > 0) {
    wait_slices<NLD, ST - 1>(min(ST - 1, nk - 1));
    lds_sync();
#pragma unroll
    for (int r = 0; r < FM + FN; ++r) rd(0, IntC<0>{}, 0, r);
    if constexpr (TR != 0) lgkm_wait<0>();
  }
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt % ST;
    static_for<0, KS - 1>([&](auto ks_c) {
      constexpr int ks = decltype(ks_c)::value;
      step(ks & 1, stage, IntC<ks + 1>{});
    });
    if (kt + 1 < nk) {
      // slice kt + 1 has landed once at most min(ST - 2, nk - 2 - kt) later slices are pending
      wait_slices<NLD, ST - 2>(min(ST - 2, nk - 2 - kt));
      if constexpr (TR != 0) lgkm_wait<0>();
      lds_sync();  // publishes slice kt + 1; every wave is done reading stage `stage`
      if (!SPREAD && kt + ST < nk) issue(kt + ST, stage);
    }
    // (after the last slice these reads fetch an unused stage: harmless, and it
    // keeps a single copy of the MFMA sequence in the loop)
    step((KS - 1) & 1, (kt + 1) % ST, IntC<0>{}, (SPREAD && kt + ST < nk) ? kt + ST : -1, stage);
  }
  if constexpr (TR != 0) lgkm_wait<0>();  // the last step's reads, before LDS is reused

  // The activation (gated and store epilogues) and the presence of gate/up
  // biases are resolved once here, so each epilogue loop below is compiled
  // for one activation with no per-element branch.
  const bool gbias = EPI == kEpiGated && (a.bias[0] || a.bias[1]);
  auto epilogue = [&](auto act_c, auto bias_c) {
    constexpr int ACT = decltype(act_c)::value;
    constexpr bool GBIAS = decltype(bias_c)::value != 0;
    // gate / up values of output column n (biases added when present)
    auto gated = [&](float g, float u, int n) {
      if constexpr (GBIAS) {
        if (a.bias[0]) g += a.bias[0][n];
        if (a.bias[1]) u += a.bias[1][n];
      }
      return act_t<ACT>(g) * u;
    };
  // ---- epilogue through LDS (16x16 MFMA; residual and q/k/v epilogues): 64
  // rows at a time the owning waves write their accumulators into a float32
  // staging tile, then all threads read it back row-major and apply the
  // epilogue with 16-byte loads and stores, whole rows per wave.  (The gated
  // gate/up epilogue stays direct: its tiles are many per CU, so their
  // stores overlap other tiles' main loops, and measured slower staged.)
  // A pass's global operands (residual and bias, the backward's gate / up
  // pre-activations) are all loaded before its staging writes: the output may
  // alias them, so loads interleaved with the stores would each wait for the
  // previous piece's round trip (one HBM latency per piece, every CU at once
  // on the shapes with one tile per CU).  The barriers order LDS only, so
  // the loads and the previous pass's stores stay in flight across them. ----
  if constexpr (MF == 16 && (EPI == kEpiResid || EPI == kEpiStore || EPI == kEpiSwigluBwd)) {
    constexpr int COLS = MODE == kModeGated ? BN / 2 : BN;  // output columns of the tile
    constexpr int SW = COLS + 4;                            // staging row stride (floats): 4 rows per
                                                            // write land 16 banks apart
    constexpr int PR = 64;                                  // rows per pass
    constexpr int PIT = PR * (COLS / 4) / NT;               // 16-byte pieces per thread per pass
    static_assert(PR * SW * 4 <= ST * STAGE_BYTES, "staging tile fits in the pipeline's LDS");
    static_assert(COLS % 4 == 0 && WTM % PR == 0 || PR % WTM == 0, "pass rows cover whole wave rows");
    static_assert(PR * (COLS / 4) % NT == 0, "a pass's pieces split evenly over the threads");
    constexpr bool GU = EPI == kEpiSwigluBwd, PRE = EPI != kEpiStore;  // PRE: operands loaded up front
    float* stg = reinterpret_cast<float*>(smem);
    const int col0 = tn * COLS;
    // A store-epilogue tile wholly inside the output skips the bounds tests,
    // addresses its pieces from a per-pass (wave-uniform) base with 32-bit
    // offsets, and takes each piece's biases (segment lookups included) from
    // registers filled once: a thread's columns are the same in every pass.
    const bool full = EPI == kEpiStore && m0 + BM <= a.M && col0 + COLS <= a.N && a.ldc <= (int64_t)1 << 24;  // (r * ldc + c < 2^31)
    // piece it of this thread: row r (within the pass), columns c .. c + 3
    auto piece = [&](int it, int& r, int& c) {
      const int idx = tid + it * NT;
      r = idx / (COLS / 4);
      c = (idx % (COLS / 4)) * 4;
    };
    f32x4 sbias[EPI == kEpiStore ? PIT : 1];
    if constexpr (EPI == kEpiStore) {
#pragma unroll
      for (int it = 0; it < PIT; ++it) sbias[it] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (full && (a.bias[0] || a.bias[1] || a.bias[2])) {
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
          int r, c;
          piece(it, r, c);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int n = col0 + c + e;
            const int sg = seg_of(a, n);
            sbias[it][e] = a.bias[sg] ? a.bias[sg][n - (sg == 0 ? 0 : a.seg_end[sg - 1])] : 0.f;
          }
        }
      }
    }
#pragma unroll 1
    for (int pass = 0; pass < BM / PR; ++pass) {
      // residual and bias (added when the piece is stored, so neither load
      // waits for the other) / gate and up
      f32x4 g0[PRE ? PIT : 1], g1[PRE ? PIT : 1];
      const int64_t prow = m0 + pass * PR;  // first row of the pass
#pragma unroll
      for (int it = 0; it < (PRE ? PIT : 0); ++it) {
        int r, c;
        piece(it, r, c);
        const int m = m0 + pass * PR + r, n = col0 + c;
        g0[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        g1[it] = g0[it];
        if (m >= a.M || n >= a.N) continue;
        if constexpr (GU) {
          const float* gu = a.resid + (int64_t)m * a.ldr + n;
          g0[it] = *reinterpret_cast<const f32x4*>(gu);
          g1[it] = *reinterpret_cast<const f32x4*>(gu + a.N);
        } else {
          if (a.resid) g0[it] = *reinterpret_cast<const f32x4*>(a.resid + (int64_t)m * a.ldr + n);
          if (a.bias[0]) g1[it] = *reinterpret_cast<const f32x4*>(a.bias[0] + n);
        }
      }
      lds_sync();  // the previous pass's staging reads (or the main loop's fragment reads) are done
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int rb = wm * WTM + i * 16;  // first tile row of block i
        if (rb / PR != pass) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = rb - pass * PR + MM::row(e, lane);
          if constexpr (MODE == kModeGated) {
#pragma unroll
            for (int jj = 0; jj < FN / 2; ++jj) {
              const int n = min(col0 + wn * (WTN / 2) + jj * 16 + (lane & 15), a.N - 1);
              stg[r * SW + wn * (WTN / 2) + jj * 16 + (lane & 15)] = gated(acc[i][jj][e], acc[i][jj + FN / 2][e], n);
            }
          } else {
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) stg[r * SW + wn * WTN + jj * 16 + (lane & 15)] = acc[i][jj][e];
          }
        }
      }
      lds_sync();
      if constexpr (PRE) {
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
          int r, c;
          piece(it, r, c);
          const int m = m0 + pass * PR + r, n = col0 + c;
          if (m >= a.M || n >= a.N) continue;
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + r * SW + c);
          if constexpr (GU) {
            // v = da; g0 / g1 the recomputed gate / up pre-activations of the same columns
            bf16x4 ov, og, ou;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float g = g0[it][e], u = g1[it][e];
              const float sg = sigmoid(g);
              const float sl = g * sg;
              ov[e] = from_f32<bf16>(sl * u);
              og[e] = from_f32<bf16>(v[e] * u * sg * (1.0f + g * (1.0f - sg)));
              ou[e] = from_f32<bf16>(v[e] * sl);
            }
            bf16* c2 = static_cast<bf16*>(a.C2) + (int64_t)m * a.ldc2 + n;
            *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + n) = ov;
            *reinterpret_cast<bf16x4*>(c2) = og;
            *reinterpret_cast<bf16x4*>(c2 + a.N) = ou;
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(a.C) + (int64_t)m * a.ldc + n) = g0[it] + (v + g1[it]);
          }
        }
      } else if (full) {  // kEpiStore, whole tile
        bf16* cb = static_cast<bf16*>(a.C) + prow * a.ldc + col0;
#pragma unroll
        for (int it = 0; it < PIT; ++it) {
          int r, c;
          piece(it, r, c);
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + r * SW + c);
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = from_f32<bf16>(act_t<ACT>(v[e] + sbias[EPI == kEpiStore ? it : 0][e]));
          *reinterpret_cast<bf16x4*>(cb + (uint32_t)(r * (int)a.ldc + c)) = o;
        }
      } else {  // kEpiStore (+ segment bias, act): no residual, the bias reads are L2 hits
        for (int idx = tid; idx < PR * (COLS / 4); idx += NT) {
          const int r = idx / (COLS / 4), c = (idx % (COLS / 4)) * 4;
          const int m = m0 + pass * PR + r, n = col0 + c;
          if (m >= a.M || n >= a.N) continue;
          const f32x4 v = *reinterpret_cast<const f32x4*>(stg + r * SW + c);
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int sg = seg_of(a, n + e);
            const float b = a.bias[sg] ? a.bias[sg][n + e - (sg == 0 ? 0 : a.seg_end[sg - 1])] : 0.f;
            o[e] = from_f32<bf16>(act_t<ACT>(v[e] + b));
          }
          *reinterpret_cast<bf16x4*>(static_cast<bf16*>(a.C) + (int64_t)m * a.ldc + n) = o;
        }
      }
    }
    return;
  }

  // ---- direct epilogue: accumulator element e of block (i, j) is row i * MF + MM::row(e, lane),
  // B row / column j * MF + lane % MF of the wave tile ----
  const int lcol = lane % MF;
  // gate / up biases of this lane's columns, loaded once (the output stores
  // below would otherwise keep the compiler from hoisting them)
  float bgv[FN / 2], buv[FN / 2];
  if constexpr (EPI == kEpiGated && GBIAS) {
#pragma unroll
    for (int j = 0; j < FN / 2; ++j) {
      const int n = min(tn * (BN / 2) + wn * (WTN / 2) + j * MF + lcol, a.N - 1);
      bgv[j] = a.bias[0] ? a.bias[0][n] : 0.f;
      buv[j] = a.bias[1] ? a.bias[1][n] : 0.f;
    }
  }
  if constexpr (EPI == kEpiGated && MF == 16) {
    // A tile wholly inside the output (every gate/up tile at the 8B shapes)
    // stores without bounds tests: the row base is wave-uniform (scalar
    // registers), the lane's offset one 32-bit register, and the column
    // blocks immediate offsets -- with the tests, every 2-byte store sat in
    // its own masked block behind a 64-bit address computation.
    if (m0 + BM <= a.M && tn * (BN / 2) + BN / 2 <= a.N && a.ldc <= (int64_t)1 << 28) {  // (32-bit lane offsets)
      const int wu = __builtin_amdgcn_readfirstlane(wave);
      const int64_t ldc = a.ldc;
      const bf16* base = static_cast<const bf16*>(a.C) + (int64_t)(m0 + (wu / WGN) * WTM) * ldc + tn * (BN / 2) +
                         (wu % WGN) * (WTN / 2);
      const uint32_t loff = (uint32_t)((lane >> 4) * 4) * (uint32_t)ldc + (uint32_t)lcol;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16* row = const_cast<bf16*>(base) + (int64_t)(i * MF + e) * ldc;
#pragma unroll
          for (int j = 0; j < FN / 2; ++j) {
            float g = acc[i][j][e], u = acc[i][j + FN / 2][e];
            if constexpr (GBIAS) {
              g += bgv[j];
              u += buv[j];
            }
            row[loff + j * MF] = from_f32<bf16>(act_t<ACT>(g) * u);
          }
        }
      }
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int e = 0; e < NACC; ++e) {
      const int m = m0 + wm * WTM + i * MF + MM::row(e, lane);
      if (m >= a.M) continue;
      if constexpr (EPI == kEpiGated) {
#pragma unroll
        for (int j = 0; j < FN / 2; ++j) {
          const int n = tn * (BN / 2) + wn * (WTN / 2) + j * MF + lcol;
          float g = acc[i][j][e], u = acc[i][j + FN / 2][e];
          if constexpr (GBIAS) {
            g += bgv[j];
            u += buv[j];
          }
          if (n < a.N) static_cast<bf16*>(a.C)[(int64_t)m * a.ldc + n] = from_f32<bf16>(act_t<ACT>(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int cb = wn * WTN + j * MF + lcol;  // B row within the tile
          const float v = acc[i][j][e];
          if (EPI == kEpiPartial) {
            int64_t nb, NB;
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
              static_cast<bf16*>(a.C)[(int64_t)m * a.ldc + n] = from_f32<bf16>(act_t<ACT>(v + b));
            }
          }
        }
      }
    }
  }
  };
  if constexpr (EPI == kEpiGated || EPI == kEpiStore) {
    with_act(a.act, [&](auto act_c) {
      if (gbias)
        epilogue(act_c, IntC<1>{});
      else
        epilogue(act_c, IntC<0>{});
    });
  } else {
    epilogue(IntC<kActNone>{}, IntC<0>{});
  }
}

template <int BM, int BN, int BK, int ST, int WGM, int WGN, int MF, int SCHED, int MODE, int EPI, int TR = 0>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t s) {
  if (a.k_split % BK != 0) return hipErrorInvalidValue;
  const int cols = MODE == kModeGated ? BN / 2 : BN;
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + cols - 1) / cols);
  hipLaunchKernelGGL((gemm_dma_kernel<BM, BN, BK, ST, WGM, WGN, MF, SCHED, MODE, EPI, TR>), dim3(tiles, a.splits),
                     dim3(WGM * WGN * 64), 0, s, a);
  return hipGetLastError();
}

// Transposed operands: 256x256 tiles only.  Whole 16-byte chunks of the
// stored K-major rows (M for a transposed A, N for a transposed B: multiples
// of 8, at least 8), 16-byte aligned rows, B's K segments ending on slice
// boundaries except the last.
template <int EPI>
hipError_t launch_trans(const GemmArgs& a, hipStream_t s) {
  const bool ta = (a.trans & 1) != 0, tb = (a.trans & 2) != 0;
  if (a.M < 1 || a.lda % 8 != 0 || (uintptr_t)a.A % 16 != 0) return hipErrorInvalidValue;
  if (ta && (a.M < 8 || a.M % 8 != 0)) return hipErrorInvalidValue;
  if (tb && (a.N < 8 || a.N % 8 != 0)) return hipErrorInvalidValue;
  if (tb) {
    if (a.ldb % 8 != 0 || a.ldb < a.N || a.seg_end[0] % 64 != 0 || a.seg_end[1] % 64 != 0 ||
        a.seg_end[0] > a.seg_end[1] || a.seg_end[1] > a.seg_end[2] || a.seg_end[2] < 1)
      return hipErrorInvalidValue;
    for (int i = 0; i < 3; ++i)
      if ((uintptr_t)a.B[i] % 16 != 0) return hipErrorInvalidValue;
  }
  if (ta && a.lda < a.M) return hipErrorInvalidValue;
  if (a.trans == 2) return launch_cfg<256, 256, 64, 2, 2, 4, 16, 1, kModeSeg, EPI, 2>(a, s);
  if constexpr (EPI != kEpiSwigluBwd)
    if (a.trans == 3) return launch_cfg<256, 256, 64, 2, 2, 4, 16, 1, kModeSeg, EPI, 3>(a, s);
  return hipErrorInvalidValue;
}

template <int MODE, int EPI>
hipError_t dispatch(const GemmArgs& a, int tile, hipStream_t s) {
  if constexpr (EPI == kEpiSwigluBwd) {
    if (MODE != kModeSeg || a.trans != 2 || tile != kTileDma256x256 || a.splits != 1 || a.N % 4 != 0 ||
        a.ldr % 4 != 0 || !a.resid || !a.C || !a.C2)
      return hipErrorInvalidValue;
    return launch_trans<EPI>(a, s);
  } else {
    if (a.trans != 0) {
      if constexpr (MODE == kModeSeg && (EPI == kEpiResid || EPI == kEpiPartial))
        return tile == kTileDma256x256 ? launch_trans<EPI>(a, s) : hipErrorInvalidValue;
      else
        return hipErrorInvalidValue;
    }
    switch (tile) {
      case kTileDma256x256: return launch_cfg<256, 256, 64, 2, 2, 4, 16, 1, MODE, EPI>(a, s);
      case kTileDma256x256n: return launch_cfg<256, 256, 64, 2, 4, 2, 16, 0, MODE, EPI>(a, s);
      case kTileDma256x256m32: return launch_cfg<256, 256, 64, 2, 2, 4, 32, 0, MODE, EPI>(a, s);
      case kTileDma256x192:
        if constexpr (MODE == kModeGated) return hipErrorInvalidValue;
        else return launch_cfg<256, 192, 64, 2, 4, 2, 16, 1, MODE, EPI>(a, s);
    }
    return hipErrorInvalidValue;
  }
}

}  // namespace

bool gemm_dma_tile(int tile) { return tile >= kTileDma256x256 && tile <= kTileDma256x192; }

hipError_t launch_gemm_dma(const GemmArgs& a, int mode, int epi, int tile, hipStream_t s) {
  if (mode == kModeGated) {
    if (epi == kEpiGated) return dispatch<kModeGated, kEpiGated>(a, tile, s);
    if (epi == kEpiPartial) return dispatch<kModeGated, kEpiPartial>(a, tile, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case kEpiStore: return dispatch<kModeSeg, kEpiStore>(a, tile, s);
    case kEpiResid: return dispatch<kModeSeg, kEpiResid>(a, tile, s);
    case kEpiPartial: return dispatch<kModeSeg, kEpiPartial>(a, tile, s);
    case kEpiSwigluBwd: return dispatch<kModeSeg, kEpiSwigluBwd>(a, tile, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gqa
