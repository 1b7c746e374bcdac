// Host runtime of the decoder-block library: the C ABI of include/gqa_block.h.
//
// It follows the mojolearn "mojolearn.transformer" API page (TransformerBlock,
// allocate_state, forward, step, TransformerState): weights keyed by Hugging
// Face names in [out, in] layout, a caller-owned KV cache, every argument
// check made on the host before any device work is enqueued.  Per call it
// only enqueues kernels on the caller's stream; nothing is allocated, nothing
// synchronises.
#include "../../../include/gqa_block.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstdarg>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../kernels/launch.h"

using namespace gqa;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

#define HIP_TRY(expr)                                                                      \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess) return fail(GQA_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

enum WIdx {
  W_IN_NORM, W_POST_NORM, W_Q, W_K, W_V, W_O, W_GATE, W_UP, W_DOWN,
  W_QB, W_KB, W_VB, W_QN, W_KN,
  W_OB, W_GB, W_UB, W_DB, W_PRE_FF, W_POST_FF, W_IN_NB, W_POST_NB, W_PRE_FFB, W_POST_FFB, W_COUNT
};
const char* const kNames[W_COUNT] = {
    "input_layernorm.weight", "post_attention_layernorm.weight", "q_proj.weight", "k_proj.weight",
    "v_proj.weight", "o_proj.weight", "gate_proj.weight", "up_proj.weight", "down_proj.weight",
    "q_proj.bias", "k_proj.bias", "v_proj.bias", "q_norm.weight", "k_norm.weight",
    "o_proj.bias", "gate_proj.bias", "up_proj.bias", "down_proj.bias",
    "pre_feedforward_layernorm.weight", "post_feedforward_layernorm.weight",
    "input_layernorm.bias", "post_attention_layernorm.bias", "pre_feedforward_layernorm.bias",
    "post_feedforward_layernorm.bias"};

bool mlp_gated(int mlp) { return mlp == GQA_MLP_SWIGLU || mlp == GQA_MLP_GEGLU_TANH || mlp == GQA_MLP_GEGLU; }
int mlp_act(int mlp) {
  switch (mlp) {
    case GQA_MLP_GEGLU_TANH: case GQA_MLP_GELU_TANH: return kActGeluTanh;
    case GQA_MLP_GEGLU: case GQA_MLP_GELU: return kActGelu;
    default: return kActSilu;
  }
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Per-kernel timing with HIP events on the caller's stream.
struct KernelTimer {
  struct Entry { std::string name; double ms = 0; int64_t count = 0; };
  struct Pending { int entry; hipEvent_t a, b; };
  bool enabled = false;
  std::vector<Entry> entries;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;

  int entry_of(const char* name) {
    for (size_t i = 0; i < entries.size(); ++i)
      if (entries[i].name == name) return (int)i;
    entries.push_back({name, 0, 0});
    return (int)entries.size() - 1;
  }
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void collect() {
    for (auto& p : pending) {
      float ms = 0.f;
      hipEventSynchronize(p.b);
      if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
        entries[p.entry].ms += ms;
        entries[p.entry].count += 1;
      }
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
  ~KernelTimer() {
    collect();
    for (auto e : pool) hipEventDestroy(e);
  }
};

struct Scope {
  KernelTimer* t;
  hipStream_t s;
  int entry = -1;
  hipEvent_t a = nullptr, b = nullptr;
  Scope(KernelTimer* t_, const char* name, hipStream_t s_) : t(t_), s(s_) {
    if (!t->enabled) return;
    entry = t->entry_of(name);
    a = t->get();
    b = t->get();
    if (a && b) hipEventRecord(a, s);
  }
  ~Scope() {
    if (!t->enabled || !a || !b) return;
    hipEventRecord(b, s);
    t->pending.push_back({entry, a, b});
  }
};

// tile: GemmTile; splits: K splits (partials + ordered reduce); waves: per
// workgroup (decode kernel).  m1 / n1 / tail_splits (large-M tiles only):
// rows [m1, M), or else columns [n1, N) -- the tiles past the last full wave
// of the CUs -- run as a separate launch with tail_splits K splits, so the
// tail fills the machine.
struct GemmPlan { int tile; int splits; int waves = 0; int m1 = 0; int tail_splits = 0; int n1 = 0; int n = 0; };
constexpr int kStatusWords = 4;

}  // namespace

struct gqa_block {
  gqa_block_config cfg;
  const void* w[W_COUNT] = {};
  int QW = 0, KW = 0, G = 0;
  size_t es = 4;           // activation / weight element size
  float* cos_tab = nullptr;
  float* sin_tab = nullptr;
  // device words: [0] a non-finite input was seen, [1] the count of non-finite
  // cached keys/values found by the GQA_CHECK_FINITE scan, [2] a device start
  // position was out of range (clamped)
  int* status = nullptr;
  bool check_finite = false;
  std::atomic<int> busy{0};
  KernelTimer timer;
};

struct gqa_state {
  const gqa_block* blk;
  int batch, max_tokens, capacity;
  void* k;
  void* v;
  int* lengths_dev;
  std::vector<int> lengths;  // host mirror
  // Pinned staging ring for gqa_state_set_lengths: the copy is asynchronous,
  // and a slot is reused only after its previous copy has completed.
  static constexpr int kRing = 4;
  int* staging = nullptr;    // kRing * batch ints (pinned host memory)
  hipEvent_t done[kRing] = {};
  int next = 0;
  ~gqa_state() {
    for (auto& e : done)
      if (e) hipEventDestroy(e);
    if (staging) hipHostFree(staging);
  }
};

namespace {

bool is_bf16(const gqa_block* b) { return b->cfg.weight_dtype == GQA_BF16; }

// The large-M tile: 256x256 on the direct-to-LDS pipelined kernel (8 waves of
// 128x64, 64-deep slices, 2 stages).  GQA_GEMM_BIG_TILE (a GemmTile value)
// overrides it for tuning.
int big_tile() {
  static int t = [] {
    const char* e = getenv("GQA_GEMM_BIG_TILE");
    return e ? atoi(e) : (int)kTileDma256x256;
  }();
  return t;
}
// Keys per decode-attention segment (GQA_DECODE_SEG_KEYS overrides, tuning).
int decode_keys_per_segment() {
  static int k = [] {
    const char* e = getenv("GQA_DECODE_SEG_KEYS");
    return e && atoi(e) > 0 ? atoi(e) : 768;
  }();
  return k;
}
// Tile order of the pipelined GEMM (GQA_GEMM_ORDER overrides the XCD-aware
// default for tuning).
int gemm_tile_order() {
  static int o = [] {
    const char* e = getenv("GQA_GEMM_ORDER");
    return e ? atoi(e) : 0;
  }();
  return o;
}
// The 256x192 tile that goes with big_tile() (same kernel family).
int big_tile_192() {
  const int t = big_tile();
  return gemm_dma_tile(t) ? (int)kTileDma256x192 : (int)kTile256x192;
}

// Tile and K-split choice for a bf16 GEMM with M rows, N output columns, K
// depth.  M > 512: the pipelined direct-to-LDS kernel, 256x256 or (when its
// estimated time is lower) 256x192 tiles.  129..512: 128x128 tiles.  65..128:
// 64x128 tiles with a K split.  M <= 64 (decode): the weight-streaming kernel
// (below), else 64x64 tiles split while there are fewer than 256 tiles.
// A large-M plan whose last wave of tiles fills at most half of the CUs:
// rows (or else columns) covered by the full waves stay as they are; the
// remaining ones are split along K so that their tiles x splits come close
// to one full wave
// (splits 64-aligned and at least 512 deep).
// Partials of the largest tail with_tail plans: at most one wave (256 units)
// of tile x split, each 256 rows x at most 256 float32 columns.
constexpr size_t kTailPartBytes = (size_t)256 * 256 * 256 * 4;

GemmPlan with_tail(GemmPlan p, int M, int N, int K, int cols) {
  // the CU count the waves are counted in (GQA_GEMM_TAIL_CUS overrides it,
  // read per plan so a test can exercise tails at small sizes; 0: no tails)
  const char* e = getenv("GQA_GEMM_TAIL_CUS");
  const int cus = e ? atoi(e) : 256;
  if (cus <= 0) return p;
  const long ntn = (N + cols - 1) / cols, ntm = (M + 255) / 256, tiles = ntm * ntn;
  if (tiles <= cus || tiles % cus == 0 || tiles % cus > cus / 2) return p;
  const long full = (tiles / cus) * cus;  // tiles in the full waves
  // K splits of a tail of t2 tiles: as many as fit one wave, 64-aligned, at least 512 deep
  auto splits_for = [&](long t2) {
    int sp = (int)std::min<long>(8, cus / t2);
    while (sp > 1 && (K % (64 * sp) != 0 || K / sp < 512)) --sp;
    return sp;
  };
  // rows: the M-tile rows wholly inside the full waves
  const long m1_tiles = full / ntn;
  if (m1_tiles > 0 && m1_tiles < ntm) {
    const int sp = splits_for((ntm - m1_tiles) * ntn);
    if (sp >= 2) {
      p.m1 = (int)(m1_tiles * 256);
      p.tail_splits = sp;
      return p;
    }
  }
  // columns: when the full waves hold whole N-tile columns
  if (full % ntm == 0) {
    const long n1_tiles = full / ntm;
    if (n1_tiles > 0 && n1_tiles < ntn) {
      const int sp = splits_for(ntm * (ntn - n1_tiles));
      if (sp >= 2) {
        p.n1 = (int)(n1_tiles * cols);
        p.n = N;
        p.tail_splits = sp;
      }
    }
  }
  return p;
}

GemmPlan plan_gemm(int M, int N, int K, bool gated) {
  if (M > 128) {
    if (M <= 512) return {kTile128x128, 1};
    const int cols256 = gated ? 128 : 256;
    const long t256 = (long)((M + 255) / 256) * ((N + cols256 - 1) / cols256);
    const GemmPlan p256 = with_tail({big_tile(), 1}, M, N, K, cols256);
    const char* e192 = getenv("GQA_GEMM_TILE192");  // tuning override (0: never the 256x192 tile)
    if (!gated && N % 192 == 0 && !(e192 && atoi(e192) == 0)) {
      // Estimated time in 64-deep slices of one 256x256 tile (1.84 us measured):
      // a wave of 256x192 tiles takes 0.87 of a 256x256 wave of the same depth
      // (8B q/k/v, Gemma2-style down); a tail split adds its depth per split and
      // its float32 partials, written and read back at ~2.5 TB/s.
      const double slices = K / 64.0;
      const long t192 = (long)((M + 255) / 256) * (N / 192);
      const double est192 = (double)((t192 + 255) / 256) * 0.87 * slices;
      double est256 = (double)((t256 + 255) / 256) * slices;
      if (p256.tail_splits > 1) {
        const long tail_tiles = p256.m1 > 0 ? ((M - p256.m1 + 255) / 256) * ((N + cols256 - 1) / cols256)
                                            : ((M + 255) / 256) * ((N - p256.n1 + cols256 - 1) / cols256);
        const double part = (double)tail_tiles * p256.tail_splits * 256.0 * 256.0 * 4.0 * 2.0;
        est256 = (double)(t256 / 256) * slices + slices / p256.tail_splits + part / (2.5e12 * 1.84e-6);
      }
      if (est192 < est256) return with_tail({big_tile_192(), 1}, M, N, K, 192);
    }
    return p256;
  }
  if (M > 64) {
    const int cols = gated ? 64 : 128;
    const long tiles = (long)((M + 63) / 64) * ((N + cols - 1) / cols);
    int splits = 1;
    while (tiles * splits < 512 && K / (splits * 2) >= 256 && (K / 64) % (splits * 2) == 0) splits *= 2;
    return {kTile64x128, splits};
  }
  // M <= 64: the weight-streaming kernel, one 16-row weight group per wave.
  // Choose the K split s (a divisor of K / 256, splits at least kmin deep) and
  // the waves per workgroup w (4..8, dividing the group count) by a time
  // model fitted to measurements on the 8B and Qwen-style decode shapes:
  // workgroups run in rounds of one per CU, each round costing a fixed
  // 4.5 us (prologue, pipeline fill, drain) plus its weight bytes (and its
  // float32 partials) at 28 GB/s per CU with 6 or more waves, proportionally
  // less below; K-split partials are read back at 2 TB/s, and a gated split
  // needs its own reduce launch (5 us).  (Measured: Qwen-style gate/up, M = 16,
  // 3456 groups, K = 5120, unsplit in 432 workgroups of 8 waves 92.9 us
  // against 120.8 + 6.7 us in 4 splits over 2304 workgroups of 6.)
  static const int cus = [] {
    const char* e = getenv("GQA_SKINNY_CUS");  // tuning override
    return e ? atoi(e) : 256;
  }();
  // Splits at least 1024 deep: on the 8B decode shapes a shallower o_proj
  // split (8 x 512) streams no faster and doubles the partials the next
  // kernel sums (measured 14.9 + 9.9 us against 13.1 + 8.5 us).
  static const int kmin = [] {
    const char* e = getenv("GQA_SKINNY_KMIN");  // tuning override
    return e ? atoi(e) : 1024;
  }();
  if (M <= 64 && K % 256 == 0) {
    const long groups = gemm_skinny_groups(N, gated);
    GemmPlan best{kTileSkinny, 0, 0};
    double best_cost = 0.0;
    for (int w = 8; w >= 4; --w)
      for (int sp = 1; sp <= K / 256; ++sp) {
        if ((K / 256) % sp != 0 || (sp > 1 && K / sp < kmin)) continue;
        if (!gemm_skinny_supported(M, N, K, K / sp, w, gated)) continue;
        const long wgs = groups / w * sp;
        const long rounds = (wgs + cus - 1) / cus;
        const double part_wg = sp > 1 ? 16.0 * w * M * 4.0 : 0.0;          // partial bytes per workgroup
        const double wg_bytes = 16.0 * w * (double)(K / sp) * 2.0 + part_wg;
        const double rate = 28e3 * (w >= 6 ? 1.0 : w / 6.0);                // bytes per us per CU
        double cost = rounds * (4.5 + wg_bytes / rate);
        if (sp > 1) cost += part_wg * wgs / 2e6 + (gated ? 5.0 : 0.0);
        if (best.waves == 0 || cost < best_cost * (1.0 - 1e-9)) {
          best_cost = cost;
          best = {kTileSkinny, sp, w};
        }
      }
    if (best.waves > 0) return best;
  }
  const int cols = gated ? 32 : 64;
  const long tiles = (N + cols - 1) / cols;
  int splits = 1;
  if (tiles < 256)
    while (tiles * splits < 512 && K / (splits * 2) >= 1024 && (K / 64) % (splits * 2) == 0) splits *= 2;
  return {kTile64x64, splits};
}

// Bytes of float32 K-split partials a plan needs for M rows of nb columns
// (nb: N, or 2 N for the gated pair): its K splits over all rows, or its tail
// splits over the tail rows.
size_t plan_part_bytes(const GemmPlan& p, int M, size_t nb) {
  size_t b = 0;
  if (p.splits > 1) b = (size_t)p.splits * M * nb * 4;
  if (p.tail_splits > 1 && p.m1 > 0 && p.m1 < M) b = std::max(b, (size_t)p.tail_splits * (M - p.m1) * nb * 4);
  if (p.tail_splits > 1 && p.n1 > 0 && p.n1 < p.n)
    b = std::max(b, (size_t)p.tail_splits * M * (nb / p.n) * (p.n - p.n1) * 4);
  return b;
}

struct WsLayout {
  size_t h, qkv, knew, vnew, ctx, x1, h2, act, part, attn_part, rows, total;
  GemmPlan p_qkv, p_o, p_gu, p_down;
  bool decode_attn;
};

WsLayout layout_for(const gqa_block* blk, int B, int L) {
  const auto& c = blk->cfg;
  WsLayout w{};
  const size_t T = (size_t)B * L, es = blk->es;
  const int d = c.d_model, QW = blk->QW, KW = blk->KW, IT = c.intermediate;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  w.h = take(T * d * es);
  w.qkv = take(T * (QW + 2 * (size_t)KW) * es);
  w.knew = take(T * KW * es);
  w.vnew = take(T * KW * es);
  w.ctx = take(T * QW * es);
  w.x1 = take(T * d * 4);
  w.h2 = take(T * d * es);
  w.act = take(T * IT * es);
  w.rows = take((size_t)B * 2 * 4);  // packed ragged rows: row_start[B], row_len[B]
  w.part = w.attn_part = 0;
  w.decode_attn = false;
  if (is_bf16(blk)) {
    const int M = (int)T;
    w.p_qkv = plan_gemm(M, QW + 2 * KW, d, false);
    w.p_o = plan_gemm(M, d, QW, false);
    const bool gated = mlp_gated(c.mlp);
    w.p_gu = plan_gemm(M, IT, d, gated);
    w.p_down = plan_gemm(M, d, IT, false);
    size_t part = 0;
    auto need = [&](const GemmPlan& p, size_t nb) { part = std::max(part, plan_part_bytes(p, M, nb)); };
    need(w.p_qkv, QW + 2 * (size_t)KW);
    need(w.p_o, d);
    need(w.p_gu, (gated ? 2 : 1) * (size_t)IT);
    need(w.p_down, d);
    // a prefill of any fewer rows (a packed ragged batch) may split a tail of
    // at most one wave of 256 x 256 tiles (with_tail): room for its partials
    if (M > 512 && L > 1) part = std::max(part, kTailPartBytes);
    if (part) w.part = take(part);
    if (L == 1 && attention_decode_bf16_supported(c.head_dim, blk->G) && B <= attention_decode_max_rows()) {
      w.decode_attn = true;
      // records [H, max segments + B, hd + 2] floats, then the row table (2 ints per row)
      w.attn_part = take((size_t)c.n_heads * (attention_decode_max_segments() + B) * (c.head_dim + 2) * 4 +
                         (size_t)B * 2 * 4);
    }
  }
  w.total = off;
  return w;
}

// RoPE frequencies theta_i, i < rope_dim/2 (DantinoX "Core Layers" page,
// Positional Encoding / RoPE: base^(-2i/d) with d the rotated dimensions),
// scaled as mojolearn ``rope_scaling`` names: "linear" divides each by the
// factor; "llama3" is Hugging Face's Llama 3 wavelength ramp (long
// wavelengths divided by the factor, short ones kept, a linear blend in
// n / wavelength between).  Double precision throughout.
std::vector<double> rope_frequencies(const gqa_block_config& c) {
  const int rd = c.rope_dim, half = rd / 2;
  std::vector<double> inv(half);
  const double f = c.rope_factor;
  for (int i = 0; i < half; ++i) {
    const double th = std::pow((double)c.rope_theta, -2.0 * i / rd);
    double out = th;
    if (c.rope_scaling == GQA_ROPE_LINEAR) {
      out = th / f;
    } else if (c.rope_scaling == GQA_ROPE_LLAMA3) {
      const double lo = c.rope_low_freq_factor, hi = c.rope_high_freq_factor;
      const double ctx = c.rope_original_max_positions;
      const double wavelen = 2.0 * M_PI / th;
      if (wavelen > ctx / lo) {
        out = th / f;
      } else if (!(wavelen < ctx / hi)) {
        const double s = (ctx / wavelen - lo) / (hi - lo);
        out = (1.0 - s) * th / f + s * th;
      }
    }
    inv[i] = out;
  }
  return inv;
}

int check_config(const gqa_block_config* c) {
  if (!c) return fail(GQA_ERR_ARG, "config is NULL");
  if (c->d_model <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->head_dim <= 0 || c->intermediate <= 0)
    return fail(GQA_ERR_SHAPE, "d_model, n_heads, n_kv_heads, head_dim and intermediate must be positive");
  if (c->n_heads % c->n_kv_heads != 0)
    return fail(GQA_ERR_SHAPE, "n_heads (%d) must be a multiple of n_kv_heads (%d)", c->n_heads, c->n_kv_heads);
  if (c->head_dim % 2 != 0) return fail(GQA_ERR_SHAPE, "head_dim (%d) must be even", c->head_dim);
  if (c->head_dim > 256) return fail(GQA_ERR_UNSUPPORTED, "head_dim %d > 256 is not supported", c->head_dim);
  if (c->window < 0) return fail(GQA_ERR_ARG, "window must be >= 0");
  if (c->max_positions <= 0) return fail(GQA_ERR_ARG, "max_positions must be positive");
  if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return fail(GQA_ERR_ARG, "rope_theta must be > 0");
  if (!(c->norm_eps >= 0.f) || !std::isfinite(c->norm_eps)) return fail(GQA_ERR_ARG, "norm_eps must be >= 0");
  if (!(c->attn_softcap >= 0.f) || !std::isfinite(c->attn_softcap))
    return fail(GQA_ERR_ARG, "attn_softcap must be >= 0 (0 = off)");
  if (c->norm != GQA_NORM_RMS && c->norm != GQA_NORM_RMS_OFFSET && c->norm != GQA_NORM_LAYER)
    return fail(GQA_ERR_ARG, "unknown norm kind");
  if (c->mlp < GQA_MLP_SWIGLU || c->mlp > GQA_MLP_GELU_TANH) return fail(GQA_ERR_ARG, "unknown mlp kind");
  for (int f : {c->qkv_bias, c->qk_norm, c->o_bias, c->mlp_bias, c->norm_bias, c->sandwich_norms})
    if (f != 0 && f != 1)
      return fail(GQA_ERR_ARG, "qkv_bias, qk_norm, o_bias, mlp_bias, norm_bias and sandwich_norms must be 0 or 1");
  if (c->norm_bias && c->norm != GQA_NORM_LAYER) return fail(GQA_ERR_ARG, "norm_bias needs norm = LayerNorm");
  if (!norm_supported(c->d_model))
    return fail(GQA_ERR_UNSUPPORTED, "d_model %d is beyond the norm kernels (16384 when a multiple of 4, "
                                     "else 12288)", c->d_model);
  if (c->weight_dtype != GQA_F32 && c->weight_dtype != GQA_BF16) return fail(GQA_ERR_DTYPE, "unknown weight dtype");
  if (c->rope_dim != 0 && (c->rope_dim < 2 || c->rope_dim > c->head_dim || c->rope_dim % 2))
    return fail(GQA_ERR_ARG, "rope_dim (%d) must be 0 (= head_dim) or even in [2, head_dim=%d]", c->rope_dim,
                c->head_dim);
  if (c->rope_scaling != GQA_ROPE_PLAIN && c->rope_scaling != GQA_ROPE_LINEAR && c->rope_scaling != GQA_ROPE_LLAMA3)
    return fail(GQA_ERR_ARG, "unknown rope_scaling kind %d", c->rope_scaling);
  if (c->rope_scaling != GQA_ROPE_PLAIN && (!(c->rope_factor > 0.f) || !std::isfinite(c->rope_factor)))
    return fail(GQA_ERR_ARG, "rope_factor must be > 0");
  if (c->rope_scaling == GQA_ROPE_LLAMA3 &&
      (!(c->rope_low_freq_factor > 0.f) || !(c->rope_high_freq_factor > c->rope_low_freq_factor) ||
       !std::isfinite(c->rope_high_freq_factor) || c->rope_original_max_positions <= 0))
    return fail(GQA_ERR_ARG, "llama3 rope scaling needs 0 < low_freq_factor < high_freq_factor and "
                             "original_max_positions > 0");
  if (c->weight_dtype == GQA_BF16) {
    const int QW = c->n_heads * c->head_dim;
    if (c->d_model % 64 || QW % 64 || c->intermediate % 64)
      return fail(GQA_ERR_UNSUPPORTED,
                  "bf16 blocks need d_model, n_heads*head_dim and intermediate to be multiples of 64 "
                  "(got %d, %d, %d)", c->d_model, QW, c->intermediate);
    if (c->head_dim % 8) return fail(GQA_ERR_UNSUPPORTED, "bf16 blocks need head_dim %% 8 == 0");
  }
  return GQA_OK;
}

int check_weights(const gqa_block_config* c, const gqa_tensor* ws, int n, const void* out[W_COUNT]) {
  if (n < 0 || (n > 0 && !ws)) return fail(GQA_ERR_ARG, "weights array is NULL");
  const int64_t d = c->d_model, hd = c->head_dim, QW = (int64_t)c->n_heads * hd,
                KW = (int64_t)c->n_kv_heads * hd, IT = c->intermediate;
  const int64_t shapes[W_COUNT][2] = {{d, 0},  {d, 0},  {QW, d}, {KW, d}, {KW, d}, {d, QW}, {IT, d},
                                      {IT, d}, {d, IT}, {QW, 0}, {KW, 0}, {KW, 0}, {hd, 0}, {hd, 0},
                                      {d, 0},  {IT, 0}, {IT, 0}, {d, 0},  {d, 0},  {d, 0},  {d, 0},
                                      {d, 0},  {d, 0},  {d, 0}};
  const bool gated = mlp_gated(c->mlp);
  bool wanted[W_COUNT];
  for (int i = 0; i < W_COUNT; ++i) wanted[i] = i <= W_DOWN;
  if (!gated) wanted[W_GATE] = false;
  if (c->qkv_bias) wanted[W_QB] = wanted[W_KB] = wanted[W_VB] = true;
  if (c->qk_norm) wanted[W_QN] = wanted[W_KN] = true;
  if (c->o_bias) wanted[W_OB] = true;
  if (c->mlp_bias) wanted[W_UB] = wanted[W_DB] = true, wanted[W_GB] = gated;
  if (c->sandwich_norms) wanted[W_PRE_FF] = wanted[W_POST_FF] = true;
  if (c->norm_bias) {
    wanted[W_IN_NB] = wanted[W_POST_NB] = true;
    if (c->sandwich_norms) wanted[W_PRE_FFB] = wanted[W_POST_FFB] = true;
  }
  for (int i = 0; i < W_COUNT; ++i) out[i] = nullptr;
  for (int t = 0; t < n; ++t) {
    const gqa_tensor& w = ws[t];
    if (!w.name) return fail(GQA_ERR_ARG, "weight %d has no name", t);
    int idx = -1;
    for (int i = 0; i < W_COUNT; ++i)
      if (!strcmp(w.name, kNames[i])) idx = i;
    if (idx < 0 || !wanted[idx]) return fail(GQA_ERR_SHAPE, "unexpected weight '%s' for this configuration", w.name);
    if (out[idx]) return fail(GQA_ERR_SHAPE, "weight '%s' given twice", w.name);
    if (!w.data_dev) return fail(GQA_ERR_ARG, "weight '%s' has a NULL pointer", w.name);
    const bool matrix = idx >= W_Q && idx <= W_DOWN;
    const int nd = matrix ? 2 : 1;
    if (w.ndim != nd || w.shape[0] != shapes[idx][0] || (nd == 2 && w.shape[1] != shapes[idx][1])) {
      if (nd == 2)
        return fail(GQA_ERR_SHAPE, "weight '%s' must have shape (%lld, %lld)", w.name, (long long)shapes[idx][0],
                    (long long)shapes[idx][1]);
      return fail(GQA_ERR_SHAPE, "weight '%s' must have shape (%lld,)", w.name, (long long)shapes[idx][0]);
    }
    const int want_dt = matrix ? c->weight_dtype : GQA_F32;
    if (w.dtype != want_dt)
      return fail(GQA_ERR_DTYPE, "weight '%s' must be %s", w.name, want_dt == GQA_BF16 ? "bfloat16" : "float32");
    out[idx] = w.data_dev;
  }
  for (int i = 0; i < W_COUNT; ++i)
    if (wanted[i] && !out[i]) return fail(GQA_ERR_SHAPE, "missing weight '%s'", kNames[i]);
  return GQA_OK;
}

struct BusyGuard {
  std::atomic<int>& f;
  bool ok, held = false;
  // take = false: the caller already holds the guard (nothing to take or release)
  explicit BusyGuard(std::atomic<int>& f_, bool take = true) : f(f_) {
    if (!take) {
      ok = true;
      return;
    }
    int z = 0;
    ok = held = f.compare_exchange_strong(z, 1);
  }
  ~BusyGuard() {
    if (held) f.store(0);
  }
};

// Packed ragged rows (a ragged prefill): `rows` tokens, row b's real tokens at
// packed rows row_start[b] .. + row_len[b] - 1 (device tables), with GEMM
// plans for that many rows.
struct PackedRows {
  const int* row_start;
  const int* row_len;
  int rows;
  GemmPlan p_qkv, p_o, p_gu, p_down;
};

// recompute_only: stop after the MLP's input norm (h2), the activations the
// backward reads (no MLP, no y); the backward holds the busy guard itself.
// pk: the tokens are packed ragged rows (x and y are [pk->rows, d]; the
// caller holds the busy guard).
int run_block(gqa_block* blk, gqa_state* st, const float* x, float* y, int B, int L, void* ws, size_t wsb,
              hipStream_t s, float* attn_lse = nullptr, bool recompute_only = false,
              const PackedRows* pk = nullptr) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  const auto& c = blk->cfg;
  if (B < 0 || L < 0) return fail(GQA_ERR_ARG, "B and L must be >= 0");
  if (st) {
    if (st->blk != blk) return fail(GQA_ERR_STATE, "state belongs to another block");
    if (B != st->batch) return fail(GQA_ERR_STATE, "batch size %d differs from the state's %d", B, st->batch);
  }
  if (B == 0 || L == 0) return GQA_OK;
  if (!x || !y) return fail(GQA_ERR_ARG, "x or y is NULL");
  for (int b = 0; b < B; ++b) {
    const long start = st ? st->lengths[b] : 0;
    if (st && start + L > st->max_tokens)
      return fail(GQA_ERR_CAPACITY, "row %d: %ld cached + %d new tokens exceed the state's max_tokens %d", b, start, L,
                  st->max_tokens);
    if (start + L > c.max_positions)
      return fail(GQA_ERR_POSITION, "row %d: position %ld is at or beyond max_positions %d", b, start + L - 1,
                  c.max_positions);
  }
  WsLayout lay = layout_for(blk, B, L);
  if (!ws || wsb < lay.total)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? wsb : (size_t)0, lay.total);
  if (pk) {
    lay.p_qkv = pk->p_qkv;
    lay.p_o = pk->p_o;
    lay.p_gu = pk->p_gu;
    lay.p_down = pk->p_down;
  }
  BusyGuard guard(blk->busy, !recompute_only && !pk);
  if (!guard.ok) return fail(GQA_ERR_BUSY, "block is in use by another call");

  char* base = static_cast<char*>(ws);
  const int T = pk ? pk->rows : B * L, d = c.d_model, QW = blk->QW, KW = blk->KW, IT = c.intermediate,
            hd = c.head_dim;
  const bool bf = is_bf16(blk);
  const int et = bf ? kBF16 : kF32;
  void* h = base + lay.h;
  void* qkv = base + lay.qkv;
  void* knew = base + lay.knew;
  void* vnew = base + lay.vnew;
  void* ctx = base + lay.ctx;
  float* x1 = reinterpret_cast<float*>(base + lay.x1);
  void* h2 = base + lay.h2;
  void* act = base + lay.act;
  float* part = lay.part ? reinterpret_cast<float*>(base + lay.part) : nullptr;
  int* lengths = st ? st->lengths_dev : nullptr;
  const int offset = c.norm == GQA_NORM_RMS_OFFSET;
  KernelTimer* tm = &blk->timer;

  // A tail-split plan's launches: a1 = the full waves of tiles, then the tail
  // a2 as K-split partials and the ordered reduce that applies the epilogue
  // (timed as name, name_tail and name_tail_reduce: one launch each).
  auto run_tail = [&](const char* name, const GemmArgs& a1, GemmArgs a2, int mode, int epi,
                      const GemmPlan& p) -> int {
    a2.bump = nullptr;  // a1 advances the lengths
    GemmArgs pa = a2;
    pa.splits = p.tail_splits;
    pa.k_split = a2.K / p.tail_splits;
    pa.partial = part;
    const std::string tn = std::string(name) + "_tail", rn = tn + "_reduce";
    {
      Scope sc(tm, name, s);
      HIP_TRY(launch_gemm_bf16(a1, mode, epi, p.tile, s));
    }
    {
      Scope sc(tm, tn.c_str(), s);
      HIP_TRY(launch_gemm_bf16(pa, mode, kEpiPartial, p.tile, s));
    }
    a2.splits = p.tail_splits;
    a2.partial = part;
    Scope sc(tm, rn.c_str(), s);
    HIP_TRY(launch_splitk_reduce(a2, mode, epi, et, s));
    return GQA_OK;
  };
  // GEMM helper: fused epilogue, or K-split partials + ordered reduce.
  // (defer_reduce: leave the K-split partials in `part` for the next kernel,
  // which sums them itself)
  auto gemm = [&](const char* name, GemmArgs a, int mode, int epi, const GemmPlan& p,
                  bool defer_reduce = false) -> int {
    a.order = gemm_tile_order();
    a.wg_waves = p.waves;
    if (!bf) {
      Scope sc(tm, name, s);
      HIP_TRY(launch_gemm_f32(a, mode, epi, s));
      return GQA_OK;
    }
    if (p.splits <= 1 && p.tail_splits > 1 && p.n1 > 0 && p.n1 < a.N && p.n == a.N && !defer_reduce) {
      // columns [0, n1): the full waves of tiles; columns [n1, N): K-split, then
      // the ordered reduce applies the epilogue to them.  Each part is the same
      // GEMM over a column range: the weight segments, biases and outputs of
      // that range.
      const int es_out = epi == kEpiResid ? 4 : (int)blk->es;
      auto columns = [&](int n0, int nend) {
        GemmArgs r = a;
        r.N = nend - n0;
        r.C = static_cast<char*>(a.C) + (size_t)n0 * es_out;
        if (a.resid) r.resid = a.resid + n0;
        if (mode == kModeGated) {  // gate / up rows n0 .. of both matrices
          for (int q = 0; q < 2; ++q) {
            r.B[q] = static_cast<const char*>(a.B[q]) + (size_t)n0 * a.K * blk->es;
            r.bias[q] = a.bias[q] ? a.bias[q] + n0 : nullptr;
          }
          return r;
        }
        const int64_t starts[3] = {0, a.seg_end[0], a.seg_end[1]};
        int k = 0;
        for (int q = 0; q < 3; ++q) {
          const int64_t lo = std::max<int64_t>(starts[q], n0), hi = std::min<int64_t>(a.seg_end[q], nend);
          if (lo >= hi) continue;
          r.B[k] = static_cast<const char*>(a.B[q]) + (size_t)(lo - starts[q]) * a.K * blk->es;
          r.bias[k] = a.bias[q] ? a.bias[q] + (lo - starts[q]) : nullptr;
          r.seg_end[k] = hi - n0;
          ++k;
        }
        for (; k < 3; ++k) {
          r.B[k] = r.B[k - 1];
          r.bias[k] = r.bias[k - 1];
          r.seg_end[k] = r.seg_end[k - 1];
        }
        return r;
      };
      GemmArgs a1 = columns(0, p.n1);
      a1.splits = 1;
      a1.k_split = a.K;
      return run_tail(name, a1, columns(p.n1, a.N), mode, epi, p);
    }
    if (p.splits <= 1 && p.tail_splits > 1 && p.m1 > 0 && p.m1 < a.M && !defer_reduce) {
      // rows [0, m1): the full waves of tiles; rows [m1, M): K-split, then the
      // ordered reduce applies the epilogue to them
      const int es_out = epi == kEpiResid ? 4 : (int)blk->es;
      const size_t a_es = blk->es;
      GemmArgs a1 = a;
      a1.M = p.m1;
      a1.splits = 1;
      a1.k_split = a.K;
      GemmArgs a2 = a;
      a2.M = a.M - p.m1;
      a2.A = static_cast<const char*>(a.A) + (size_t)p.m1 * a.lda * a_es;
      a2.C = static_cast<char*>(a.C) + (size_t)p.m1 * a.ldc * es_out;
      if (a.resid) a2.resid = a.resid + (size_t)p.m1 * a.ldr;
      return run_tail(name, a1, a2, mode, epi, p);
    }
    if (p.splits <= 1) {
      a.splits = 1;
      a.k_split = a.K;
      Scope sc(tm, name, s);
      HIP_TRY(launch_gemm_bf16(a, mode, epi, p.tile, s));
      return GQA_OK;
    }
    GemmArgs pa = a;
    pa.splits = p.splits;
    pa.k_split = a.K / p.splits;
    pa.partial = part;
    if (!defer_reduce) pa.bump = nullptr;  // the reduce kernel advances the lengths instead
    {
      Scope sc(tm, name, s);
      HIP_TRY(launch_gemm_bf16(pa, mode, kEpiPartial, p.tile, s));
    }
    if (defer_reduce) return GQA_OK;
    a.splits = p.splits;
    a.partial = part;
    {
      std::string rn = std::string(name) + "_reduce";
      Scope sc(tm, rn.c_str(), s);
      HIP_TRY(launch_splitk_reduce(a, mode, epi, et, s));
    }
    return GQA_OK;
  };

  // Norm steps: the block's kind with a weight (and LayerNorm bias) pair.
  const int nk = c.norm == GQA_NORM_LAYER ? kNormLayer : c.norm == GQA_NORM_RMS_OFFSET ? kNormRmsOffset : kNormRms;
  auto spec = [&](int wi, int bi) {
    return NormSpec{static_cast<const float*>(blk->w[wi]), static_cast<const float*>(blk->w[bi]), nk};
  };
  auto norm = [&](const char* name, NormArgs na) -> int {
    na.d = d;
    na.eps = c.norm_eps;
    Scope sc(tm, name, s);
    HIP_TRY(launch_norm(na, et, T, s));
    return GQA_OK;
  };
  const bool sandwich = c.sandwich_norms != 0;
  const float* o_bias = static_cast<const float*>(blk->w[W_OB]);
  const float* down_bias = static_cast<const float*>(blk->w[W_DB]);

  // 0. (GQA_CHECK_FINITE) non-finite values among the rows' cached keys/values
  if (st && blk->check_finite) {
    Scope sc(tm, "check_cache", s);
    HIP_TRY(launch_cache_nonfinite(st->k, st->v, lengths, et, B, c.n_kv_heads, st->capacity, hd, blk->status + 1, s));
  }
  // 1. input norm (flags non-finite x)
  {
    NormArgs na{};
    na.x = x; na.norm = spec(W_IN_NORM, W_IN_NB); na.out = h; na.flag = blk->status;
    if (int r = norm("rmsnorm", na)) return r;
  }
  // 2. q/k/v projections (+ bias) in one GEMM over three weight segments (a
  // K-split GEMM leaves its partials to the RoPE/append kernel when it can sum them)
  const bool fuse_qkv = bf && lay.p_qkv.splits > 1 && rope_append_fuses_reduce(hd, c.rope_dim, QW + 2 * KW, et);
  {
    GemmArgs a{};
    a.A = h; a.lda = d;
    a.B[0] = blk->w[W_Q]; a.B[1] = blk->w[W_K]; a.B[2] = blk->w[W_V];
    a.seg_end[0] = QW; a.seg_end[1] = QW + KW; a.seg_end[2] = QW + 2 * KW;
    a.bias[0] = static_cast<const float*>(blk->w[W_QB]);
    a.bias[1] = static_cast<const float*>(blk->w[W_KB]);
    a.bias[2] = static_cast<const float*>(blk->w[W_VB]);
    a.M = T; a.N = QW + 2 * KW; a.K = d;
    a.C = qkv; a.ldc = QW + 2 * KW;
    if (int r = gemm("gemm_qkv", a, kModeSeg, kEpiStore, lay.p_qkv, fuse_qkv)) return r;
  }
  // 3. q/k norm + RoPE; keys/values of this call to knew/vnew and into the cache
  // (a windowed call with L > 1 writes the ring after attention instead).  On
  // the matrix-core prefill path with whole-head rotation the attention kernel
  // normalises and rotates q as it loads it, so this step handles k and v only
  // (not for the backward, which reads the rotated q back).
  const char* rq_env = getenv("GQA_ROPE_Q_IN_ATTN");  // tuning override (0: q rotated by the RoPE kernel)
  const bool rope_q_env = !(rq_env && atoi(rq_env) == 0);
  const bool rope_in_attn = rope_q_env && bf && !lay.decode_attn && !recompute_only && !fuse_qkv &&
                            c.rope_dim == hd && hd <= 128 && attention_prefill_bf16_supported(hd, blk->G) &&
                            rope_append_fuses_reduce(hd, c.rope_dim, QW + 2 * KW, et);
  RopeArgs r{};
  {
    r.qkv = qkv; r.ld = QW + 2 * KW;
    r.knew = knew; r.vnew = vnew;
    r.kcache = st ? st->k : nullptr; r.vcache = st ? st->v : nullptr;
    r.lengths = lengths;
    r.cos_tab = blk->cos_tab; r.sin_tab = blk->sin_tab;
    r.q_norm = static_cast<const float*>(blk->w[W_QN]);
    r.k_norm = static_cast<const float*>(blk->w[W_KN]);
    r.B = B; r.L = L; r.H = c.n_heads; r.KV = c.n_kv_heads; r.hd = hd; r.rd = c.rope_dim;
    r.cap = st ? st->capacity : 0; r.window = c.window; r.offset = offset; r.eps = c.norm_eps;
    r.max_pos = c.max_positions; r.pos_flag = blk->status + 2;
    r.defer_append = st && c.window > 0 && L > 1;
    if (pk) {
      r.row_start = pk->row_start;
      r.row_len = pk->row_len;
    }
    r.prows = T;
    r.skip_q = rope_in_attn;
    if (fuse_qkv) {
      r.part = part;
      r.splits = lay.p_qkv.splits;
      r.bias[0] = static_cast<const float*>(blk->w[W_QB]);
      r.bias[1] = static_cast<const float*>(blk->w[W_KB]);
      r.bias[2] = static_cast<const float*>(blk->w[W_VB]);
    }
    Scope sc(tm, "rope_append", s);
    HIP_TRY(launch_rope_append(r, et, s));
  }
  // 4. attention
  {
    AttnArgs a{};
    a.q = qkv; a.ldq = QW + 2 * KW;
    a.knew = knew; a.vnew = vnew;
    a.kcache = st ? st->k : nullptr; a.vcache = st ? st->v : nullptr;
    a.lengths = lengths; a.ctx = ctx;
    a.B = B; a.L = L; a.H = c.n_heads; a.KV = c.n_kv_heads; a.hd = hd;
    a.cap = st ? st->capacity : 0; a.window = c.window; a.softcap = c.attn_softcap;
    a.max_pos = c.max_positions;
    if (bf && lay.decode_attn) {
      a.part = reinterpret_cast<float*>(base + lay.attn_part);
      // equal key segments over the rows' attended keys (host mirror of the
      // lengths; the device recomputes the same split from its own copy)
      int64_t total = 0;
      for (int b = 0; b < B; ++b) {
        const int p = st ? st->lengths[b] : 0;
        total += p + 1 - (c.window > 0 ? std::max(0, p - c.window + 1) : 0);
      }
      a.nseg = attention_decode_segments(total, decode_keys_per_segment());
      a.rec_stride = attention_decode_max_segments() + B;
      {
        Scope sc(tm, "attn_decode", s);
        HIP_TRY(launch_attention_decode_bf16(a, s));
      }
      Scope sc(tm, "attn_combine", s);
      HIP_TRY(launch_attention_decode_combine(a, s));
    } else if (bf && attention_prefill_bf16_supported(hd, blk->G)) {
      a.lse = attn_lse;
      if (rope_in_attn) {
        a.rope_q = 1;
        a.cos_tab = blk->cos_tab; a.sin_tab = blk->sin_tab;
        a.q_norm = static_cast<const float*>(blk->w[W_QN]);
        a.rd = c.rope_dim; a.offset = offset; a.eps = c.norm_eps;
      }
      if (pk) {
        a.row_start = pk->row_start;
        a.row_len = pk->row_len;
      }
      Scope sc(tm, "attn_prefill", s);
      HIP_TRY(launch_attention_prefill_bf16(a, s));
    } else {
      Scope sc(tm, "attn_generic", s);
      HIP_TRY(launch_attention_generic(a, et, s));
    }
  }
  if (r.defer_append) {
    Scope sc(tm, "kv_append", s);
    HIP_TRY(launch_kv_append(r, et, s));
  }
  // 5. o_proj (+ bias) and the residual: x1 = x + ctx Wo^T.  With sandwich
  // norms the projection's output is normalised first (post_attention_layernorm),
  // so the GEMM writes it alone (float32, into y, which is free until step 8)
  // and the norm kernel forms x1.  A K-split decode GEMM leaves its partials
  // to that kernel.
  const bool fuse_o = bf && lay.p_o.splits > 1;
  {
    GemmArgs a{};
    a.A = ctx; a.lda = QW;
    a.B[0] = a.B[1] = a.B[2] = blk->w[W_O];
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = d;
    a.bias[0] = o_bias;
    a.M = T; a.N = d; a.K = QW;
    a.C = sandwich ? y : x1; a.ldc = d; a.resid = sandwich ? nullptr : x; a.ldr = d;
    if (int r = gemm("gemm_o", a, kModeSeg, kEpiResid, lay.p_o, fuse_o)) return r;
  }
  // 6. the MLP's input norm (post_attention_layernorm; pre_feedforward_layernorm
  // with sandwich norms), forming x1 first where step 5 left it undone
  {
    NormArgs na{};
    if (fuse_o) {
      na.part = part; na.splits = lay.p_o.splits; na.bias = o_bias;
    } else {
      na.x = sandwich ? y : x1;
    }
    if (sandwich) na.out_norm = spec(W_POST_NORM, W_POST_NB);
    if (fuse_o || sandwich) {
      na.resid = x; na.x1 = x1;
    }
    na.norm = sandwich ? spec(W_PRE_FF, W_PRE_FFB) : spec(W_POST_NORM, W_POST_NB);
    na.out = h2;
    if (int r = norm(fuse_o || sandwich ? "resid_rmsnorm" : "rmsnorm_post", na)) return r;
  }
  if (recompute_only) return GQA_OK;
  // 7. gate/up (+ biases) and act(gate) * up; ungated MLPs: act(up (+ bias))
  if (mlp_gated(c.mlp)) {
    GemmArgs a{};
    a.A = h2; a.lda = d;
    a.B[0] = blk->w[W_GATE]; a.B[1] = blk->w[W_UP]; a.B[2] = nullptr;
    a.bias[0] = static_cast<const float*>(blk->w[W_GB]);
    a.bias[1] = static_cast<const float*>(blk->w[W_UB]);
    a.M = T; a.N = IT; a.K = d;
    a.C = act; a.ldc = IT;
    a.act = mlp_act(c.mlp);
    if (int r = gemm("gemm_gate_up", a, kModeGated, kEpiGated, lay.p_gu)) return r;
  } else {
    GemmArgs a{};
    a.A = h2; a.lda = d;
    a.B[0] = a.B[1] = a.B[2] = blk->w[W_UP];
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = IT;
    a.bias[0] = a.bias[1] = a.bias[2] = static_cast<const float*>(blk->w[W_UB]);
    a.M = T; a.N = IT; a.K = d;
    a.C = act; a.ldc = IT;
    a.act = mlp_act(c.mlp);
    if (int r = gemm("gemm_up", a, kModeSeg, kEpiStore, lay.p_gu)) return r;
  }
  // 8. down (+ bias) and the residual: y = x1 + act Wd^T; with sandwich norms
  // y = x1 + post_feedforward_layernorm(act Wd^T), the norm kernel reading the
  // GEMM's output (or its K-split partials) from y.  The down GEMM also
  // advances the lengths (no later kernel reads them).
  const bool fuse_down = sandwich && bf && lay.p_down.splits > 1;
  {
    GemmArgs a{};
    a.A = act; a.lda = IT;
    a.B[0] = a.B[1] = a.B[2] = blk->w[W_DOWN];
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = d;
    a.bias[0] = down_bias;
    a.M = T; a.N = d; a.K = IT;
    a.C = y; a.ldc = d; a.resid = sandwich ? nullptr : x1; a.ldr = d;
    if (st) { a.bump = lengths; a.bump_n = B; a.bump_by = L; }
    if (int r = gemm("gemm_down", a, kModeSeg, kEpiResid, lay.p_down, fuse_down)) return r;
  }
  if (sandwich) {
    NormArgs na{};
    if (fuse_down) {
      na.part = part; na.splits = lay.p_down.splits; na.bias = down_bias;
    } else {
      na.x = y;
    }
    na.out_norm = spec(W_POST_FF, W_POST_FFB);
    na.resid = x1; na.x1 = y;
    if (int r = norm("resid_norm_out", na)) return r;
  }
  if (st)
    for (int b = 0; b < B; ++b) st->lengths[b] += L;
  return GQA_OK;
}

// ---- backward of a zero-state prefill ----

// mojolearn TransformerBlock.backward: the default block options only (the
// window is honoured).
bool backward_supported(const gqa_block_config& c) {
  return c.norm == GQA_NORM_RMS && c.mlp == GQA_MLP_SWIGLU && !c.qkv_bias && !c.qk_norm && c.attn_softcap == 0.f &&
         !c.o_bias && !c.mlp_bias && !c.norm_bias && !c.sandwich_norms && c.rope_scaling == GQA_ROPE_PLAIN &&
         c.rope_dim == c.head_dim;
}

// Backward products that read K-major operands in place (the pipelined
// kernel's transposed-operand mode, 256x256 tiles): the input-gradient
// products take the weights [out, in] as they are (tr_dx), the
// weight-gradient products take the activations and their gradients
// [tokens, features] as they are, K = tokens (tr_dw).  Otherwise those
// operands are first transposed into K-contiguous copies.
bool bwd_trans_dx(const gqa_block* blk, int T) {
  const auto& c = blk->cfg;
  const int d = c.d_model, IT = c.intermediate, QW = blk->QW, KW = blk->KW;
  for (int i : {W_DOWN, W_GATE, W_UP, W_O, W_Q, W_K, W_V})
    if (reinterpret_cast<uintptr_t>(blk->w[i]) % 16 != 0) return false;
  return is_bf16(blk) && T > 512 && gemm_dma_tile(plan_gemm(T, d, 2 * IT, false).tile) && d % 8 == 0 &&
         IT % 64 == 0 && QW % 64 == 0 && KW % 64 == 0;
}
bool bwd_trans_dw(const gqa_block* blk, int T) {
  const auto& c = blk->cfg;
  const int d = c.d_model, IT = c.intermediate, QW = blk->QW, KW = blk->KW;
  return is_bf16(blk) && T >= 256 && T % 64 == 0 && d % 8 == 0 && IT % 8 == 0 && QW % 8 == 0 && KW % 8 == 0;
}
// K splits of a transposed-operand product: enough to bring a small grid of
// 256x256 tiles near the CU count, keeping each split 64-aligned and at least
// 256 deep.
int trans_splits(int M, int N, int K) {
  const long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
  int sp = 1;
  while (sp < 8 && tiles * sp < 192 && K % (128 * sp) == 0 && K / (2 * sp) >= 256) sp *= 2;
  return sp;
}

// Plan of a backward product on K-contiguous operands: the forward's plan,
// except that a grid of 256x256 tiles well short of the 256 CUs (the k/v
// weight gradients: 64 tiles) takes 128x128 tiles instead.
GemmPlan bwd_gemm_plan(int M, int N, int K) {
  GemmPlan p = plan_gemm(M, N, K, false);
  if (gemm_dma_tile(p.tile) && (long)((M + 255) / 256) * ((N + 255) / 256) < 192) p = GemmPlan{kTile128x128, 1, 0};
  return p;
}

struct BwdLayout {
  WsLayout fwd;  // the recomputed forward's workspace, at offset 0
  bool tr_dx, tr_dw;
  bool fuse_swiglu;  // SwiGLU's backward in the epilogue of the da product (no da buffer)
  size_t y, gu, lse, dsum, wdT, wguT, woT, wqkvT, dy_op, dyT, da, act, actT, dgu, dguT, h2T, dh2, dx1, dx1_op, dx1T,
      wpart, cpart, ctxT, dctx, dq, dk, dv, dob, dqkv, dqkvT, hT, dh, part, total;
  int Tp;  // token count padded to 256: the depth of the weight-gradient GEMMs
  int Kq;  // q | k | v width padded to 64: the depth of the dh GEMM
};

BwdLayout bwd_layout_for(const gqa_block* blk, int B, int L) {
  const auto& c = blk->cfg;
  BwdLayout w{};
  w.fwd = layout_for(blk, B, L);
  size_t off = w.fwd.total;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  const size_t T = (size_t)B * L, es = blk->es;
  const size_t d = c.d_model, QW = blk->QW, KW = blk->KW, IT = c.intermediate, H = c.n_heads;
  w.Tp = (int)((T + 255) / 256 * 256);
  w.Kq = (int)((QW + 2 * KW + 63) / 64 * 64);
  w.tr_dx = bwd_trans_dx(blk, (int)T);
  w.tr_dw = bwd_trans_dw(blk, (int)T);
  w.fuse_swiglu = w.tr_dx && trans_splits((int)T, (int)IT, (int)d) == 1;
  const bool cx = !w.tr_dx, cw = !w.tr_dw;  // transposed copies needed
  const size_t Tp = w.Tp, Kq = w.Kq;
  w.y = take(T * d * 4);
  w.gu = take(T * 2 * IT * 4);
  const size_t lse_n = (size_t)B * H * (((size_t)L + 3) & ~(size_t)3);  // [B, H, L padded to 4] (>= T * H)
  w.lse = take(lse_n * 4);
  w.dsum = take(lse_n * 4);
  w.wdT = cx ? take(IT * d * es) : 0;
  w.wguT = cx ? take(d * 2 * IT * es) : 0;
  w.woT = cx ? take(QW * d * es) : 0;
  w.wqkvT = cx ? take(d * Kq * es) : 0;
  w.dy_op = take(T * d * es);
  w.dyT = cw ? take(d * Tp * es) : 0;
  w.da = w.fuse_swiglu ? 0 : take(T * IT * 4);
  w.act = take(T * IT * es);
  w.actT = cw ? take(IT * Tp * es) : 0;
  w.dgu = take(T * 2 * IT * es);
  w.dguT = cw ? take(2 * IT * Tp * es) : 0;
  w.h2T = cw ? take(d * Tp * es) : 0;
  w.dh2 = take(T * d * 4);
  w.dx1 = take(T * d * 4);
  w.dx1_op = take(T * d * es);
  w.dx1T = cw ? take(d * Tp * es) : 0;
  const int wparts = rms_bwd_parts((int)T, (int)d);  // RMSNorm weight-gradient partial rows
  w.wpart = take((size_t)wparts * d * 4);
  w.cpart = take((size_t)colsum_chunks(wparts) * d * 4);
  w.ctxT = cw ? take(QW * Tp * es) : 0;
  w.dctx = take(T * QW * 4);
  w.dq = take(T * QW * 4);
  const size_t parts = (size_t)blk->G;  // per-head partials of the matrix-core path
  w.dk = take(parts * T * KW * 4);
  w.dv = take(parts * T * KW * 4);
  w.dob = take(T * QW * 2);
  w.dqkv = take(T * Kq * es);
  w.dqkvT = cw ? take(Kq * Tp * es) : 0;
  w.hT = cw ? take(d * Tp * es) : 0;
  w.dh = take(T * d * 4);
  size_t part = 0;  // K-split partials of any product whose plan splits
  if (is_bf16(blk)) {
    auto need = [&](size_t M, size_t N, size_t K) {
      const GemmPlan p = plan_gemm((int)M, (int)N, (int)K, false);
      if (p.splits > 1) part = std::max(part, (size_t)p.splits * M * N * 4);
    };
    auto need_t = [&](size_t M, size_t N, size_t K) {
      const int sp = trans_splits((int)M, (int)N, (int)K);
      if (sp > 1) part = std::max(part, (size_t)sp * M * N * 4);
    };
    auto dx = [&](size_t M, size_t N, size_t K) { w.tr_dx ? need_t(M, N, K) : need(M, N, K); };
    auto dw = [&](size_t M, size_t N) { w.tr_dw ? need_t(M, N, T) : need(M, N, Tp); };
    dx(T, IT, d);         // da
    dw(d, IT);            // dWd
    dx(T, d, 2 * IT);     // dh2
    dw(IT, d);            // dWg, dWu
    dx(T, QW, d);         // dctx
    dw(d, QW);            // dWo
    dx(T, d, Kq);         // dh
    dw(QW, d);            // dWq
    dw(KW, d);            // dWk, dWv
    need(T, IT, d);       // gate / up of the recompute
  }
  w.part = part ? take(part) : 0;
  w.total = off;
  return w;
}

int run_backward(gqa_block* blk, const float* x, const float* dy, float* dx, float* const* dw, int B, int L, void* ws,
                 size_t wsb, hipStream_t s) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  const auto& c = blk->cfg;
  if (!backward_supported(c))
    return fail(GQA_ERR_UNSUPPORTED, "backward supports the default block options only (RMSNorm, SwiGLU, no "
                                     "biases, q/k norm, softcap, RoPE scaling, partial rotary or sandwich norms)");
  if (B < 0 || L < 0) return fail(GQA_ERR_ARG, "B and L must be >= 0");
  if (L > c.max_positions)
    return fail(GQA_ERR_POSITION, "position %d is at or beyond max_positions %d", L - 1, c.max_positions);
  if (B == 0 || L == 0) return GQA_OK;
  if (!x || !dy || !dx || !dw) return fail(GQA_ERR_ARG, "x, grad_output, grad_x or the gradient table is NULL");
  for (int i = 0; i < 9; ++i)
    if (!dw[i]) return fail(GQA_ERR_ARG, "gradient %d (%s) is NULL", i, kNames[i]);
  const BwdLayout lay = bwd_layout_for(blk, B, L);
  if (!ws || wsb < lay.total)
    return fail(GQA_ERR_WORKSPACE, "workspace of %zu bytes given, %zu needed", ws ? wsb : (size_t)0, lay.total);

  BusyGuard guard(blk->busy);
  if (!guard.ok) return fail(GQA_ERR_BUSY, "block is in use by another call");
  char* base = static_cast<char*>(ws);
  float* y = reinterpret_cast<float*>(base + lay.y);
  // 0. forward from an empty cache (positions 0 .. L-1), leaving its activations
  // (and, on the matrix-core attention path, each row's log-sum-exp)
  const bool mfma_attn = is_bf16(blk) && !lay.fwd.decode_attn &&
                         attention_prefill_bf16_supported(c.head_dim, blk->G) &&
                         attention_bwd_mfma_supported(c.head_dim, blk->G);
  if (int r = run_block(blk, nullptr, x, y, B, L, ws, lay.fwd.total, s,
                        mfma_attn ? reinterpret_cast<float*>(base + lay.lse) : nullptr, true))
    return r;

  const int T = B * L, d = c.d_model, QW = blk->QW, KW = blk->KW, IT = c.intermediate, H = c.n_heads;
  const int Tp = lay.Tp, Kq = lay.Kq;
  const bool bf = is_bf16(blk);
  const int et = bf ? kBF16 : kF32;
  const size_t es = blk->es;
  KernelTimer* tm = &blk->timer;
  auto at = [&](size_t off) { return static_cast<void*>(base + off); };
  auto atf = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  const void* h = at(lay.fwd.h);
  const void* qkv = at(lay.fwd.qkv);
  const void* ctx = at(lay.fwd.ctx);
  const float* x1 = atf(lay.fwd.x1);
  const void* h2 = at(lay.fwd.h2);
  float* part = lay.part ? atf(lay.part) : nullptr;
  auto sub = [&](const void* p, size_t elems) { return static_cast<const void*>(static_cast<const char*>(p) + elems * es); };

  // C[M, N] (float32, row stride ldc) = A[M, K] B[N, K]^T: the forward's GEMMs,
  // K-split when their plan says so (partials summed in split order)
  auto gemm = [&](const char* name, const void* A, int64_t lda, const void* Bm, int M, int N, int K, float* C,
                  int64_t ldc) -> int {
    GemmArgs a{};
    a.A = A; a.lda = lda;
    a.B[0] = a.B[1] = a.B[2] = Bm;
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = N;
    a.M = M; a.N = N; a.K = K;
    a.C = C; a.ldc = ldc;
    a.order = gemm_tile_order();
    Scope sc(tm, name, s);
    if (!bf) {
      HIP_TRY(launch_gemm_f32(a, kModeSeg, kEpiResid, s));
      return GQA_OK;
    }
    const GemmPlan p = bwd_gemm_plan(M, N, K);
    a.wg_waves = p.waves;
    if (p.splits <= 1) {
      a.splits = 1;
      a.k_split = K;
      HIP_TRY(launch_gemm_bf16(a, kModeSeg, kEpiResid, p.tile, s));
      return GQA_OK;
    }
    GemmArgs pa = a;
    pa.splits = p.splits;
    pa.k_split = K / p.splits;
    pa.partial = part;
    HIP_TRY(launch_gemm_bf16(pa, kModeSeg, kEpiPartial, p.tile, s));
    a.splits = p.splits;
    a.partial = part;
    HIP_TRY(launch_splitk_reduce(a, kModeSeg, kEpiResid, kF32, s));
    return GQA_OK;
  };
  // C[M, N] (float32) = A B^T with B given K-major (B^T[K, N], row stride ldb,
  // rows from up to three segments b0 | b1 | b2 ending at K rows e0, e1, e2)
  // and A given K-major too when ta (A^T[K, M], row stride lda)
  auto gemm_t = [&](const char* name, const void* A, int64_t lda, bool ta, const void* b0, const void* b1,
                    const void* b2, int64_t e0, int64_t e1, int64_t e2, int64_t ldb, int M, int N, int K, float* C,
                    int64_t ldc) -> int {
    GemmArgs a{};
    a.A = A; a.lda = lda;
    a.B[0] = b0; a.B[1] = b1; a.B[2] = b2;
    a.seg_end[0] = e0; a.seg_end[1] = e1; a.seg_end[2] = e2;
    a.ldb = ldb;
    a.trans = (ta ? 1 : 0) | 2;
    a.M = M; a.N = N; a.K = K;
    a.C = C; a.ldc = ldc;
    a.order = gemm_tile_order();
    Scope sc(tm, name, s);
    const int sp = trans_splits(M, N, K);
    if (sp <= 1) {
      a.splits = 1;
      a.k_split = K;
      HIP_TRY(launch_gemm_bf16(a, kModeSeg, kEpiResid, kTileDma256x256, s));
      return GQA_OK;
    }
    GemmArgs pa = a;
    pa.splits = sp;
    pa.k_split = K / sp;
    pa.partial = part;
    HIP_TRY(launch_gemm_bf16(pa, kModeSeg, kEpiPartial, kTileDma256x256, s));
    a.splits = sp;
    a.partial = part;
    HIP_TRY(launch_splitk_reduce(a, kModeSeg, kEpiResid, kF32, s));
    return GQA_OK;
  };
  auto tr = [&](const char* name, const void* in, int in_t, int64_t ld, int R, int C, void* out, int64_t ldo,
                int Rp) -> int {
    Scope sc(tm, name, s);
    HIP_TRY(launch_transpose(in, in_t, ld, R, C, out, et, ldo, Rp, s));
    return GQA_OK;
  };
#define BWD(expr) \
  do {            \
    if (int r_ = (expr)) return r_; \
  } while (0)

  // 1. gate and up pre-activations of the recomputed forward (float32, gate | up
  // per row): one gated GEMM whose single-split partial epilogue writes exactly
  // that layout, else two plain products
  float* gu = atf(lay.gu);
  const GemmPlan pgu = bf ? plan_gemm(T, IT, d, true) : GemmPlan{0, 0, 0};
  if (bf && pgu.tile != kTileSkinny) {
    GemmArgs a{};
    a.A = h2; a.lda = d;
    a.B[0] = blk->w[W_GATE]; a.B[1] = blk->w[W_UP]; a.B[2] = nullptr;
    a.M = T; a.N = IT; a.K = d;
    a.splits = 1; a.k_split = d; a.partial = gu;
    a.order = gemm_tile_order();
    Scope sc(tm, "bwd_gate_up", s);
    HIP_TRY(launch_gemm_bf16(a, kModeGated, kEpiPartial, pgu.tile, s));
  } else {
    BWD(gemm("bwd_gate", h2, d, blk->w[W_GATE], T, IT, d, gu, 2 * IT));
    BWD(gemm("bwd_up", h2, d, blk->w[W_UP], T, IT, d, gu + IT, 2 * IT));
  }
  // 2. weights as the other product operand (transposed, K-contiguous)
  void* wdT = at(lay.wdT);
  void* wguT = at(lay.wguT);
  void* woT = at(lay.woT);
  void* wqkvT = at(lay.wqkvT);
  if (!lay.tr_dx) {
    BWD(tr("bwd_transpose_w", blk->w[W_DOWN], et, IT, d, IT, wdT, d, d));
    BWD(tr("bwd_transpose_w", blk->w[W_GATE], et, d, IT, d, wguT, 2 * IT, IT));
    BWD(tr("bwd_transpose_w", blk->w[W_UP], et, d, IT, d, static_cast<char*>(wguT) + (size_t)IT * es, 2 * IT, IT));
    BWD(tr("bwd_transpose_w", blk->w[W_O], et, QW, d, QW, woT, d, d));
    BWD(tr("bwd_transpose_w", blk->w[W_Q], et, d, QW, d, wqkvT, Kq, QW));
    BWD(tr("bwd_transpose_w", blk->w[W_K], et, d, KW, d, static_cast<char*>(wqkvT) + (size_t)QW * es, Kq, KW));
    BWD(tr("bwd_transpose_w", blk->w[W_V], et, d, KW, d, static_cast<char*>(wqkvT) + (size_t)(QW + KW) * es, Kq,
           Kq - QW - KW));
  }
  // weight gradient dW[M, N] = sum over tokens of g[t, m] x[t, n]: g and x
  // read in place when tr_dw, else from their transposed copies
  auto gemm_dw = [&](const void* g, int64_t ldg, const void* gT, const void* xx, int64_t ldx, const void* xT, int M,
                     int N, float* C) -> int {
    if (lay.tr_dw) return gemm_t("bwd_gemm_dw", g, ldg, true, xx, xx, xx, T, T, T, ldx, M, N, T, C, N);
    return gemm("bwd_gemm_dw", gT, Tp, xT, M, N, Tp, C, N);
  };
  // 3. down: da = dy Wd, dWd = dy^T a
  const void* dy_op = dy;
  if (bf) {
    Scope sc(tm, "bwd_convert", s);
    HIP_TRY(launch_convert(dy, at(lay.dy_op), et, (int64_t)T * d, s));
    dy_op = at(lay.dy_op);
  }
  void* dyT = at(lay.dyT);
  if (!lay.tr_dw) BWD(tr("bwd_transpose", dy, kF32, d, T, d, dyT, Tp, Tp));
  // 4. SwiGLU: a = silu(g) u (for dWd), dg | du -- in the da product's
  // epilogue when it runs as one K split on the pipelined kernel
  void* act = at(lay.act);
  void* dgu = at(lay.dgu);
  if (lay.fuse_swiglu) {
    const void* wd = blk->w[W_DOWN];
    GemmArgs a{};
    a.A = dy_op; a.lda = d;
    a.B[0] = a.B[1] = a.B[2] = wd;
    a.seg_end[0] = a.seg_end[1] = a.seg_end[2] = d;
    a.ldb = IT;
    a.trans = 2;
    a.M = T; a.N = IT; a.K = d;
    a.splits = 1; a.k_split = d;
    a.resid = gu; a.ldr = 2 * (int64_t)IT;
    a.C = act; a.ldc = IT;
    a.C2 = dgu; a.ldc2 = 2 * (int64_t)IT;
    a.order = gemm_tile_order();
    Scope sc(tm, "bwd_gemm_da_swiglu", s);
    HIP_TRY(launch_gemm_bf16(a, kModeSeg, kEpiSwigluBwd, kTileDma256x256, s));
  } else {
    float* da = atf(lay.da);
    if (lay.tr_dx) {
      const void* wd = blk->w[W_DOWN];
      BWD(gemm_t("bwd_gemm_da", dy_op, d, false, wd, wd, wd, d, d, d, IT, T, IT, d, da, IT));
    } else {
      BWD(gemm("bwd_gemm_da", dy_op, d, wdT, T, IT, d, da, IT));
    }
    Scope sc(tm, "bwd_swiglu", s);
    HIP_TRY(launch_swiglu_bwd(gu, da, T, IT, act, dgu, et, s));
  }
  void* actT = at(lay.actT);
  if (!lay.tr_dw) BWD(tr("bwd_transpose", act, et, IT, T, IT, actT, Tp, Tp));
  BWD(gemm_dw(dy_op, d, dyT, act, IT, actT, d, IT, dw[8]));
  // 5. gate / up: dh2 = dg Wg + du Wu, dWg = dg^T h2, dWu = du^T h2
  float* dh2 = atf(lay.dh2);
  if (lay.tr_dx)
    BWD(gemm_t("bwd_gemm_dh2", dgu, 2 * IT, false, blk->w[W_GATE], blk->w[W_UP], blk->w[W_UP], IT, 2 * IT, 2 * IT,
               d, T, d, 2 * IT, dh2, d));
  else
    BWD(gemm("bwd_gemm_dh2", dgu, 2 * IT, wguT, T, d, 2 * IT, dh2, d));
  void* dguT = at(lay.dguT);
  void* h2T = at(lay.h2T);
  if (!lay.tr_dw) {
    BWD(tr("bwd_transpose", dgu, et, 2 * IT, T, 2 * IT, dguT, Tp, Tp));
    BWD(tr("bwd_transpose", h2, et, d, T, d, h2T, Tp, Tp));
  }
  BWD(gemm_dw(dgu, 2 * IT, dguT, h2, d, h2T, IT, d, dw[6]));
  BWD(gemm_dw(sub(dgu, IT), 2 * IT, lay.tr_dw ? nullptr : sub(dguT, (size_t)IT * Tp), h2, d, h2T, IT, d, dw[7]));
  // 6. post-attention RMSNorm backward + the residual: dx1 = dy + norm'(dh2)
  float* dx1 = atf(lay.dx1);
  void* dx1_op = bf ? at(lay.dx1_op) : static_cast<void*>(dx1);
  float* wpart = atf(lay.wpart);
  {
    Scope sc(tm, "bwd_norm", s);
    HIP_TRY(launch_rms_bwd(dh2, x1, static_cast<const float*>(blk->w[W_POST_NORM]), dy, T, d, c.norm_eps, dx1,
                           bf ? dx1_op : nullptr, et, wpart, s));
    HIP_TRY(launch_colsum(wpart, rms_bwd_parts(T, d), d, atf(lay.cpart), dw[1], s));
  }
  // 7. o_proj: dctx = dx1 Wo, dWo = dx1^T ctx
  float* dctx = atf(lay.dctx);
  if (lay.tr_dx) {
    const void* wo = blk->w[W_O];
    BWD(gemm_t("bwd_gemm_dctx", dx1_op, d, false, wo, wo, wo, d, d, d, QW, T, QW, d, dctx, QW));
  } else {
    BWD(gemm("bwd_gemm_dctx", dx1_op, d, woT, T, QW, d, dctx, QW));
  }
  void* dx1T = at(lay.dx1T);
  void* ctxT = at(lay.ctxT);
  if (!lay.tr_dw) {
    BWD(tr("bwd_transpose", dx1, kF32, d, T, d, dx1T, Tp, Tp));
    BWD(tr("bwd_transpose", ctx, et, QW, T, QW, ctxT, Tp, Tp));
  }
  BWD(gemm_dw(dx1_op, d, dx1T, ctx, QW, ctxT, d, QW, dw[5]));
  // 8. attention, then RoPE's backward, packed as the q/k/v GEMM's rows
  BwdAttnArgs ba{};
  ba.q = qkv; ba.ldq = QW + 2 * KW;
  ba.k = at(lay.fwd.knew); ba.v = at(lay.fwd.vnew);
  ba.o = ctx; ba.ldo = QW;
  ba.dout = dctx;
  ba.lse = atf(lay.lse); ba.dsum = atf(lay.dsum);
  ba.dq = atf(lay.dq); ba.dk = atf(lay.dk); ba.dv = atf(lay.dv);
  ba.cos_tab = blk->cos_tab; ba.sin_tab = blk->sin_tab;
  ba.B = B; ba.L = L; ba.H = H; ba.KV = c.n_kv_heads; ba.hd = c.head_dim; ba.window = c.window;
  ba.scale = 1.0f / std::sqrt((float)c.head_dim);
  ba.lse_ld = (L + 3) & ~3;
  ba.kv_parts = mfma_attn ? blk->G : 1;
  ba.kv_part_stride = (int64_t)T * KW;
  {
    Scope sc(tm, "bwd_attention", s);
    if (mfma_attn)
      HIP_TRY(launch_attention_bwd_mfma(ba, at(lay.dob), s));
    else
      HIP_TRY(launch_attention_bwd(ba, et, s));
  }
  void* dqkv = at(lay.dqkv);
  {
    Scope sc(tm, "bwd_rope", s);
    HIP_TRY(launch_rope_bwd_pack(ba, dqkv, Kq, et, s));
  }
  // 9. q/k/v: dh = [dq|dk|dv] [Wq;Wk;Wv], dW = d^T h
  float* dh = atf(lay.dh);
  if (lay.tr_dx)
    BWD(gemm_t("bwd_gemm_dh", dqkv, Kq, false, blk->w[W_Q], blk->w[W_K], blk->w[W_V], QW, QW + KW, QW + 2 * KW, d,
               T, d, Kq, dh, d));
  else
    BWD(gemm("bwd_gemm_dh", dqkv, Kq, wqkvT, T, d, Kq, dh, d));
  void* dqkvT = at(lay.dqkvT);
  void* hT = at(lay.hT);
  if (!lay.tr_dw) {
    BWD(tr("bwd_transpose", dqkv, et, Kq, T, Kq, dqkvT, Tp, Tp));
    BWD(tr("bwd_transpose", h, et, d, T, d, hT, Tp, Tp));
  }
  const bool tw = lay.tr_dw;
  BWD(gemm_dw(dqkv, Kq, dqkvT, h, d, hT, QW, d, dw[2]));
  BWD(gemm_dw(sub(dqkv, QW), Kq, tw ? nullptr : sub(dqkvT, (size_t)QW * Tp), h, d, hT, KW, d, dw[3]));
  BWD(gemm_dw(sub(dqkv, (size_t)QW + KW), Kq, tw ? nullptr : sub(dqkvT, (size_t)(QW + KW) * Tp), h, d, hT, KW, d,
              dw[4]));
  // 10. input RMSNorm backward + the residual: dx = dx1 + norm'(dh)
  {
    Scope sc(tm, "bwd_norm", s);
    HIP_TRY(launch_rms_bwd(dh, x, static_cast<const float*>(blk->w[W_IN_NORM]), dx1, T, d, c.norm_eps, dx, nullptr,
                           et, wpart, s));
    HIP_TRY(launch_colsum(wpart, rms_bwd_parts(T, d), d, atf(lay.cpart), dw[0], s));
  }
#undef BWD
  return GQA_OK;
}

// Text description of the launch plan (see gqa_block_describe_plan).
std::string describe_plan(const gqa_block* blk, int kind, int B, int L) {
  const auto& c = blk->cfg;
  std::string out;
  char line[160];
  auto add = [&](const char* fmt, auto... v) {
    snprintf(line, sizeof line, fmt, v...);
    out += line;
    out += '\n';
  };
  const int T = B * L, d = c.d_model, QW = blk->QW, KW = blk->KW, IT = c.intermediate;
  const bool bf = is_bf16(blk);
  add("dtype=%s", bf ? "bf16" : "f32");
  if (kind == 0) {
    const WsLayout lay = layout_for(blk, B, L);
    auto g = [&](const char* name, const GemmPlan& p) {
      if (bf && p.tail_splits > 1 && p.n1 > 0)
        add("%s tile=%d splits=%d waves=%d tail_cols_from=%d tail_splits=%d", name, p.tile, p.splits, p.waves, p.n1,
            p.tail_splits);
      else if (bf && p.tail_splits > 1)
        add("%s tile=%d splits=%d waves=%d tail_rows_from=%d tail_splits=%d", name, p.tile, p.splits, p.waves, p.m1,
            p.tail_splits);
      else if (bf) add("%s tile=%d splits=%d waves=%d", name, p.tile, p.splits, p.waves);
      else add("%s f32", name);
    };
    g("gemm_qkv", lay.p_qkv);
    g("gemm_o", lay.p_o);
    g(mlp_gated(c.mlp) ? "gemm_gate_up" : "gemm_up", lay.p_gu);
    g("gemm_down", lay.p_down);
    add("attention=%s", bf && lay.decode_attn ? "decode_splitk"
                        : bf && attention_prefill_bf16_supported(c.head_dim, blk->G) ? "prefill_mfma" : "generic");
    add("workspace=%zu", lay.total);
    return out;
  }
  const BwdLayout lay = bwd_layout_for(blk, B, L);
  const bool mfma_attn = bf && !lay.fwd.decode_attn && attention_prefill_bf16_supported(c.head_dim, blk->G) &&
                         attention_bwd_mfma_supported(c.head_dim, blk->G);
  add("tr_dx=%d tr_dw=%d fuse_swiglu=%d mfma_attention=%d", lay.tr_dx, lay.tr_dw, lay.fuse_swiglu, mfma_attn);
  if (!bf) return out;
  const GemmPlan pgu = plan_gemm(T, IT, d, true);
  add("bwd_gate_up tile=%d", pgu.tile);
  const int Tp = lay.Tp, Kq = lay.Kq;
  auto dx = [&](const char* name, int M, int N, int K) {
    if (lay.tr_dx) add("%s transposed tile=%d splits=%d", name, (int)kTileDma256x256, trans_splits(M, N, K));
    else {
      const GemmPlan p = bwd_gemm_plan(M, N, K);
      add("%s tile=%d splits=%d", name, p.tile, p.splits);
    }
  };
  auto dw = [&](const char* name, int M, int N) {
    if (lay.tr_dw) add("%s transposed tile=%d splits=%d", name, (int)kTileDma256x256, trans_splits(M, N, T));
    else {
      const GemmPlan p = bwd_gemm_plan(M, N, Tp);
      add("%s tile=%d splits=%d", name, p.tile, p.splits);
    }
  };
  if (lay.fuse_swiglu) add("da_swiglu transposed tile=%d splits=1", (int)kTileDma256x256);
  else dx("da", T, IT, d);
  dw("dWd", d, IT);
  dx("dh2", T, d, 2 * IT);
  dw("dWg_dWu", IT, d);
  dx("dctx", T, QW, d);
  dw("dWo", d, QW);
  dx("dh", T, d, Kq);
  dw("dWq", QW, d);
  dw("dWk_dWv", KW, d);
  return out;
}

}  // namespace

namespace gqa_host {
// Sets the calling thread's last-error text (for the library's other entry
// points compiled in other files) and returns `code`.
int report(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return fail(code, "%s", buf);
}
}  // namespace gqa_host

extern "C" {

const char* gqa_last_error(void) { return g_last_error.c_str(); }
const char* gqa_version(void) { return "gqa_block 0.1 (gfx950)"; }

int gqa_block_create(const gqa_block_config* cfg, const gqa_tensor* weights, int32_t n_weights, gqa_block** out) {
  if (!out) return fail(GQA_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (int r = check_config(cfg)) return r;
  const void* wp[W_COUNT];
  if (int r = check_weights(cfg, weights, n_weights, wp)) return r;

  gqa_block* blk = new gqa_block();
  blk->cfg = *cfg;
  for (int i = 0; i < W_COUNT; ++i) blk->w[i] = wp[i];
  blk->QW = cfg->n_heads * cfg->head_dim;
  blk->KW = cfg->n_kv_heads * cfg->head_dim;
  blk->G = cfg->n_heads / cfg->n_kv_heads;
  blk->es = cfg->weight_dtype == GQA_BF16 ? 2 : 4;

  auto cleanup = [&](int code) {
    gqa_block_destroy(blk);
    return code;
  };
  // RoPE table: angle p * theta_i and its cos/sin in double, stored as float32
  // [max_positions, rope_dim/2].
  if (blk->cfg.rope_dim == 0) blk->cfg.rope_dim = cfg->head_dim;
  const int half = blk->cfg.rope_dim / 2;
  const size_t n = (size_t)cfg->max_positions * half;
  std::vector<float> ct(n), sn(n);
  const std::vector<double> inv = rope_frequencies(blk->cfg);
  for (int p = 0; p < cfg->max_positions; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * inv[i];
      ct[(size_t)p * half + i] = (float)std::cos(a);
      sn[(size_t)p * half + i] = (float)std::sin(a);
    }
  hipError_t e;
  if ((e = hipMalloc(&blk->cos_tab, n * 4)) != hipSuccess || (e = hipMalloc(&blk->sin_tab, n * 4)) != hipSuccess ||
      (e = hipMalloc(&blk->status, kStatusWords * 4)) != hipSuccess)
    return cleanup(fail(GQA_ERR_HIP, "device allocation failed: %s", hipGetErrorString(e)));
  if ((e = hipMemcpy(blk->cos_tab, ct.data(), n * 4, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemcpy(blk->sin_tab, sn.data(), n * 4, hipMemcpyHostToDevice)) != hipSuccess ||
      (e = hipMemset(blk->status, 0, kStatusWords * 4)) != hipSuccess)
    return cleanup(fail(GQA_ERR_HIP, "device copy failed: %s", hipGetErrorString(e)));
  {
    // GQA_CHECK_FINITE=1: count non-finite cached keys/values at every call
    // with a state (a debug option: it reads each row's used cache once more)
    const char* cf = getenv("GQA_CHECK_FINITE");
    blk->check_finite = cf && atoi(cf) != 0;
  }

  // Non-finite weights are refused before any computation.
  const int64_t d = cfg->d_model, hd = cfg->head_dim, QW = blk->QW, KW = blk->KW, IT = cfg->intermediate;
  const int64_t counts[W_COUNT] = {d, d, QW * d, KW * d, KW * d, d * QW, IT * d, IT * d, d * IT, QW, KW, KW, hd, hd,
                                   d, IT, IT, d, d, d, d, d, d, d};
  for (int i = 0; i < W_COUNT; ++i) {
    if (!blk->w[i]) continue;
    const bool matrix = i >= W_Q && i <= W_DOWN;
    const int elem = matrix && cfg->weight_dtype == GQA_BF16 ? kBF16 : kF32;
    if ((e = launch_count_nonfinite(blk->w[i], elem, counts[i], blk->status, nullptr)) != hipSuccess)
      return cleanup(fail(GQA_ERR_HIP, "weight check launch failed: %s", hipGetErrorString(e)));
  }
  int flag = 0;
  if ((e = hipMemcpy(&flag, blk->status, 4, hipMemcpyDeviceToHost)) != hipSuccess)
    return cleanup(fail(GQA_ERR_HIP, "weight check failed: %s", hipGetErrorString(e)));
  if (flag) return cleanup(fail(GQA_ERR_NONFINITE, "a weight holds a non-finite value"));
  *out = blk;
  return GQA_OK;
}

void gqa_block_destroy(gqa_block* blk) {
  if (!blk) return;
  blk->timer.collect();
  if (blk->cos_tab) hipFree(blk->cos_tab);
  if (blk->sin_tab) hipFree(blk->sin_tab);
  if (blk->status) hipFree(blk->status);
  delete blk;
}

int gqa_state_bytes(const gqa_block* blk, int32_t batch, int32_t max_tokens, size_t* bytes) {
  if (!blk || !bytes) return fail(GQA_ERR_ARG, "block or output is NULL");
  if (batch <= 0 || max_tokens <= 0) return fail(GQA_ERR_ARG, "batch and max_tokens must be positive");
  const int cap = blk->cfg.window > 0 ? blk->cfg.window : max_tokens;
  *bytes = (size_t)batch * blk->cfg.n_kv_heads * cap * blk->cfg.head_dim * blk->es;
  return GQA_OK;
}

int gqa_block_allocate_state(const gqa_block* blk, int32_t batch, int32_t max_tokens, void* k, void* v,
                             int32_t* lengths_dev, gqa_state** out) {
  if (!out) return fail(GQA_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  if (batch <= 0 || max_tokens <= 0) return fail(GQA_ERR_ARG, "batch and max_tokens must be positive");
  if (!k || !v || !lengths_dev) return fail(GQA_ERR_ARG, "state buffers must not be NULL");
  gqa_state* st = new gqa_state();
  st->blk = blk;
  st->batch = batch;
  st->max_tokens = max_tokens;
  st->capacity = blk->cfg.window > 0 ? blk->cfg.window : max_tokens;
  st->k = k;
  st->v = v;
  st->lengths_dev = lengths_dev;
  st->lengths.assign(batch, 0);
  hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&st->staging), (size_t)gqa_state::kRing * batch * 4,
                               hipHostMallocDefault);
  if (e != hipSuccess) {
    st->staging = nullptr;
    delete st;
    return fail(GQA_ERR_HIP, "pinned staging allocation failed: %s", hipGetErrorString(e));
  }
  for (auto& ev : st->done) {
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
      ev = nullptr;
      delete st;
      return fail(GQA_ERR_HIP, "event creation failed: %s", hipGetErrorString(e));
    }
  }
  *out = st;
  return GQA_OK;
}

int gqa_state_set_lengths(gqa_state* st, const int32_t* lengths_host, void* stream) {
  if (!st || !lengths_host) return fail(GQA_ERR_ARG, "state or lengths is NULL");
  for (int b = 0; b < st->batch; ++b) {
    if (lengths_host[b] < 0 || lengths_host[b] > st->max_tokens)
      return fail(GQA_ERR_CAPACITY, "row %d: length %d outside [0, max_tokens=%d]", b, lengths_host[b], st->max_tokens);
    if (lengths_host[b] > st->blk->cfg.max_positions)
      return fail(GQA_ERR_POSITION, "row %d: length %d beyond max_positions", b, lengths_host[b]);
  }
  const int slot = st->next;
  st->next = (st->next + 1) % gqa_state::kRing;
  HIP_TRY(hipEventSynchronize(st->done[slot]));  // the slot's previous copy has finished
  int* stage = st->staging + (size_t)slot * st->batch;
  std::copy(lengths_host, lengths_host + st->batch, stage);
  HIP_TRY(hipMemcpyAsync(st->lengths_dev, stage, (size_t)st->batch * 4, hipMemcpyHostToDevice,
                         static_cast<hipStream_t>(stream)));
  HIP_TRY(hipEventRecord(st->done[slot], static_cast<hipStream_t>(stream)));
  st->lengths.assign(lengths_host, lengths_host + st->batch);
  return GQA_OK;
}

int gqa_state_get_lengths(const gqa_state* st, int32_t* lengths_host) {
  if (!st || !lengths_host) return fail(GQA_ERR_ARG, "state or lengths is NULL");
  std::copy(st->lengths.begin(), st->lengths.end(), lengths_host);
  return GQA_OK;
}

void gqa_state_free(gqa_state* st) { delete st; }

int gqa_workspace_bytes(const gqa_block* blk, int32_t B, int32_t L, size_t* out) {
  if (!blk || !out) return fail(GQA_ERR_ARG, "block or output is NULL");
  if (B < 0 || L < 0) return fail(GQA_ERR_ARG, "B and L must be >= 0");
  *out = (B == 0 || L == 0) ? 0 : layout_for(blk, B, L).total;
  return GQA_OK;
}

int gqa_block_forward(gqa_block* blk, gqa_state* st, const float* x, float* y, int32_t B, int32_t L, void* ws,
                      size_t wsb, void* stream) {
  return run_block(blk, st, x, y, B, L, ws, wsb, static_cast<hipStream_t>(stream));
}

int gqa_block_forward_ragged(gqa_block* blk, const float* x, float* y, int32_t B, int32_t L,
                             const int32_t* lengths, void* ws, size_t wsb, void* stream) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  if (B < 0 || L < 0) return fail(GQA_ERR_ARG, "B and L must be >= 0");
  if (B > 0 && L > 0 && !lengths) return fail(GQA_ERR_ARG, "lengths is NULL");
  for (int b = 0; b < B && L > 0; ++b)
    if (lengths[b] < 1 || lengths[b] > L)
      return fail(GQA_ERR_ARG, "row %d: length %d outside [1, %d]", b, lengths[b], L);
  if (B == 0 || L == 0) return run_block(blk, nullptr, x, y, B, L, ws, wsb, static_cast<hipStream_t>(stream));
  const auto& c = blk->cfg;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int d = c.d_model;
  int64_t rows = 0;
  for (int b = 0; b < B; ++b) rows += lengths[b];
  // Packed path: only the real tokens go through the norms, GEMMs, RoPE and
  // attention (cost proportional to the sum of the lengths).  The matrix-core
  // prefill attention takes per-row tables; the residual stream lives in the
  // workspace's float32 x1 buffer (gathered from x, updated in place by the
  // o_proj and down residual epilogues, scattered to y with +0.0 padding).
  // Other blocks (float32, sandwich norms, L = 1) take the padded path.
  const WsLayout lay = layout_for(blk, B, L);
  bool packed = is_bf16(blk) && attention_prefill_bf16_supported(c.head_dim, blk->G) && !c.sandwich_norms && L > 1 &&
                d % 4 == 0 && ws && wsb >= lay.total;
  PackedRows pk{};
  if (packed) {
    const int M = (int)rows, QW = blk->QW, KW = blk->KW, IT = c.intermediate;
    const bool gated = mlp_gated(c.mlp);
    pk.p_qkv = plan_gemm(M, QW + 2 * KW, d, false);
    pk.p_o = plan_gemm(M, d, QW, false);
    pk.p_gu = plan_gemm(M, IT, d, gated);
    pk.p_down = plan_gemm(M, d, IT, false);
    size_t part = 0;
    auto need = [&](const GemmPlan& p, size_t nb) { part = std::max(part, plan_part_bytes(p, M, nb)); };
    need(pk.p_qkv, QW + 2 * (size_t)KW);
    need(pk.p_o, d);
    need(pk.p_gu, (gated ? 2 : 1) * (size_t)IT);
    need(pk.p_down, d);
    // the workspace holds the K-split partials of the padded batch's plans;
    // packed plans needing more fall back to the padded path
    const size_t have = lay.part ? (lay.attn_part ? lay.attn_part : lay.total) - lay.part : 0;
    packed = part <= have;
  }
  if (!packed) {
    // Causal (and windowed) attention never lets a real position read a later
    // one, and every other step is per token, so the real positions of the
    // padded batch are exactly those of each row run alone; the padding
    // positions are then overwritten with +0.0.
    if (int r = run_block(blk, nullptr, x, y, B, L, ws, wsb, s)) return r;
    HIP_TRY(launch_zero_padding(y, lengths, B, L, d, s));
    return GQA_OK;
  }
  if (!x || !y) return fail(GQA_ERR_ARG, "x or y is NULL");
  BusyGuard guard(blk->busy);
  if (!guard.ok) return fail(GQA_ERR_BUSY, "block is in use by another call");
  char* base = static_cast<char*>(ws);
  int* row_start = reinterpret_cast<int*>(base + lay.rows);
  int* row_len = row_start + B;
  float* xp = reinterpret_cast<float*>(base + lay.x1);
  pk.row_start = row_start;
  pk.row_len = row_len;
  pk.rows = (int)rows;
  KernelTimer* tm = &blk->timer;
  {
    Scope sc(tm, "ragged_gather", s);
    HIP_TRY(launch_row_tables(lengths, B, row_start, row_len, s));
    HIP_TRY(launch_gather_rows(x, xp, row_start, row_len, B, L, d, s));
  }
  if (int r = run_block(blk, nullptr, xp, xp, B, L, ws, wsb, s, nullptr, false, &pk)) return r;
  Scope sc(tm, "ragged_scatter", s);
  HIP_TRY(launch_scatter_rows(xp, y, row_start, row_len, B, L, d, s));
  return GQA_OK;
}

int gqa_backward_workspace_bytes(const gqa_block* blk, int32_t B, int32_t L, size_t* out) {
  if (!blk || !out) return fail(GQA_ERR_ARG, "block or output is NULL");
  if (B < 0 || L < 0) return fail(GQA_ERR_ARG, "B and L must be >= 0");
  *out = (B == 0 || L == 0) ? 0 : bwd_layout_for(blk, B, L).total;
  return GQA_OK;
}

int gqa_block_backward(gqa_block* blk, const float* x, const float* grad_out, float* grad_x, float* const* grad_w,
                       int32_t B, int32_t L, void* ws, size_t wsb, void* stream) {
  return run_backward(blk, x, grad_out, grad_x, grad_w, B, L, ws, wsb, static_cast<hipStream_t>(stream));
}

int gqa_block_step(gqa_block* blk, gqa_state* st, const float* x, float* y, int32_t B, void* ws, size_t wsb,
                   void* stream) {
  if (!st) return fail(GQA_ERR_STATE, "step requires a state");
  return run_block(blk, st, x, y, B, 1, ws, wsb, static_cast<hipStream_t>(stream));
}

int gqa_block_status(gqa_block* blk, void* stream) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  HIP_TRY(hipStreamSynchronize(static_cast<hipStream_t>(stream)));
  int w[kStatusWords] = {};
  HIP_TRY(hipMemcpy(w, blk->status, sizeof w, hipMemcpyDeviceToHost));
  if (w[0] || w[1] || w[2]) {
    HIP_TRY(hipMemset(blk->status, 0, sizeof w));
    if (w[2])
      return fail(GQA_ERR_POSITION, "a device position was beyond the state's capacity or max_positions (clamped; "
                                    "outputs since the last check are not valid): a replayed captured step must "
                                    "restore the rows' lengths");
    if (w[0] && w[1])
      return fail(GQA_ERR_NONFINITE, "a non-finite input value was seen; %d non-finite cached key/value values", w[1]);
    if (w[0]) return fail(GQA_ERR_NONFINITE, "a non-finite input value was seen");
    return fail(GQA_ERR_NONFINITE, "%d non-finite cached key/value values", w[1]);
  }
  return GQA_OK;
}

int gqa_block_describe_plan(const gqa_block* blk, int32_t kind, int32_t B, int32_t L, char* buf, size_t buf_bytes,
                            size_t* needed) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  if (kind != 0 && kind != 1) return fail(GQA_ERR_ARG, "kind must be 0 (forward) or 1 (backward)");
  if (B < 1 || L < 1) return fail(GQA_ERR_ARG, "B and L must be >= 1");
  if ((int64_t)B * L > INT32_MAX / 2) return fail(GQA_ERR_ARG, "B * L is too large");
  const std::string d = describe_plan(blk, kind, B, L);
  if (needed) *needed = d.size() + 1;
  if (buf && buf_bytes) {
    const size_t n = std::min(buf_bytes - 1, d.size());
    memcpy(buf, d.data(), n);
    buf[n] = 0;
  }
  return GQA_OK;
}

int gqa_block_set_timing(gqa_block* blk, int32_t enable) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  blk->timer.collect();
  blk->timer.enabled = enable != 0;
  if (!enable) blk->timer.entries.clear();
  return GQA_OK;
}

int gqa_block_kernel_times(gqa_block* blk, const char** names, double* total_ms, int64_t* counts, int32_t cap) {
  if (!blk) return fail(GQA_ERR_ARG, "block is NULL");
  blk->timer.collect();
  const int n = (int)blk->timer.entries.size();
  for (int i = 0; i < n && i < cap; ++i) {
    if (names) names[i] = blk->timer.entries[i].name.c_str();
    if (total_ms) total_ms[i] = blk->timer.entries[i].ms;
    if (counts) counts[i] = blk->timer.entries[i].count;
  }
  return n;
}

}  // extern "C"
