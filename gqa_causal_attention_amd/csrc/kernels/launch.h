// Host-side launchers of the block's kernels (C++ linkage, internal to the
// library).  Every launcher enqueues on `stream` and returns hipSuccess or the
// launch error; shapes are validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

enum ElemType { kF32 = 0, kBF16 = 1 };

// B-operand row layouts of a "TN" GEMM  C[m, n] = sum_k A[m, k] * Brow(n)[k].
enum GemmMode {
  kModeSeg = 0,    // B rows come from up to 3 stacked [rows, K] matrices (q/k/v)
  kModeGated = 1,  // gate/up pair: output column n reads gate row n and up row n
};
enum GemmEpi {
  kEpiStore = 0,    // C = act(acc + bias) (act kActNone: acc + bias), in the activation type
  kEpiResid = 1,    // C (float32) = resid + (acc + bias[0]); resid and bias may be null
  kEpiGated = 2,    // C = act(acc_gate + bias[0]) * (acc_up + bias[1]), in the activation type
  kEpiPartial = 3,  // float32 partial sums of one K split (split-K; raw B-row order)
  // SwiGLU's backward on the product da (pipelined kernel, B transposed, one
  // K split): with g = resid[m, n], u = resid[m, N + n] (float32, row stride
  // ldr), C[m, n] = silu(g) u, C2[m, n] = da u silu'(g), C2[m, N + n] = da silu(g)
  // (activation type; row strides ldc, ldc2)
  kEpiSwigluBwd = 4,
};
// MLP activations (the values act_fn in common.h switches on).
enum ActKind { kActNone = 0, kActSilu = 1, kActGeluTanh = 2, kActGelu = 3 };

struct GemmArgs {
  const void* A;           // [M, K] activations, row stride lda
  int64_t lda;
  const void* B[3];        // weight segments [rows_s, K] (row stride K)
  int64_t seg_end[3];      // cumulative row ends of the segments (kModeSeg)
  const float* bias[3];    // kEpiStore: per-segment bias; kEpiResid: bias[0]; kEpiGated: gate, up
                           // biases (each may be null)
  int M, N, K;             // N = output columns (kModeGated: IT)
  void* C;                 // output, row stride ldc
  int64_t ldc;
  const float* resid;      // kEpiResid: [M, N] float32, row stride ldr
  int64_t ldr;
  int act;                 // ActKind (kEpiGated; kEpiStore when not kActNone)
  float* partial;          // kEpiPartial: [splits, M, NB] float32, NB = B rows
  int splits;              // number of K splits (grid z)
  int k_split;             // K elements per split (multiple of 64)
  int* bump;               // if non-null: bump[i] += bump_by for i < bump_n (once)
  int bump_n, bump_by;
  int order;               // tile order of the pipelined kernel (0 = XCD-aware groups; others for tuning)
  int wg_waves;            // weight-streaming kernel: waves (16-row weight groups) per workgroup
  // Transposed operands (pipelined kernel, 256x256 tiles, kModeSeg, residual or
  // partial epilogue): bit 0: A is stored K-major, A^T[K, M] with row stride
  // lda; bit 1: B is stored K-major, B^T[K, N] with row stride ldb, its rows
  // taken from the segments B[s] along K (seg_end = cumulative K ends; rows
  // past seg_end[2] repeat the last one and must meet zero A columns).
  int trans;
  int64_t ldb;
  void* C2;                // kEpiSwigluBwd: second output, row stride ldc2
  int64_t ldc2;
};

// Tile shapes of the bf16 MFMA GEMM.
enum GemmTile { kTile256x256 = 0, kTile256x192 = 1, kTile64x128 = 2, kTile128x128 = 3, kTile256x256w4 = 4,
                kTile64x64 = 5, kTileSkinny = 6,
                // direct-to-LDS pipelined tiles: 64-deep slices, 2 stages, 8 waves
                kTileDma256x256 = 7,      // waves 128x64, 16x16x32 MFMA, A re-read per row
                kTileDma256x256n = 8,     // waves 64x128, 16x16x32 MFMA, double-buffered fragments
                kTileDma256x256m32 = 9,   // waves 128x64, 32x32x16 MFMA, double-buffered fragments
                kTileDma256x192 = 10,     // waves 64x96, 16x16x32 MFMA, A re-read per row
};

// kTileSkinny dispatches to launch_gemm_skinny, kTileDma* to launch_gemm_dma.
hipError_t launch_gemm_bf16(const GemmArgs& a, int mode, int epi, int tile, hipStream_t s);
// Direct-to-LDS pipelined GEMM for prefill-sized M (k_split a multiple of the slice depth).
bool gemm_dma_tile(int tile);
hipError_t launch_gemm_dma(const GemmArgs& a, int mode, int epi, int tile, hipStream_t s);
// Weight-streaming GEMM for M <= 64 (decode); K split in multiples of 256.
// Its weight groups: 16 rows each (gated: 8 gate + 8 up rows of 8 columns).
int64_t gemm_skinny_groups(int N, bool gated);
bool gemm_skinny_supported(int M, int N, int K, int k_split, int waves, bool gated);
hipError_t launch_gemm_skinny(const GemmArgs& a, int mode, int epi, hipStream_t s);
hipError_t launch_gemm_f32(const GemmArgs& a, int mode, int epi, hipStream_t s);
// Sum the K-split partials in split order, then apply `epi` (kEpiStore / kEpiResid /
// kEpiGated) writing a.C; `out_type` is the element type of a.C for Store/Gated.
hipError_t launch_splitk_reduce(const GemmArgs& a, int mode, int epi, int out_type, hipStream_t s);

// Row normalisation with its residual plumbing (norm.hip).
enum NormKind { kNormRms = 0, kNormRmsOffset = 1, kNormLayer = 2 };
struct NormSpec {
  const float* w;          // gain [d]; null: this norm step is skipped
  const float* b;          // LayerNorm bias [d] or null
  int kind;                // NormKind
};
// Per row, each step optional: t = x + sum_z part[z] (+ bias); t = out_norm(t);
// t = resid + t; x1 = t; out = norm(t).  x and part may not both be null.
struct NormArgs {
  const float* x;          // [rows, d] float32 (non-finite values set *flag)
  const float* part;       // [splits, rows, d] K-split partial sums, or null
  int splits;
  const float* bias;       // [d] projection bias, or null
  NormSpec out_norm;       // sandwich norm of a sublayer output
  const float* resid;      // [rows, d] residual stream, or null
  float* x1;               // [rows, d] float32 store of t after the residual add, or null
  NormSpec norm;           // out = norm(t), written in out_type
  void* out;
  int d;
  float eps;
  int* flag;
};
bool norm_supported(int d);
hipError_t launch_norm(const NormArgs& a, int out_type, int rows, hipStream_t s);

struct RopeArgs {
  void* qkv;               // [T, ld] activations: q | k | v columns
  int64_t ld;
  void* knew;              // [B, KV, L, hd] post-RoPE keys of this call
  void* vnew;              // [B, KV, L, hd] values of this call
  void* kcache;            // [B, KV, cap, hd] or null
  void* vcache;
  const int* lengths;      // [B] start positions (null: zeros)
  const float* cos_tab;    // [max_positions, rd/2]
  const float* sin_tab;
  const float* q_norm;     // [hd] or null
  const float* k_norm;
  int B, L, H, KV, hd, cap, window, offset;
  int max_pos;             // rows of the cos/sin tables (device starts past them are clamped, *pos_flag set)
  int* pos_flag;
  int rd;                  // rotated dimensions (even, <= hd); hd .. rd-1 pass through
  int defer_append;        // 1: leave the cache to launch_kv_append (after attention)
  float eps;
  // Optional fused K-split reduction of the q/k/v GEMM: if `part` is set, the
  // q|k|v row is the sum over z < splits of part[z, token, :] (row stride ld)
  // plus the per-segment bias, rounded to the activation type, and q is
  // written (rotated) to qkv.  Only the vector form takes it.
  const float* part;
  int splits;
  const float* bias[3];    // q, k, v biases (may be null)
  // Packed ragged rows (a ragged prefill with no state): row b's t-th token
  // (t < row_len[b]) is q|k|v row row_start[b] + t; tokens t >= row_len[b]
  // are padding and skipped.  Null: token (b, t) is row b * L + t.
  const int* row_start;
  const int* row_len;
  int64_t prows;           // rows of the q|k|v activations (and of each K split of `part`); 0: B * L
  int skip_q;              // vector form without `part`: leave q to the attention kernel (keys/values only)
};
// True if launch_rope_append takes `part` for this shape and element type.
bool rope_append_fuses_reduce(int hd, int rd, int64_t ld, int elem);
hipError_t launch_rope_append(const RopeArgs& a, int elem, hipStream_t s);
hipError_t launch_kv_append(const RopeArgs& a, int elem, hipStream_t s);

struct AttnArgs {
  const void* q;           // [T, ldq] (query head h at column h*hd)
  int64_t ldq;
  const void* knew;        // [B, KV, L, hd]
  const void* vnew;
  const void* kcache;      // [B, KV, cap, hd] or null
  const void* vcache;
  const int* lengths;      // [B] start positions (null: zeros)
  void* ctx;               // [T, H*hd]
  int B, L, H, KV, hd, cap, window;
  int max_pos;             // positions the block allows (device starts are clamped into range)
  float softcap;           // 0 = off
  float* part;             // decode partials [H, rec_stride, hd + 2]: record s + b = row b's piece of segment s
  int nseg, rec_stride;    // decode: key segments per kv head; records per head (>= nseg + B)
  float* lse;              // prefill (bf16 kernel): if set, [B, H, Lp] log2-sum-exp2 of the scaled scores,
                           //   Lp = L rounded up to a multiple of 4
  // Packed ragged rows (prefill bf16 kernel): query / output token t < row_len[b]
  // of row b is row row_start[b] + t of q and ctx; its keys/values stay in
  // knew/vnew [B, KV, L, hd].  Null: token (b, t) is row b * L + t.
  const int* row_start;
  const int* row_len;
  // Prefill bf16 kernel: if rope_q, q is read as the projection left it and the
  // kernel applies the per-head q norm (q_norm, eps, offset: weight 1 + w) and
  // RoPE at positions start + t (tables [max_positions, rd/2], rd % 32 == 0)
  // itself, rounding to bf16 as the RoPE kernel would have stored it.
  int rope_q;
  const float* cos_tab;
  const float* sin_tab;
  const float* q_norm;
  int rd, offset;
  float eps;
};
hipError_t launch_attention_generic(const AttnArgs& a, int elem, hipStream_t s);
hipError_t launch_attention_prefill_bf16(const AttnArgs& a, hipStream_t s);
bool attention_prefill_bf16_supported(int hd, int G);
// Decode (L = 1): per-chunk partials into a.part, then the in-order combine into a.ctx.
hipError_t launch_attention_decode_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_decode_combine(const AttnArgs& a, hipStream_t s);
bool attention_decode_bf16_supported(int hd, int G);
int attention_decode_max_rows();
int attention_decode_max_segments();
int attention_decode_segments(int64_t total_keys, int keys_per_seg);

// Backward of a zero-state prefill (backward.hip).
struct BwdAttnArgs {
  const void* q;           // post-RoPE queries [T, ldq] (head h at column h*hd)
  int64_t ldq;
  const void* k;           // post-RoPE keys [B, KV, L, hd]
  const void* v;           // values [B, KV, L, hd]
  const void* o;           // attention output [T, ldo]
  int64_t ldo;
  const float* dout;       // gradient of the attention output [T, ldo], float32
  float* lse;              // row log-sum-exp of the scaled scores, base 2: [T, H] (wave kernels, written)
                           //   or [B, H, lse_ld] (matrix-core kernels, from the forward)
  float* dsum;             // rowsum(dO * O), same layout as lse (written)
  float* dq;               // [T, H, hd] gradient of the post-RoPE queries
  float* dk;               // [kv_parts][B, KV, L, hd] gradient of the post-RoPE keys (partials summed
  float* dv;               //   in part order by launch_rope_bwd_pack)
  int kv_parts;            // 1, or G per-head partials (matrix-core path)
  int64_t kv_part_stride;  // elements between partials: B * KV * L * hd
  const float* cos_tab;    // [max_positions, hd/2] (RoPE backward)
  const float* sin_tab;
  int B, L, H, KV, hd, window;
  int lse_ld;              // matrix-core layout: L rounded up to a multiple of 4
  float scale;             // 1 / sqrt(hd)
};
// [R, C] (row stride ld) -> out[c * ldo + r] for r < Rp (zero for r >= R).
hipError_t launch_transpose(const void* in, int in_type, int64_t ld, int R, int C, void* out, int out_type,
                            int64_t ldo, int Rp, hipStream_t s);
hipError_t launch_convert(const float* in, void* out, int elem, int64_t n, hipStream_t s);
// gu [rows, 2 IT] float32 (gate | up), da [rows, IT] -> act = silu(g) u and dgu = dg | du.
hipError_t launch_swiglu_bwd(const float* gu, const float* da, int64_t rows, int IT, void* act, void* dgu, int elem,
                             hipStream_t s);
// dx = resid + RMSNorm backward of dy at input x (gain w); dx_op: the same in elem (or null);
// wpart [rms_bwd_parts(rows, d), d]: the weight gradient's summands dy * x^,
// summed in row order over consecutive chunks of rows (their column sums are
// the weight gradient).
hipError_t launch_rms_bwd(const float* dy, const float* x, const float* w, const float* resid, int rows, int d,
                          float eps, float* dx, void* dx_op, int elem, float* wpart, hipStream_t s);
int rms_bwd_parts(int rows, int d);
int colsum_chunks(int R);  // rows of the `part` scratch of launch_colsum (times C floats)
hipError_t launch_colsum(const float* a, int R, int C, float* part, float* out, hipStream_t s);
// dq | dk | dv, RoPE undone on dq and dk, into the q/k/v GEMM's row layout [T, ld]
// (ld >= (H + 2 KV) hd; the columns past that width are zero).
hipError_t launch_rope_bwd_pack(const BwdAttnArgs& a, void* dqkv, int64_t ld, int elem, hipStream_t s);
// lse, dsum, dq, dk, dv of the attention (causal, optional window): wave kernels, any hd.
hipError_t launch_attention_bwd(const BwdAttnArgs& a, int elem, hipStream_t s);
// Matrix-core form (bf16, hd 64 / 128): needs the forward's lse, writes dsum, a bf16
// copy of dout into dob [T, ldo], dq, and G per-head partials of dk and dv.
bool attention_bwd_mfma_supported(int hd, int G);
hipError_t launch_attention_bwd_mfma(const BwdAttnArgs& a, void* dob, hipStream_t s);

hipError_t launch_count_nonfinite(const void* p, int elem, int64_t n, int* flag, hipStream_t s);
hipError_t launch_bump_lengths(int* lengths, int n, int by, hipStream_t s);
// Packed ragged rows: device tables row_start[b] (prefix of the lengths) and
// row_len[b] from host lengths; x [B, L, d] real tokens -> packed rows xp; and
// packed rows -> y [B, L, d] with +0.0 at padding positions (d % 4 == 0).
hipError_t launch_row_tables(const int32_t* lengths_host, int B, int* row_start, int* row_len, hipStream_t s);
hipError_t launch_gather_rows(const float* x, float* xp, const int* row_start, const int* row_len, int B, int L, int d,
                              hipStream_t s);
hipError_t launch_scatter_rows(const float* xp, float* y, const int* row_start, const int* row_len, int B, int L,
                               int d, hipStream_t s);
hipError_t launch_cache_nonfinite(const void* k, const void* v, const int* lengths, int elem, int B, int KV,
                                  int cap, int hd, int* count, hipStream_t s);
// y [B, L, d] float32: positions t >= lengths_host[b] of row b set to +0.0.
hipError_t launch_zero_padding(float* y, const int32_t* lengths_host, int B, int L, int d, hipStream_t s);

}  // namespace gqa
