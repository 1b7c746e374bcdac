/*
 * gqa_block.h — C ABI of one Llama-shaped transformer decoder block on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the block documented on the mojolearn.transformer API page
 * (class TransformerBlock, whose description states that it computes Hugging
 * Face's LlamaDecoderLayer forward pass): input RMSNorm, q/k/v projections with
 * [out, in] weights keyed by Hugging Face names, RoPE, grouped-query causal
 * attention over a caller-owned KV cache (optionally a sliding window over a
 * ring of W slots), o_proj plus residual, post-attention RMSNorm, gated MLP
 * plus residual.  Component formulas are those of the DantinoX "Core Layers —
 * Deep Reference" page (RMSNorm, RoPE, GELU, SwiGLU, pre-norm Block).
 *
 * Conventions for every function below:
 *   - Return value 0 on success, a negative gqa_status on failure; the text of
 *     the last failure on the calling thread is gqa_last_error().
 *   - Argument checks run on the host before any device work is enqueued; a
 *     failed check leaves the device, the state and the outputs untouched (the
 *     page's "raise an error before any computation").
 *   - Pointers named *_dev are device pointers (hipMalloc / torch CUDA
 *     tensors); the library never frees memory it did not allocate.
 *   - Work is enqueued asynchronously on the caller's HIP stream
 *     (hipStream_t passed as void*; NULL = the null stream).  No call
 *     allocates device memory except gqa_block_create (a RoPE table and a
 *     status word, freed by gqa_block_destroy).
 *   - Handles are not thread-safe; concurrent calls on one block return
 *     GQA_ERR_BUSY (the page's decode session refuses re-entrant use).
 */
#ifndef GQA_BLOCK_H
#define GQA_BLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_ARG = -1,          /* NULL pointer, bad enum, non-positive size */
  GQA_ERR_SHAPE = -2,        /* weight name missing/extra/misshapen, head geometry */
  GQA_ERR_DTYPE = -3,        /* tensor dtype differs from the block's */
  GQA_ERR_NONFINITE = -4,    /* non-finite weight (create), input or cache value (status) */
  GQA_ERR_CAPACITY = -5,     /* lengths[b] + L beyond the state's max_tokens */
  GQA_ERR_POSITION = -6,     /* a position at or beyond max_positions */
  GQA_ERR_STATE = -7,        /* state missing, from another block, or batch mismatch */
  GQA_ERR_WORKSPACE = -8,    /* workspace NULL or smaller than gqa_workspace_bytes */
  GQA_ERR_BUSY = -9,         /* re-entrant use of a block */
  GQA_ERR_HIP = -10,         /* a HIP runtime call failed (no device, launch failure) */
  GQA_ERR_UNSUPPORTED = -11  /* a shape this build's kernels do not cover */
} gqa_status;

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;
/* mojolearn ``norm``: RMSNorm with gain w, RMSNorm with gain 1 + w (Gemma), LayerNorm
 * (DantinoX "Core Layers" page, Normalisation / LayerNorm: population variance,
 * gain w, bias with norm_bias). */
typedef enum { GQA_NORM_RMS = 0, GQA_NORM_RMS_OFFSET = 1, GQA_NORM_LAYER = 2 } gqa_norm_kind;
/* mojolearn ``mlp``: gated down(act(gate(x)) * up(x)) with act = SiLU ('swiglu'),
 * tanh-GELU ('geglu_tanh') or exact erf GELU ('geglu'); ungated down(act(up(x)))
 * with exact ('gelu') or tanh ('gelu_tanh') GELU (no gate_proj). */
typedef enum {
  GQA_MLP_SWIGLU = 0, GQA_MLP_GEGLU_TANH = 1, GQA_MLP_GEGLU = 2, GQA_MLP_GELU = 3, GQA_MLP_GELU_TANH = 4
} gqa_mlp_kind;
/* RoPE frequency scaling (mojolearn ``rope_scaling``: None, "linear", "llama3"). */
typedef enum { GQA_ROPE_PLAIN = 0, GQA_ROPE_LINEAR = 1, GQA_ROPE_LLAMA3 = 2 } gqa_rope_scaling;

/* Block options: mojolearn TransformerBlock constructor parameters. */
typedef struct {
  int32_t d_model;        /* hidden size d */
  int32_t n_heads;        /* H query heads */
  int32_t n_kv_heads;     /* KV heads; n_heads % n_kv_heads == 0 (grouped-query) */
  int32_t head_dim;       /* hd, even; QW = H*hd may differ from d_model */
  int32_t intermediate;   /* IT, rows of gate_proj.weight */
  int32_t window;         /* 0: full causal.  W > 0: position p attends keys
                             [max(0, p-W+1), p] and the cache is a ring of W slots
                             (``window`` parameter) */
  int32_t max_positions;  /* absolute positions must stay below this (``max_positions``) */
  float rope_theta;       /* RoPE base (``rope_theta``) */
  float norm_eps;         /* RMSNorm epsilon, inside the square root (``norm_eps``) */
  float attn_softcap;     /* 0: off; c > 0: scores become c*tanh(s/c) (``attn_softcap``) */
  int32_t norm;           /* a gqa_norm_kind value: mojolearn ``norm``; every norm of the
                             block but qk_norm */
  int32_t mlp;            /* a gqa_mlp_kind value: mojolearn ``mlp`` */
  int32_t qkv_bias;       /* 1: q/k/v projection biases (``qkv_bias``) */
  int32_t qk_norm;        /* 1: per-head RMSNorm of q and k over head_dim before RoPE
                             (``qk_norm``); same eps and norm kind as the block */
  int32_t weight_dtype;   /* gqa_dtype of the weights, the GEMM operands, the
                             activations between kernels and the KV cache.  x and y
                             are always float32 and the residual stream is float32. */
  /* RoPE options (mojolearn ``rope_dim`` and ``rope_scaling``; frequencies of
   * the DantinoX "Core Layers" page, Positional Encoding / RoPE).  A zeroed
   * tail gives plain RoPE over every dimension. */
  int32_t rope_dim;       /* rotated dimensions per head, r: 0 = head_dim, else even
                             and in [2, head_dim].  Pairs (i, i + r/2), i < r/2, turn
                             at p * base^(-2i/r); dimensions r .. hd-1 pass through
                             (partial rotary) */
  int32_t rope_scaling;   /* gqa_rope_scaling.  LINEAR: every frequency / rope_factor.
                             LLAMA3: with wavelength w = 2 pi / freq and
                             n = rope_original_max_positions, w > n / low_freq_factor
                             divides by rope_factor, w < n / high_freq_factor keeps,
                             between blends (1 - s) freq / factor + s freq with
                             s = (n / w - low) / (high - low) */
  float rope_factor;              /* > 0 (LINEAR, LLAMA3) */
  float rope_low_freq_factor;     /* LLAMA3: > 0 and < rope_high_freq_factor */
  float rope_high_freq_factor;    /* LLAMA3 */
  int32_t rope_original_max_positions; /* LLAMA3: > 0 */
  /* Bias and norm options (mojolearn ``o_bias``, ``mlp_bias``, ``norm_bias``) and
   * Gemma 2/3's sandwich norms (the dew DecoderBlock page's output norms). */
  int32_t o_bias;         /* 1: o_proj.bias (d) */
  int32_t mlp_bias;       /* 1: up_proj.bias (IT), down_proj.bias (d) and, gated, gate_proj.bias (IT) */
  int32_t norm_bias;      /* 1 (LayerNorm only): a bias (d) beside every norm weight */
  int32_t sandwich_norms; /* 1: x1 = x + post_attention_layernorm(o_proj(attn)),
                             y = x1 + post_feedforward_layernorm(mlp(pre_feedforward_layernorm(x1)));
                             needs pre_/post_feedforward_layernorm.weight (d) */
} gqa_block_config;

/* One weight tensor, keyed by its Hugging Face parameter name, in torch's
 * [out, in] layout (row-major, contiguous) — the weight table of the
 * TransformerBlock class description.  Required: input_layernorm.weight (d),
 * post_attention_layernorm.weight (d), q_proj.weight (QW,d),
 * k_proj.weight (KW,d), v_proj.weight (KW,d), o_proj.weight (d,QW),
 * gate_proj.weight (IT,d; gated MLPs only), up_proj.weight (IT,d),
 * down_proj.weight (d,IT).  With qkv_bias: q_proj.bias (QW), k_proj.bias (KW),
 * v_proj.bias (KW).  With qk_norm: q_norm.weight (hd), k_norm.weight (hd).
 * With o_bias / mlp_bias / sandwich_norms / norm_bias: the tensors named in
 * the config fields above.  Norm weights and biases are float32; matrices are
 * in weight_dtype.  Weights are BORROWED
 * device pointers: keep them alive and unchanged until gqa_block_destroy. */
typedef struct {
  const char* name;
  const void* data_dev;
  int32_t dtype;          /* gqa_dtype */
  int32_t ndim;           /* 1 or 2 */
  int64_t shape[2];
} gqa_tensor;

typedef struct gqa_block gqa_block;
typedef struct gqa_state gqa_state;

/* Validate the config and the weight table (names, shapes, dtypes), upload
 * the RoPE cos/sin table (frequencies and angles formed in double precision,
 * stored as float32 [max_positions, rope_dim/2]) and check every weight for non-finite values
 * (one device pass, synchronous, on the null stream).  Errors: ARG, SHAPE,
 * DTYPE, NONFINITE, UNSUPPORTED, HIP.  On success *out owns the block. */
int gqa_block_create(const gqa_block_config* cfg, const gqa_tensor* weights, int32_t n_weights,
                     gqa_block** out);
void gqa_block_destroy(gqa_block* blk);

/* Bytes of ONE cache buffer (k or v) for a state of `batch` rows holding up to
 * `max_tokens` positions: batch * n_kv_heads * capacity * head_dim * elem,
 * capacity = window if window > 0 else max_tokens, elem = size of weight_dtype
 * (mojolearn allocate_state / TransformerState.capacity). */
int gqa_state_bytes(const gqa_block* blk, int32_t batch, int32_t max_tokens, size_t* bytes_per_cache);

/* Wrap caller-owned state buffers: k_cache_dev and v_cache_dev of
 * gqa_state_bytes each, laid out [batch, n_kv_heads, capacity, head_dim]
 * (slot = position, or position mod window), and lengths_dev: int32[batch],
 * the number of positions each row holds.  The buffers are BORROWED; this call
 * enqueues nothing and does not clear them (a new sequence needs lengths = 0,
 * see gqa_state_set_lengths).  It allocates a small pinned host staging buffer
 * for gqa_state_set_lengths, freed by gqa_state_free.  The cache holds post-RoPE keys and raw values.
 * Departure from the page: one length per row instead of one cached_tokens. */
int gqa_block_allocate_state(const gqa_block* blk, int32_t batch, int32_t max_tokens,
                             void* k_cache_dev, void* v_cache_dev, int32_t* lengths_dev,
                             gqa_state** out);

/* Set every row's length (host values, copied to lengths_dev on `stream`
 * through a pinned staging buffer, so the call does not wait for the GPU; the
 * values are also kept as the host mirror the argument checks use).  Used to
 * start a sequence (zeros) or to resume a pre-filled cache.  Errors: ARG,
 * CAPACITY, POSITION, HIP. */
int gqa_state_set_lengths(gqa_state* st, const int32_t* lengths_host, void* hip_stream);
/* Copy the host mirror of the lengths into lengths_host[batch]. */
int gqa_state_get_lengths(const gqa_state* st, int32_t* lengths_host);
void gqa_state_free(gqa_state* st);

/* Workspace bytes a forward of B rows x L tokens (L = 1 for step) needs. */
int gqa_workspace_bytes(const gqa_block* blk, int32_t B, int32_t L, size_t* out);

/* mojolearn TransformerBlock.forward: x_dev float32 [B, L, d] -> y_dev float32
 * [B, L, d] (may not alias x).  state NULL: a self-contained prefill at
 * positions [0, L) whose cache is discarded.  With a state: row b runs at
 * positions lengths[b] + t, reads the cache, appends its keys/values in place
 * and lengths[b] += L.  Errors (host, before any launch): ARG, STATE (batch
 * differs), CAPACITY, POSITION, WORKSPACE, BUSY, HIP. */
int gqa_block_forward(gqa_block* blk, gqa_state* st, const float* x_dev, float* y_dev, int32_t B,
                      int32_t L, void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* mojolearn TransformerBlock.forward with `lengths` (a ragged batch, no state):
 * row b is real at positions [0, lengths[b]) and padding after.  Each real
 * position's output equals that row run alone at its own length; padding
 * positions output exactly +0.0.  lengths is a HOST array of B values in
 * [1, L] (checked before any launch; not retained).  x, y, workspace as in
 * gqa_block_forward with state NULL (workspace sized by gqa_workspace_bytes(B, L)).
 * Errors: ARG (NULL lengths, a length outside [1, L]), and those of
 * gqa_block_forward. */
int gqa_block_forward_ragged(gqa_block* blk, const float* x_dev, float* y_dev, int32_t B, int32_t L,
                             const int32_t* lengths_host, void* workspace_dev, size_t workspace_bytes,
                             void* hip_stream);

/* Workspace bytes gqa_block_backward needs for B rows x L tokens. */
int gqa_backward_workspace_bytes(const gqa_block* blk, int32_t B, int32_t L, size_t* out);

/* mojolearn TransformerBlock.backward(x, grad_output): gradients of a
 * zero-state prefill.  The forward is recomputed from an empty cache at
 * positions [0, L) (window honoured) and grad_out_dev (float32 [B, L, d],
 * dL/dy) is propagated back: grad_x_dev (float32 [B, L, d]) receives dL/dx and
 * grad_w_dev (a HOST array of 9 device pointers, float32, each in its tensor's
 * shape, in the weight table's order: input_layernorm, post_attention_layernorm,
 * q_proj, k_proj, v_proj, o_proj, gate_proj, up_proj, down_proj) the weight
 * gradients, each summed over the B * L tokens (overwritten, not accumulated).
 * The default block options only (RMSNorm with gain w, SwiGLU, no biases, q/k
 * norm, softcap, RoPE scaling, partial rotary or sandwich norms); any window.
 * bf16 blocks run the products in bf16 with float32 accumulation.  Errors:
 * UNSUPPORTED (another option), ARG, POSITION (L > max_positions), WORKSPACE,
 * BUSY, HIP. */
int gqa_block_backward(gqa_block* blk, const float* x_dev, const float* grad_out_dev, float* grad_x_dev,
                       float* const* grad_w_dev, int32_t B, int32_t L, void* workspace_dev, size_t workspace_bytes,
                       void* hip_stream);

/* mojolearn TransformerBlock.step: forward with L = 1 on a required state; x
 * is [B, d] or [B, 1, d] (the same memory).  Errors: as forward, STATE if st
 * is NULL. */
int gqa_block_step(gqa_block* blk, gqa_state* st, const float* x_dev, float* y_dev, int32_t B,
                   void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* gqa_block_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same step, with its workspace taken from a fixed array of this library
 * in device memory instead of a caller-supplied buffer.  The caller still
 * passes the state, x_dev and y_dev as for gqa_block_step.  The array holds
 * 64 MiB (67108864 bytes) on each GPU the call runs on, from the first call on
 * that GPU until the process ends; a step whose workspace
 * (gqa_workspace_bytes(blk, B, 1)) is larger returns GQA_ERR_WORKSPACE before
 * any launch (the 8B-shaped block fits up to 64 rows).  No call allocates or
 * frees memory.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads, other blocks) race and
 * must be serialised by the caller.  Errors: those of gqa_block_step, and
 * WORKSPACE as above. */
int gqa_block_step_noalloc(gqa_block* blk, gqa_state* st, const float* x_dev, float* y_dev, int32_t B,
                           void* hip_stream);

/* Synchronise `stream` and report whether any x read since the last call was
 * non-finite (GQA_ERR_NONFINITE, flag cleared) — the input check the page
 * makes before computing, moved after it so the hot path never syncs.
 * Cache values (the page checks them too): with the environment variable
 * GQA_CHECK_FINITE set to a non-zero integer when the block is created, every
 * forward/step with a state first counts the non-finite values among each
 * row's used slots of the cached keys and values (slots below the row's
 * length, all W slots of a full window ring); a non-zero count is reported
 * here as GQA_ERR_NONFINITE with the count in the message, and cleared.  Off
 * by default: the scan reads the used cache once more, which would double a
 * decode step's cache traffic.
 * Positions: the capacity and max_positions checks of each call read the
 * state's host copy of the lengths.  A forward/step captured into a HIP graph
 * advances only the device lengths when replayed, so a replayed step must
 * restore them itself (a device copy in the graph, or gqa_state_set_lengths)
 * or the host copy no longer describes the cache.  As a guard, the kernels
 * clamp any device start position that would fall outside the cache or the
 * RoPE tables (so nothing is read or written out of bounds) and raise a flag
 * reported here as GQA_ERR_POSITION (cleared); outputs since the previous
 * check are then not valid.  Non-finite reports take second place. */
int gqa_block_status(gqa_block* blk, void* hip_stream);

/* Launch plan of a call, as text (introspection; no device work, nothing
 * launched).  kind 0: a forward/step of B rows x L tokens -- per projection
 * GEMM the kernel tile (a GemmTile value), K split and waves per workgroup,
 * the attention form, the workspace size; kind 1: the backward of a
 * zero-state prefill of B x L -- whether the gradient products read weights
 * (tr_dx) and activations (tr_dw) in place, whether SwiGLU's backward runs in
 * a product's epilogue, and each product's tile and K split.  One
 * "name value ..." item per line.  Writes at most buf_bytes - 1 characters
 * plus a terminating NUL into buf (which may be NULL with buf_bytes 0) and
 * the full length + 1 into *needed (if not NULL).  Errors: ARG for a NULL
 * block, another kind, or B or L below 1. */
int gqa_block_describe_plan(const gqa_block* blk, int32_t kind, int32_t B, int32_t L, char* buf,
                            size_t buf_bytes, size_t* needed);

/* Per-kernel timing.  When enabled, each launch of a forward/step is
 * bracketed by HIP events on the caller's stream and its duration added to a
 * per-kernel total.  gqa_block_kernel_times syncs the events, then writes up to
 * `cap` entries (name, total milliseconds, launch count) and returns the
 * number of kernels seen.  Names stay valid for the block's lifetime. */
int gqa_block_set_timing(gqa_block* blk, int32_t enable);
int gqa_block_kernel_times(gqa_block* blk, const char** names, double* total_ms, int64_t* counts,
                           int32_t cap);

/* Text of the last failure on this thread ("" if none). */
const char* gqa_last_error(void);

/* Library version string. */
const char* gqa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GQA_BLOCK_H */
