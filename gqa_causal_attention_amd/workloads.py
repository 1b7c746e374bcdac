"""Seeded synthetic workloads for one Llama-shaped decoder block.

This module is data only: block shapes, the order in which random inputs are
drawn, and round-to-nearest-even rounding of those draws to bfloat16 values.
It holds none of the block's arithmetic, and both the GPU path's tests/bench
and the CPU oracle's tests take their inputs from here.

Weight names and [out, in] layouts follow the weight table of the mojolearn
``TransformerBlock`` API page (class description); the draw recipe
(``default_rng(seed)``, ``standard_normal(shape, dtype=float32)`` times 0.02)
follows that page's usage example.
"""
from __future__ import annotations

import numpy as np

# Required tensors, in the order of the page's weight table.
REQUIRED_NAMES = (
    "input_layernorm.weight",
    "post_attention_layernorm.weight",
    "q_proj.weight",
    "k_proj.weight",
    "v_proj.weight",
    "o_proj.weight",
    "gate_proj.weight",
    "up_proj.weight",
    "down_proj.weight",
)
BIAS_NAMES = ("q_proj.bias", "k_proj.bias", "v_proj.bias")
QK_NORM_NAMES = ("q_norm.weight", "k_norm.weight")
# Optional tensors of the page's other options, in the order they are drawn
# (after the ones above, so turning an option on leaves earlier draws alone).
O_BIAS_NAMES = ("o_proj.bias",)
MLP_BIAS_NAMES = ("gate_proj.bias", "up_proj.bias", "down_proj.bias")
SANDWICH_NAMES = ("pre_feedforward_layernorm.weight", "post_feedforward_layernorm.weight")
NORM_BIAS_NAMES = ("input_layernorm.bias", "post_attention_layernorm.bias",
                   "pre_feedforward_layernorm.bias", "post_feedforward_layernorm.bias")
UNGATED_MLPS = ("gelu", "gelu_tanh")

# Block configurations.  Keys mirror the C struct gqa_block_config; the
# workload keys (batch, seq_len, ...) describe the synthetic run.
_BASE = dict(window=0, rope_theta=10000.0, norm_eps=1e-6, attn_softcap=0.0,
             norm="rmsnorm", mlp="swiglu", qkv_bias=False, qk_norm=False,
             max_positions=8192, o_bias=False, mlp_bias=False, norm_bias=False,
             sandwich_norms=False)

LLAMA3_8B_BLOCK = dict(_BASE, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                       intermediate=14336, rope_theta=500000.0, dtype="bf16")
GEMMA2_WINDOW_BLOCK = dict(_BASE, d_model=2304, n_heads=8, n_kv_heads=4, head_dim=256,
                           intermediate=9216, window=4096, attn_softcap=50.0,
                           mlp="geglu_tanh", norm="rmsnorm_offset", dtype="bf16")
QWEN_LONG_BLOCK = dict(_BASE, d_model=5120, n_heads=40, n_kv_heads=8, head_dim=128,
                       intermediate=27648, qkv_bias=True, qk_norm=True,
                       max_positions=32769, dtype="bf16")
TINY_LLAMA_BLOCK = dict(_BASE, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16,
                        intermediate=172, rope_theta=10000.0, dtype="f32")

WORKLOADS = {
    # tiny fp32 block: prefill of 16 tokens, then 8 single-token decode steps
    "tiny_llama_f32": dict(block=TINY_LLAMA_BLOCK, seed=1, batch=1, seq_len=16,
                           decode_steps=8, capacity=24, kind="prefill+decode"),
    # Llama-3-8B-shaped prefill, one sequence of 4096 tokens
    "llama3_8b_prefill_4k": dict(block=LLAMA3_8B_BLOCK, seed=2, batch=1, seq_len=4096,
                                 capacity=4096, kind="prefill"),
    # Llama-3-8B-shaped decode: 64 rows, cache of 8192 slots pre-filled up to
    # a per-row position drawn uniformly from [1024, 8192)
    "llama3_8b_decode_b64": dict(block=LLAMA3_8B_BLOCK, seed=3, batch=64, seq_len=1,
                                 capacity=8192, pos_range=(1024, 8192), kind="decode"),
    # Gemma2-style sliding window (W=4096) prefill, 2 x 8192 tokens
    "gemma2_window_prefill_8k": dict(block=GEMMA2_WINDOW_BLOCK, seed=4, batch=2,
                                     seq_len=8192, capacity=8192, kind="prefill"),
    # Qwen-style long-context prefill, one sequence of 32768 tokens
    "qwen_long_prefill_32k": dict(block=QWEN_LONG_BLOCK, seed=5, batch=1, seq_len=32768,
                                  capacity=32768, kind="prefill"),
    # Qwen-style decode: 16 rows at cache length 32768 (new token at 32768)
    "qwen_long_decode_b16": dict(block=QWEN_LONG_BLOCK, seed=5, batch=16, seq_len=1,
                                 capacity=32769, fixed_pos=32768, kind="decode"),
}


def weight_shapes(cfg: dict) -> dict:
    """HF names -> [out, in] shapes for the block described by ``cfg``."""
    d, hd = cfg["d_model"], cfg["head_dim"]
    qw, kw, it = cfg["n_heads"] * hd, cfg["n_kv_heads"] * hd, cfg["intermediate"]
    shapes = {
        "input_layernorm.weight": (d,),
        "post_attention_layernorm.weight": (d,),
        "q_proj.weight": (qw, d),
        "k_proj.weight": (kw, d),
        "v_proj.weight": (kw, d),
        "o_proj.weight": (d, qw),
        "gate_proj.weight": (it, d),
        "up_proj.weight": (it, d),
        "down_proj.weight": (d, it),
    }
    if cfg.get("qkv_bias"):
        shapes.update({"q_proj.bias": (qw,), "k_proj.bias": (kw,), "v_proj.bias": (kw,)})
    if cfg.get("qk_norm"):
        shapes.update({"q_norm.weight": (hd,), "k_norm.weight": (hd,)})
    ungated = cfg.get("mlp", "swiglu") in UNGATED_MLPS
    if ungated:
        del shapes["gate_proj.weight"]
    if cfg.get("o_bias"):
        shapes["o_proj.bias"] = (d,)
    if cfg.get("mlp_bias"):
        if not ungated:
            shapes["gate_proj.bias"] = (it,)
        shapes.update({"up_proj.bias": (it,), "down_proj.bias": (d,)})
    if cfg.get("sandwich_norms"):
        shapes.update({n: (d,) for n in SANDWICH_NAMES})
    if cfg.get("norm_bias"):
        for n in NORM_BIAS_NAMES:
            if n.replace(".bias", ".weight") in shapes:
                shapes[n] = (d,)
    return shapes


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32.

    Non-finite inputs are not expected here (all draws are finite normals).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # finite values: u + 0x8000 never wraps a uint32
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _is_norm_weight(name: str) -> bool:
    return name.endswith("layernorm.weight") or name in QK_NORM_NAMES


def _is_norm_bias(name: str) -> bool:
    return name.endswith("layernorm.bias")


def draw_weights(cfg: dict, rng: np.random.Generator) -> dict:
    """Draw the block's tensors in the fixed order: required table, biases, q/k norms.

    Projection weights and biases: 0.02 * N(0, 1).  Norm gains: 1 + 0.1 * N(0, 1)
    for a plain RMSNorm or LayerNorm; for the (1 + w) RMSNorm the stored w is
    0.1 * N(0, 1), so the effective gain has the same law.  LayerNorm biases:
    0.1 * N(0, 1).  Tensors an option does not use are not drawn.
    """
    shapes = weight_shapes(cfg)
    order = [n for n in REQUIRED_NAMES if n in shapes]
    if cfg.get("qkv_bias"):
        order += list(BIAS_NAMES)
    if cfg.get("qk_norm"):
        order += list(QK_NORM_NAMES)
    order += [n for n in O_BIAS_NAMES + MLP_BIAS_NAMES + SANDWICH_NAMES + NORM_BIAS_NAMES if n in shapes]
    out = {}
    offset_norm = cfg.get("norm") == "rmsnorm_offset"
    for name in order:
        z = rng.standard_normal(shapes[name], dtype=np.float32)
        if _is_norm_weight(name):
            # q_norm/k_norm follow the block's norm kind as well
            w = z * np.float32(0.1)
            if not offset_norm:
                w = w + np.float32(1.0)
        elif _is_norm_bias(name):
            w = z * np.float32(0.1)
        else:
            w = z * np.float32(0.02)
        out[name] = w.astype(np.float32)
    if cfg["dtype"] == "bf16":
        out = {k: round_bf16(v) for k, v in out.items()}
    return out


def make_workload(name: str, *, batch: int | None = None, seq_len: int | None = None,
                  capacity: int | None = None, fill_kv: bool = True) -> dict:
    """Build the seeded inputs of a named workload.

    Returns a dict with ``cfg`` (block config), ``weights`` (float32 arrays,
    bf16-representable for bf16 blocks), ``x`` [B, L, d] float32, and for
    decode workloads ``lengths`` [B] int32 and ``k_fill``/``v_fill``
    [B, KV, capacity, hd] float32 (bf16-representable for bf16 blocks, zero
    beyond each row's length).  For the tiny workload, ``x_steps``
    [steps, B, 1, d] holds the decode inputs.

    ``batch``/``seq_len``/``capacity`` override the workload's sizes (smaller
    parity cases of the same shape family); the draw order is unchanged.
    """
    wl = WORKLOADS[name]
    cfg = dict(wl["block"])
    B = wl["batch"] if batch is None else batch
    L = wl["seq_len"] if seq_len is None else seq_len
    cap = wl["capacity"] if capacity is None else capacity
    rng = np.random.default_rng(wl["seed"])
    weights = draw_weights(cfg, rng)
    d = cfg["d_model"]
    x = rng.standard_normal((B, L, d), dtype=np.float32)
    out = dict(name=name, cfg=cfg, weights=weights, x=x, batch=B, seq_len=L,
               capacity=cap, kind=wl["kind"])
    if wl["kind"] == "decode":
        if "pos_range" in wl:
            lo, hi = wl["pos_range"]
            hi = min(hi, cap)
            lo = min(lo, hi - 1)
            lengths = rng.integers(lo, hi, size=B).astype(np.int32)
        else:
            lengths = np.full(B, min(wl["fixed_pos"], cap - 1), dtype=np.int32)
        out["lengths"] = lengths
        if fill_kv:
            KV, hd = cfg["n_kv_heads"], cfg["head_dim"]
            kf = rng.standard_normal((B, KV, cap, hd), dtype=np.float32)
            vf = rng.standard_normal((B, KV, cap, hd), dtype=np.float32)
            if cfg["dtype"] == "bf16":
                kf, vf = round_bf16(kf), round_bf16(vf)
            # slots at or beyond a row's length are unused: keep them zero
            slot = np.arange(cap)[None, None, :, None]
            used = slot < lengths[:, None, None, None]
            out["k_fill"] = np.where(used, kf, np.float32(0.0))
            out["v_fill"] = np.where(used, vf, np.float32(0.0))
    if wl.get("decode_steps"):
        out["x_steps"] = rng.standard_normal((wl["decode_steps"], B, 1, d), dtype=np.float32)
    return out


def rng_array(seed: int, shape, scale: float = 1.0, dtype: str = "f32") -> np.ndarray:
    """A seeded N(0, scale^2) float32 array (bf16-rounded when dtype == 'bf16')."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    return round_bf16(a) if dtype == "bf16" else a.astype(np.float32)


def random_block(seed: int, *, dtype: str = "f32", **overrides) -> tuple[dict, dict]:
    """A small random block config + weights for parity sweeps (same recipe)."""
    cfg = dict(_BASE, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
               dtype=dtype)
    cfg.update(overrides)
    rng = np.random.default_rng(seed)
    return cfg, draw_weights(cfg, rng)
