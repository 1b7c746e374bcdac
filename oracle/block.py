"""CPU oracle of one Llama-shaped decoder block (plain, slow, eager numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
executes this module: only the tests, the smoke check and the bench's CPU
baseline leg do.  It shares no code with the HIP path (no kernels, tables,
constants or helpers); the two meet only at the seeded inputs.

What it computes is the decoder block of the mojolearn ``TransformerBlock`` API
page (class description: a Llama-shaped block whose forward is Hugging Face's
LlamaDecoderLayer forward pass): input RMSNorm, q/k/v
projections with [out, in] weights, RoPE, grouped-query causal attention over
a caller-owned KV cache (optionally a sliding window over a ring of W slots),
o_proj plus residual, post-attention RMSNorm, gated MLP plus residual.  The
component formulas are the ones printed on the DantinoX "Core Layers — Deep
Reference" page: RMSNorm (Normalisation / RMSNorm equations), RoPE (Positional
Encoding / RoPE rotation and frequency), GELU and SwiGLU (Feed-Forward
Network), and the pre-norm residual block (`Block` — the unified transformer
block).

Readings of points the pages leave open (each is listed with its reason in the
design notes of the repository):
  * RoPE rotates the Hugging Face "rotate-half" pairs (i, i + hd/2) with the
    page's frequencies theta_i = base^(-2i/hd); the DantinoX page prints the
    interleaved pairs (2i, 2i+1), which is the same map up to a fixed
    permutation of each head's dimensions.  Angles and cos/sin are formed in
    float64 and rounded to the oracle's working precision.
  * Partial rotary (``rope_dim`` r < hd) rotates the rotate-half pairs
    (i, i + r/2) of a head's first r dimensions with frequencies
    base^(-2i/r) and leaves dimensions r .. hd-1 as they are (Hugging Face's
    partial_rotary_factor convention, which the page's layer follows).
  * ``norm='layernorm'`` uses the population variance (mean of squared
    deviations); its biases exist only with ``norm_bias``.  qk_norm stays an
    RMSNorm (the page: "RMS-normalize"), with gain 1 + w under
    ``rmsnorm_offset`` and w otherwise.
  * ``mlp``: 'gelu' / 'geglu' are the exact (erf) GELU, '_tanh' the tanh
    approximation (the dew page calls the tanh gated form "geglu" and the erf
    one "geglu_exact"; the mojolearn names are kept).  Ungated forms have no
    gate_proj.
  * Sandwich norms (not a mojolearn option; Gemma 2/3 as the dew pages
    describe them): post_attention_layernorm normalises the attention output
    before its residual add, pre_feedforward_layernorm is the MLP's input
    norm and post_feedforward_layernorm normalises the MLP output before its
    add, all of the block's norm kind (Hugging Face's names).
  * ``rope_scaling`` "linear" divides every frequency by its factor; "llama3"
    applies Hugging Face's Llama 3 wavelength ramp (``rope_inv_freq``); the
    page names both and their parameters but prints neither formula.
  * A window W means W keys including the query's own position: keys
    [max(0, p - W + 1), p] (mojolearn ``window`` parameter).
  * Masked keys are excluded from the softmax (not given a -1e9 bias).
  * The softcap is c * tanh(s / c) applied to the scaled score
    s = q.k / sqrt(hd), before the mask and the softmax.
  * The attention scale is 1 / sqrt(hd).
  * qk_norm normalises each head's q and k over head_dim after the
    projection (and its bias) and before RoPE, with the block's eps and norm
    kind.
  * The cache holds post-RoPE keys and raw values; under a window each
    (row, kv head) keeps a ring of W slots with slot = position mod W.
  * Each batch row carries its own cached length (positions of row b in a
    call are lengths[b] + t).
  * Keys of positions produced in the same call are read from the call's
    fresh k/v, so a windowed prefill longer than W is exact; afterwards the
    ring holds the last W positions.

Precision: float32 by default (the page's block is float32 in and out);
``dtype=np.float64`` gives a float64 run used to bound the float32 oracle's
own rounding error.  ``layout="rowwise"`` computes every token with the same
vector operations whether it arrives in a prefill or in a decode step, so
decode and prefill agree bit for bit (the page's "identical" mode claim).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rms_norm", "layer_norm", "gelu_erf", "MLP_KINDS", "rope_inv_freq", "rope_cos_sin", "apply_rope", "silu", "gelu_tanh", "attention_row",
    "OracleState", "block_forward", "block_step", "block_forward_rows",
    "BACKWARD_WEIGHTS", "backward_supported", "block_backward",
]


# --------------------------------------------------------------------------
# Sublayers
# --------------------------------------------------------------------------
def rms_norm(x: np.ndarray, w: np.ndarray, eps: float, offset: bool = False) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g.

    DantinoX "Core Layers" page, Normalisation / RMSNorm: RMS(x) =
    sqrt(mean(x_i^2) + eps), y = x / RMS(x) * gamma (eps inside the square
    root, no bias).  mojolearn ``norm='rmsnorm_offset'`` scales by 1 + w
    (Gemma) instead of w.  Computed in the dtype of ``x``.
    """
    dt = x.dtype
    ms = np.mean(x * x, axis=-1, keepdims=True)
    g = w.astype(dt)
    if offset:
        g = dt.type(1.0) + g
    return x / np.sqrt(ms + dt.type(eps)) * g


def layer_norm(x: np.ndarray, w: np.ndarray, b: np.ndarray | None, eps: float) -> np.ndarray:
    """LayerNorm over the last axis: (x - mu) / sqrt(var + eps) * gamma + beta.

    DantinoX "Core Layers" page, Normalisation / LayerNorm: mean and variance
    over the d features of each token (the population variance), eps inside
    the square root, a gain and a bias.  mojolearn ``norm='layernorm'``; the
    bias is present with ``norm_bias`` (else beta = 0).  Computed in the dtype
    of ``x``.
    """
    dt = x.dtype
    mu = np.mean(x, axis=-1, keepdims=True)
    xc = x - mu
    var = np.mean(xc * xc, axis=-1, keepdims=True)
    y = xc / np.sqrt(var + dt.type(eps)) * w.astype(dt)
    if b is not None:
        y = y + b.astype(dt)
    return y


def rope_inv_freq(rot_dim: int, theta: float, scaling: dict | None = None) -> np.ndarray:
    """Inverse frequencies theta_i for i in [0, rot_dim/2), in float64.

    DantinoX "Core Layers" page, Positional Encoding / RoPE: theta_i =
    base^(-2i/d) with d the number of rotated dimensions; the base is the
    block's ``rope_theta`` (mojolearn parameter; the page's NTK-aware variant
    is this same formula with the base multiplied by lambda).  mojolearn
    ``rope_dim`` (partial rotary) sets d below head_dim.

    mojolearn ``rope_scaling`` (the TransformerBlock parameter list):
      * {"type": "linear", "factor": f}: every frequency divided by f, so
        position p turns as position p / f did.
      * {"type": "llama3", "factor": f, "low_freq_factor": lo,
        "high_freq_factor": hi, "original_max_position_embeddings": n}: the
        Llama 3 ramp the block inherits from Hugging Face's layer, read from
        wavelengths w_i = 2 pi / theta_i.  A frequency whose wavelength is
        longer than n / lo is divided by f; one shorter than n / hi is kept;
        between the two it is the blend (1 - s) theta_i / f + s theta_i with
        s = (n / w_i - lo) / (hi - lo), which meets the two ends continuously.
    """
    i = np.arange(rot_dim // 2, dtype=np.float64)
    inv = np.float64(theta) ** (-2.0 * i / rot_dim)
    if not scaling:
        return inv
    kind = scaling.get("type", scaling.get("rope_type"))
    f = np.float64(scaling["factor"])
    if kind == "linear":
        return inv / f
    if kind != "llama3":
        raise ValueError(f"unknown rope_scaling type {kind!r}")
    lo = np.float64(scaling["low_freq_factor"])
    hi = np.float64(scaling["high_freq_factor"])
    n = np.float64(scaling["original_max_position_embeddings"])
    out = np.empty_like(inv)
    for j, th in enumerate(inv):
        wavelen = 2.0 * np.pi / th
        if wavelen > n / lo:          # long wavelengths: interpolated by f
            out[j] = th / f
        elif wavelen < n / hi:        # short wavelengths: unchanged
            out[j] = th
        else:                         # the ramp between them
            s = (n / wavelen - lo) / (hi - lo)
            out[j] = (1.0 - s) * th / f + s * th
    return out


def rope_cos_sin(positions: np.ndarray, rot_dim: int, theta: float,
                 scaling: dict | None = None) -> tuple[np.ndarray, np.ndarray]:
    """cos and sin of p * theta_i for i in [0, rot_dim/2), in float64.

    DantinoX "Core Layers" page, Positional Encoding / RoPE: the rotation of
    each dimension pair by the angle p * theta_i, theta_i from
    ``rope_inv_freq``.  Returns arrays of shape positions.shape + (rot_dim/2,).
    """
    inv_freq = rope_inv_freq(rot_dim, theta, scaling)
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    return np.cos(ang), np.sin(ang)


def apply_rope(u: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs (i, i + r/2) of the first r = 2 * cos.shape[-1] dims.

    u'_i       = u_i cos a_i - u_{i+r/2} sin a_i
    u'_{i+r/2} = u_{i+r/2} cos a_i + u_i sin a_i
    (the page's 2x2 rotation, applied to Hugging Face's rotate-half pairs);
    dimensions r .. hd-1 pass through unchanged (partial rotary, mojolearn
    ``rope_dim``).  ``cos``/``sin`` broadcast against u[..., :r/2].
    """
    half = cos.shape[-1]
    r = 2 * half
    a, b, rest = u[..., :half], u[..., half:r], u[..., r:]
    c, s = cos.astype(u.dtype), sin.astype(u.dtype)
    return np.concatenate([a * c - b * s, b * c + a * s, rest], axis=-1)


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU / swish: z * sigmoid(z) = z / (1 + exp(-z)) (DantinoX page, SwiGLU)."""
    with np.errstate(over="ignore"):
        return z / (z.dtype.type(1.0) + np.exp(-z))


def gelu_tanh(z: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).

    DantinoX page, Feed-Forward Network / GELU equation; dew's GatedMLP calls
    this form "geglu" when it gates.
    """
    t = z.dtype.type
    c = t(np.sqrt(2.0 / np.pi))
    return t(0.5) * z * (t(1.0) + np.tanh(c * (z + t(0.044715) * z * z * z)))


def gelu_erf(z: np.ndarray) -> np.ndarray:
    """GELU, exact form: z * Phi(z) = 0.5 z (1 + erf(z / sqrt(2))).

    DantinoX page, Feed-Forward Network / GELU: x times the standard normal
    CDF (the page prints the tanh approximation beside it).  mojolearn
    ``mlp='gelu'`` (ungated) and ``'geglu'`` (gated) use this form; the
    ``_tanh`` names the approximation.
    """
    from scipy.special import erf
    t = z.dtype.type
    return (t(0.5) * z * (t(1.0) + erf(z / t(np.sqrt(2.0))))).astype(z.dtype)


# mojolearn ``mlp``: name -> (activation, gated)
MLP_KINDS = {
    "swiglu": (silu, True),
    "geglu_tanh": (gelu_tanh, True),
    "geglu": (gelu_erf, True),
    "gelu_tanh": (gelu_tanh, False),
    "gelu": (gelu_erf, False),
}


def attention_row(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                  k_pos: np.ndarray, window: int, softcap: float,
                  q_chunk: int = 1024) -> np.ndarray:
    """Grouped-query causal attention for one batch row.

    q [Lq, H, hd], k/v [Lk, KV, hd] with absolute positions q_pos [Lq] and
    k_pos [Lk].  Query head h reads kv head h // G with G = H / KV (DantinoX
    page, MHA and GQA: a group of n_heads // kv_heads query heads shares one
    kv head).  Key s is in the set of query t iff k_pos[s] <= q_pos[t] and,
    with a window W > 0, k_pos[s] >= q_pos[t] - W + 1 (mojolearn ``window``).
    Scores q.k / sqrt(hd), optional softcap c * tanh(s / c), softmax over the
    key set (excluded keys take no part), weighted sum of values.

    Queries are processed in chunks of ``q_chunk`` rows to bound memory; each
    row's arithmetic does not depend on the chunking.
    """
    Lq, H, hd = q.shape
    KV = k.shape[1]
    G = H // KV
    dt = q.dtype
    scale = dt.type(1.0 / np.sqrt(hd))
    out = np.zeros((Lq, H, hd), dtype=dt)
    for c0 in range(0, Lq, q_chunk):
        c1 = min(Lq, c0 + q_chunk)
        qp = q_pos[c0:c1]
        allowed = k_pos[None, :] <= qp[:, None]
        if window > 0:
            allowed &= k_pos[None, :] >= qp[:, None] - (window - 1)
        cols = np.nonzero(allowed.any(axis=0))[0]
        if cols.size == 0:
            continue
        lo, hi = cols[0], cols[-1] + 1
        allowed = allowed[:, lo:hi]
        for h in range(H):
            j = h // G
            s = (q[c0:c1, h, :] @ k[lo:hi, j, :].T) * scale
            if softcap:
                cap = dt.type(softcap)
                s = cap * np.tanh(s / cap)
            s = np.where(allowed, s, dt.type(-np.inf))
            m = np.max(s, axis=-1, keepdims=True)
            e = np.exp(s - m)
            p = e / np.sum(e, axis=-1, keepdims=True)
            out[c0:c1, h, :] = p @ v[lo:hi, j, :]
    return out


def _attention_token(q_t: np.ndarray, k: np.ndarray, v: np.ndarray, window: int,
                     softcap: float, p: int) -> np.ndarray:
    """Rowwise attention of one query token at position p over keys at 0..p
    (k, v hold exactly positions 0..p).  Same definition as attention_row."""
    H, hd = q_t.shape
    KV = k.shape[1]
    G = H // KV
    dt = q_t.dtype
    lo = max(0, p - window + 1) if window > 0 else 0
    scale = dt.type(1.0 / np.sqrt(hd))
    out = np.empty((H, hd), dtype=dt)
    for h in range(H):
        j = h // G
        s = (k[lo:p + 1, j, :] @ q_t[h]) * scale
        if softcap:
            cap = dt.type(softcap)
            s = cap * np.tanh(s / cap)
        e = np.exp(s - np.max(s))
        out[h] = (e / np.sum(e)) @ v[lo:p + 1, j, :]
    return out


# --------------------------------------------------------------------------
# State (the caller-owned KV cache)
# --------------------------------------------------------------------------
class OracleState:
    """KV cache of the oracle block.

    mojolearn ``TransformerState``: per (row, kv head) a buffer of ``capacity``
    slots; without a window slot j holds position j and capacity is
    ``max_tokens``; with a window W it is a ring of W slots, slot = p mod W.
    Unlike the page's single ``cached_tokens``, each row carries its own
    length.
    """

    def __init__(self, cfg: dict, batch: int, max_tokens: int, dtype=np.float32):
        self.window = int(cfg.get("window", 0))
        self.capacity = self.window if self.window > 0 else int(max_tokens)
        self.max_tokens = int(max_tokens)
        KV, hd = cfg["n_kv_heads"], cfg["head_dim"]
        self.k = np.zeros((batch, KV, self.capacity, hd), dtype=dtype)
        self.v = np.zeros((batch, KV, self.capacity, hd), dtype=dtype)
        self.lengths = np.zeros(batch, dtype=np.int64)

    @classmethod
    def from_fill(cls, cfg, k_fill, v_fill, lengths, dtype=np.float32):
        st = cls(cfg, k_fill.shape[0], k_fill.shape[2], dtype)
        st.k[...] = k_fill
        st.v[...] = v_fill
        st.lengths[...] = lengths
        return st

    def slot(self, pos):
        return pos % self.window if self.window > 0 else pos

    def copy(self):
        st = object.__new__(OracleState)
        st.window, st.capacity, st.max_tokens = self.window, self.capacity, self.max_tokens
        st.k, st.v, st.lengths = self.k.copy(), self.v.copy(), self.lengths.copy()
        return st


# --------------------------------------------------------------------------
# The block
# --------------------------------------------------------------------------
def _linear(h, w, b=None):
    y = h @ w.T
    if b is not None:
        y = y + b
    return y


def _rope(cfg, positions):
    """cos/sin tables of the block's RoPE options (rope_theta, rope_dim, rope_scaling)."""
    rd = cfg.get("rope_dim") or cfg["head_dim"]
    return rope_cos_sin(positions, rd, cfg["rope_theta"], cfg.get("rope_scaling"))


def _project(cfg, W, x, dt, positions, layout):
    """Steps up to RoPE: returns q [B,L,H,hd], k, v [B,L,KV,hd] (k, q rotated)."""
    B, L, d = x.shape
    H, KV, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    offset = cfg.get("norm", "rmsnorm") == "rmsnorm_offset"
    eps = cfg["norm_eps"]
    w = {k: v.astype(dt) for k, v in W.items()}
    h = _norm(cfg, w, "input_layernorm", x)
    if layout == "rowwise":
        q = np.stack([np.stack([w["q_proj.weight"] @ h[b, t] for t in range(L)]) for b in range(B)])
        k = np.stack([np.stack([w["k_proj.weight"] @ h[b, t] for t in range(L)]) for b in range(B)])
        v = np.stack([np.stack([w["v_proj.weight"] @ h[b, t] for t in range(L)]) for b in range(B)])
        if cfg.get("qkv_bias"):
            q, k, v = q + w["q_proj.bias"], k + w["k_proj.bias"], v + w["v_proj.bias"]
    else:
        q = _linear(h, w["q_proj.weight"], w.get("q_proj.bias"))
        k = _linear(h, w["k_proj.weight"], w.get("k_proj.bias"))
        v = _linear(h, w["v_proj.weight"], w.get("v_proj.bias"))
    q = q.reshape(B, L, H, hd)
    k = k.reshape(B, L, KV, hd)
    v = v.reshape(B, L, KV, hd)
    if cfg.get("qk_norm"):
        q = rms_norm(q, w["q_norm.weight"], eps, offset)
        k = rms_norm(k, w["k_norm.weight"], eps, offset)
    cos, sin = _rope(cfg, positions)  # [B, L, rope_dim/2]
    q = apply_rope(q, cos[:, :, None, :], sin[:, :, None, :])
    k = apply_rope(k, cos[:, :, None, :], sin[:, :, None, :])
    return w, q, k, v


def _norm(cfg, w, name, x):
    """The block's norm kind (mojolearn ``norm``) applied with weights ``name``.*:
    RMSNorm with gain w or 1 + w, or LayerNorm with gain w and, with
    ``norm_bias``, bias ``name``.bias."""
    kind = cfg.get("norm", "rmsnorm")
    if kind == "layernorm":
        return layer_norm(x, w[name + ".weight"], w.get(name + ".bias"), cfg["norm_eps"])
    if kind not in ("rmsnorm", "rmsnorm_offset"):
        raise ValueError(f"unknown norm {kind!r}")
    return rms_norm(x, w[name + ".weight"], cfg["norm_eps"], kind == "rmsnorm_offset")


def _attn_residual(cfg, w, x, ctx2, layout):
    """x1 = x + o_proj(ctx) (+ o_proj.bias with ``o_bias``).  With sandwich
    norms the attention output is normalised by post_attention_layernorm
    before the add (Hugging Face's Gemma 2/3 naming; the dew DecoderBlock
    page's output norms, and the gemma4 text page's block equations)."""
    if layout == "rowwise":
        B, L, _ = x.shape
        a = np.empty_like(x)
        for b in range(B):
            for t in range(L):
                a[b, t] = w["o_proj.weight"] @ ctx2[b, t]
    else:
        a = ctx2 @ w["o_proj.weight"].T
    if "o_proj.bias" in w:
        a = a + w["o_proj.bias"]
    if cfg.get("sandwich_norms"):
        a = _norm(cfg, w, "post_attention_layernorm", a)
    return x + a


def _mlp(cfg, w, x1, layout):
    """y = x1 + MLP(norm(x1)).

    Gated (mojolearn ``mlp`` swiglu / geglu / geglu_tanh): down(act(gate(h)) *
    up(h)); ungated (gelu / gelu_tanh): down(act(up(h))); each projection
    adds its bias with ``mlp_bias``.  The pre-MLP norm is
    post_attention_layernorm, or pre_feedforward_layernorm with sandwich norms,
    which also normalise the MLP output by post_feedforward_layernorm before
    the add.
    """
    sandwich = bool(cfg.get("sandwich_norms"))
    h2 = _norm(cfg, w, "pre_feedforward_layernorm" if sandwich else "post_attention_layernorm", x1)
    act, gated = MLP_KINDS[cfg.get("mlp", "swiglu")]
    bg, bu, bd = w.get("gate_proj.bias"), w.get("up_proj.bias"), w.get("down_proj.bias")

    def ff_row(h):  # one token, matrix-vector products
        u = w["up_proj.weight"] @ h
        if bu is not None:
            u = u + bu
        if gated:
            g = w["gate_proj.weight"] @ h
            if bg is not None:
                g = g + bg
            m = act(g) * u
        else:
            m = act(u)
        o = w["down_proj.weight"] @ m
        return o + bd if bd is not None else o

    if layout == "rowwise":
        B, L, _ = x1.shape
        f = np.empty_like(x1)
        for b in range(B):
            for t in range(L):
                f[b, t] = ff_row(h2[b, t])
    else:
        u = _linear(h2, w["up_proj.weight"], bu)
        m = act(_linear(h2, w["gate_proj.weight"], bg)) * u if gated else act(u)
        f = _linear(m, w["down_proj.weight"], bd)
    if sandwich:
        f = _norm(cfg, w, "post_feedforward_layernorm", f)
    return x1 + f


def block_forward(cfg: dict, W: dict, x: np.ndarray, state: OracleState | None = None,
                  *, dtype=np.float32, layout: str = "batched", lengths=None) -> np.ndarray:
    """Run the block on x [B, L, d]; returns y [B, L, d] in ``dtype``.

    mojolearn ``TransformerBlock.forward``: with ``state=None`` a
    self-contained prefill from an empty cache; with a state, row b continues
    at position state.lengths[b], the cache is read at entry and updated, and
    the lengths advance by L.  Positions must stay below ``max_positions``
    and, without a window, within the state's capacity (the page's errors
    before any computation).

    ``lengths`` (the page's ragged batch; not allowed with a state): B values
    in [1, L]; row i is real at positions [0, lengths[i]) and padding after.
    Written as the page states it: each row's real positions are that row run
    alone at its own length, and padding positions are exactly +0.0.
    """
    if lengths is not None:
        if state is not None:
            raise ValueError("lengths is not allowed together with state")
        x = np.asarray(x)
        B, L = x.shape[0], x.shape[1]
        lens = [int(n) for n in lengths]
        if len(lens) != B or any(n < 1 or n > L for n in lens):
            raise ValueError("lengths must hold B values in [1, L]")
        y = np.zeros(x.shape, dtype=np.dtype(dtype))
        for i, n in enumerate(lens):
            y[i, :n] = block_forward(cfg, W, x[i:i + 1, :n], dtype=dtype, layout=layout)[0]
        return y
    dt = np.dtype(dtype)
    x = np.asarray(x).astype(dt)
    B, L, d = x.shape
    if d != cfg["d_model"]:
        raise ValueError("x last dim must equal d_model")
    H, KV, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    window = int(cfg.get("window", 0))
    start = np.zeros(B, dtype=np.int64) if state is None else state.lengths.astype(np.int64)
    if state is not None:
        if state.k.shape[0] != B:
            raise ValueError("batch size differs from the state's")
        if window == 0 and np.any(start + L > state.capacity):
            raise ValueError("state capacity exceeded")
        if np.any(start + L > state.max_tokens):
            raise ValueError("state max_tokens exceeded")
    if np.any(start + L > cfg["max_positions"]):
        raise ValueError("position at or beyond max_positions")
    positions = start[:, None] + np.arange(L)[None, :]            # [B, L]
    w, q, k, v = _project(cfg, W, x, dt, positions, layout)

    ctx = np.empty((B, L, H, hd), dtype=dt)
    for b in range(B):
        s0 = int(start[b])
        # keys of this row: cached positions [lo, s0) then the call's own [s0, s0+L)
        lo = max(0, s0 - window) if window > 0 else 0
        if state is not None and s0 > lo:
            cpos = np.arange(lo, s0)
            slots = state.slot(cpos)
            kc = np.transpose(state.k[b][:, slots, :], (1, 0, 2)).astype(dt)
            vc = np.transpose(state.v[b][:, slots, :], (1, 0, 2)).astype(dt)
            kall = np.concatenate([kc, k[b]], axis=0)
            vall = np.concatenate([vc, v[b]], axis=0)
            kpos = np.concatenate([cpos, positions[b]])
        else:
            kall, vall, kpos = k[b], v[b], positions[b]
        if layout == "rowwise":
            for t in range(L):
                p = s0 + t
                n = p + 1 - int(kpos[0])
                ctx[b, t] = _attention_token(q[b, t], _pad_front(kall[:n], kpos[0]),
                                             _pad_front(vall[:n], kpos[0]), window,
                                             cfg.get("attn_softcap", 0.0), p)
        else:
            ctx[b] = attention_row(q[b], kall, vall, positions[b], kpos, window,
                                   cfg.get("attn_softcap", 0.0))

    if state is not None:
        for b in range(B):
            s0 = int(start[b])
            first = max(s0, s0 + L - window) if window > 0 else s0
            for p in range(first, s0 + L):
                sl = state.slot(p)
                state.k[b, :, sl, :] = k[b, p - s0]
                state.v[b, :, sl, :] = v[b, p - s0]
        state.lengths += L

    ctx2 = ctx.reshape(B, L, H * hd)
    x1 = _attn_residual(cfg, w, x, ctx2, layout)
    return _mlp(cfg, w, x1, layout)


def _pad_front(a: np.ndarray, first_pos: int) -> np.ndarray:
    """Place keys that start at absolute position ``first_pos`` at index
    first_pos of an array indexed by position (rows before it are unused)."""
    first_pos = int(first_pos)
    if first_pos == 0:
        return a
    pad = np.zeros((first_pos,) + a.shape[1:], dtype=a.dtype)
    return np.concatenate([pad, a], axis=0)


def block_step(cfg: dict, W: dict, x: np.ndarray, state: OracleState, **kw) -> np.ndarray:
    """mojolearn ``TransformerBlock.step``: forward with L = 1 on a required state.
    x may be (B, 1, d) or (B, d); returns (B, 1, d)."""
    if state is None:
        raise ValueError("step requires a state")
    x = np.asarray(x)
    if x.ndim == 2:
        x = x[:, None, :]
    return block_forward(cfg, W, x, state, **kw)


def block_forward_rows(cfg: dict, W: dict, x: np.ndarray, rows, state: OracleState | None = None,
                       *, dtype=np.float32) -> np.ndarray:
    """Outputs of ``block_forward`` at selected (b, t) positions only.

    Same definition as ``block_forward`` restricted to output rows: keys and
    values are formed for every position (any query may read them), queries,
    attention, o_proj and the MLP only for the requested rows.  The state is
    read, not updated.  Returns an array [len(rows), d].
    """
    dt = np.dtype(dtype)
    x = np.asarray(x)
    B, L, d = x.shape
    H, KV, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    window = int(cfg.get("window", 0))
    offset = cfg.get("norm", "rmsnorm") == "rmsnorm_offset"
    eps = cfg["norm_eps"]
    w = {k: v.astype(dt) for k, v in W.items()}
    start = np.zeros(B, dtype=np.int64) if state is None else state.lengths.astype(np.int64)
    out = np.empty((len(rows), d), dtype=dt)
    by_row = {}
    for i, (b, t) in enumerate(rows):
        by_row.setdefault(int(b), []).append((i, int(t)))
    for b, items in by_row.items():
        s0 = int(start[b])
        xb = x[b].astype(dt)
        h = _norm(cfg, w, "input_layernorm", xb)                                # [L, d]
        k = _linear(h, w["k_proj.weight"], w.get("k_proj.bias")).reshape(L, KV, hd)
        v = _linear(h, w["v_proj.weight"], w.get("v_proj.bias")).reshape(L, KV, hd)
        if cfg.get("qk_norm"):
            k = rms_norm(k, w["k_norm.weight"], eps, offset)
        pos = s0 + np.arange(L)
        cos, sin = _rope(cfg, pos)
        k = apply_rope(k, cos[:, None, :], sin[:, None, :])
        lo = max(0, s0 - window) if window > 0 else 0
        if state is not None and s0 > lo:
            cpos = np.arange(lo, s0)
            slots = state.slot(cpos)
            kall = np.concatenate([np.transpose(state.k[b][:, slots, :], (1, 0, 2)).astype(dt), k], axis=0)
            vall = np.concatenate([np.transpose(state.v[b][:, slots, :], (1, 0, 2)).astype(dt), v], axis=0)
            kpos = np.concatenate([cpos, pos])
        else:
            kall, vall, kpos = k, v, pos
        ts = np.array([t for _, t in items])
        hq = h[ts]
        q = _linear(hq, w["q_proj.weight"], w.get("q_proj.bias")).reshape(len(ts), H, hd)
        if cfg.get("qk_norm"):
            q = rms_norm(q, w["q_norm.weight"], eps, offset)
        cq, sq = _rope(cfg, s0 + ts)
        q = apply_rope(q, cq[:, None, :], sq[:, None, :])
        ctx = attention_row(q, kall, vall, s0 + ts, kpos, window, cfg.get("attn_softcap", 0.0))
        x1 = _attn_residual(cfg, w, xb[ts][None], ctx.reshape(1, len(ts), H * hd), "batched")
        y = _mlp(cfg, w, x1, "batched")[0]
        for (i, _), yr in zip(items, y):
            out[i] = yr
    return out


# --------------------------------------------------------------------------
# Backward of a zero-state prefill
# --------------------------------------------------------------------------
BACKWARD_WEIGHTS = ("input_layernorm.weight", "post_attention_layernorm.weight", "q_proj.weight",
                    "k_proj.weight", "v_proj.weight", "o_proj.weight", "gate_proj.weight",
                    "up_proj.weight", "down_proj.weight")


def backward_supported(cfg: dict) -> bool:
    """mojolearn ``TransformerBlock.backward``: the default block options only
    (RMSNorm with gain w, SwiGLU, no biases, no q/k norm, no softcap, plain
    RoPE over every dimension, no sandwich norms); the window is honoured."""
    return (cfg.get("norm", "rmsnorm") == "rmsnorm" and cfg.get("mlp", "swiglu") == "swiglu"
            and not cfg.get("qkv_bias") and not cfg.get("qk_norm") and not cfg.get("attn_softcap")
            and not cfg.get("o_bias") and not cfg.get("mlp_bias") and not cfg.get("norm_bias")
            and not cfg.get("sandwich_norms") and not cfg.get("rope_scaling")
            and (cfg.get("rope_dim") or cfg["head_dim"]) == cfg["head_dim"])


def _rms_backward(dy, xhat, r, w):
    """RMSNorm y = x r w, r = (mean(x^2) + eps)^(-1/2), x^ = x r: with g = dy w,
    dx = r (g - x^ mean(g x^)) (r depends on every x_j through the mean), and
    dw = sum over tokens of dy x^."""
    g = dy * w
    dx = r * (g - xhat * np.mean(g * xhat, axis=-1, keepdims=True))
    dw = np.sum((dy * xhat).reshape(-1, dy.shape[-1]), axis=0)
    return dx, dw


def block_backward(cfg: dict, W: dict, x: np.ndarray, dy: np.ndarray, *, dtype=np.float64) -> dict:
    """Gradients of a zero-state prefill: mojolearn ``TransformerBlock.backward(x,
    grad_output)``: the forward is recomputed from an empty cache at positions
    [0, L) (window honoured) and grad_output = dL/dy is propagated back to x and
    the nine weights, each weight gradient summed over the B * L tokens.
    Returns {"x": [B, L, d], name: gradient in the tensor's shape}.

    The chain rule through the block of ``block_forward`` (DantinoX "Core
    Layers" page formulas), step by step in reverse: y = x1 + down(silu(g) u);
    g, u = gate(h2), up(h2); h2 = RMSNorm(x1); x1 = x + o_proj(ctx); ctx =
    softmax(q k^T / sqrt(hd) + mask) v per head (kv head h // G); q, k = RoPE
    of the projections of h = RMSNorm(x).  The softmax backward is dS = P (dP -
    rowsum(P dP)); RoPE's backward is the rotation by the opposite angle.
    """
    if not backward_supported(cfg):
        raise ValueError("backward supports the default block options only")
    dt = np.dtype(dtype)
    x = np.asarray(x).astype(dt)
    dy = np.asarray(dy).astype(dt)
    B, L, d = x.shape
    H, KV, hd = cfg["n_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    G = H // KV
    window = int(cfg.get("window", 0))
    if L > cfg["max_positions"]:
        raise ValueError("position at or beyond max_positions")
    eps = dt.type(cfg["norm_eps"])
    w = {k: v.astype(dt) for k, v in W.items()}
    scale = dt.type(1.0 / np.sqrt(hd))

    # ---- forward, keeping what the backward reads ----
    r1 = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    xh1 = x * r1
    h = xh1 * w["input_layernorm.weight"]
    q = (h @ w["q_proj.weight"].T).reshape(B, L, H, hd)
    k = (h @ w["k_proj.weight"].T).reshape(B, L, KV, hd)
    v = (h @ w["v_proj.weight"].T).reshape(B, L, KV, hd)
    cos, sin = _rope(cfg, np.arange(L))                          # [L, hd/2]
    c4, s4 = cos[None, :, None, :], sin[None, :, None, :]
    qr, kr = apply_rope(q, c4, s4), apply_rope(k, c4, s4)
    pos = np.arange(L)
    allowed = pos[None, :] <= pos[:, None]
    if window > 0:
        allowed &= pos[None, :] >= pos[:, None] - (window - 1)
    P = np.empty((B, H, L, L), dtype=dt)
    ctx = np.empty((B, L, H, hd), dtype=dt)
    for b in range(B):
        for hh in range(H):
            j = hh // G
            s = (qr[b, :, hh, :] @ kr[b, :, j, :].T) * scale
            s = np.where(allowed, s, -np.inf)
            e = np.exp(s - np.max(s, axis=-1, keepdims=True))
            P[b, hh] = e / np.sum(e, axis=-1, keepdims=True)
            ctx[b, :, hh, :] = P[b, hh] @ v[b, :, j, :]
    ctx2 = ctx.reshape(B, L, H * hd)
    x1 = x + ctx2 @ w["o_proj.weight"].T
    r2 = 1.0 / np.sqrt(np.mean(x1 * x1, axis=-1, keepdims=True) + eps)
    xh2 = x1 * r2
    h2 = xh2 * w["post_attention_layernorm.weight"]
    g = h2 @ w["gate_proj.weight"].T
    u = h2 @ w["up_proj.weight"].T
    sg = 1.0 / (1.0 + np.exp(-g))
    a = g * sg * u

    T = B * L
    flat = lambda t: t.reshape(T, t.shape[-1])
    out = {}
    # ---- y = x1 + a Wd^T ----
    out["down_proj.weight"] = flat(dy).T @ flat(a)
    da = dy @ w["down_proj.weight"]
    # ---- a = silu(g) u: d silu(g)/dg = sg (1 + g (1 - sg)) ----
    dg = da * u * sg * (1.0 + g * (1.0 - sg))
    du = da * g * sg
    out["gate_proj.weight"] = flat(dg).T @ flat(h2)
    out["up_proj.weight"] = flat(du).T @ flat(h2)
    dh2 = dg @ w["gate_proj.weight"] + du @ w["up_proj.weight"]
    dx1, out["post_attention_layernorm.weight"] = _rms_backward(dh2, xh2, r2, w["post_attention_layernorm.weight"])
    dx1 = dx1 + dy
    # ---- x1 = x + ctx Wo^T ----
    out["o_proj.weight"] = flat(dx1).T @ flat(ctx2)
    dctx = (dx1 @ w["o_proj.weight"]).reshape(B, L, H, hd)
    # ---- attention, per row and head ----
    dqr = np.zeros_like(qr)
    dkr = np.zeros_like(kr)
    dv = np.zeros_like(v)
    for b in range(B):
        for hh in range(H):
            j = hh // G
            p = P[b, hh]
            dO = dctx[b, :, hh, :]
            dv[b, :, j, :] += p.T @ dO
            dp = dO @ v[b, :, j, :].T
            ds = p * (dp - np.sum(p * dp, axis=-1, keepdims=True))
            dqr[b, :, hh, :] = (ds @ kr[b, :, j, :]) * scale
            dkr[b, :, j, :] += (ds.T @ qr[b, :, hh, :]) * scale
    # ---- RoPE: rotation back by the opposite angle ----
    dq = apply_rope(dqr, c4, -s4).reshape(B, L, H * hd)
    dk = apply_rope(dkr, c4, -s4).reshape(B, L, KV * hd)
    dv = dv.reshape(B, L, KV * hd)
    out["q_proj.weight"] = flat(dq).T @ flat(h)
    out["k_proj.weight"] = flat(dk).T @ flat(h)
    out["v_proj.weight"] = flat(dv).T @ flat(h)
    dh = dq @ w["q_proj.weight"] + dk @ w["k_proj.weight"] + dv @ w["v_proj.weight"]
    dxn, out["input_layernorm.weight"] = _rms_backward(dh, xh1, r1, w["input_layernorm.weight"])
    out["x"] = dx1 + dxn
    return out
