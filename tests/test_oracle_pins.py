"""Pins of the CPU oracle's sublayers to things other than itself.

Each pin is chosen so that a plausible slip in the oracle fails it: eps
outside the square root, a wrong reduction axis, the (1 + w) gain missed, the
wrong RoPE pairing / frequency / sign, the wrong GQA head mapping, a window of
W + 1 keys, the softcap on the wrong quantity, a transposed operand.

Sources of truth: closed forms of the formulas printed on the DantinoX "Core
Layers" page (RMSNorm, RoPE, GELU, SwiGLU), hand-derivable special cases,
brute-force loops on tiny inputs, and library routines (torch's rms_norm,
silu, gelu, scaled_dot_product_attention; Hugging Face's rotary helpers).
"""
import math

import numpy as np
import pytest
import torch

from oracle import apply_rope, attention_row, gelu_tanh, rms_norm, rope_cos_sin, silu


# ----------------------------------------------------------------- RMSNorm --
def test_rmsnorm_hand_case():
    # x = [3, 4]: mean(x^2) = 12.5 ; with w = [1, 2], eps = 0:
    # y = [3, 8] / sqrt(12.5)
    x = np.array([3.0, 4.0])
    y = rms_norm(x, np.array([1.0, 2.0]), 0.0)
    np.testing.assert_allclose(y, [3 / math.sqrt(12.5), 8 / math.sqrt(12.5)], rtol=1e-15)
    # eps sits inside the square root: sqrt(12.5 + 0.5) = sqrt(13)
    y = rms_norm(x, np.ones(2), 0.5)
    np.testing.assert_allclose(y, [3 / math.sqrt(13.0), 4 / math.sqrt(13.0)], rtol=1e-15)


def test_rmsnorm_unit_gain_mean_square():
    # With g = 1, mean(out^2) = ms / (ms + eps) exactly (in exact arithmetic).
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 33))
    eps = 0.3
    y = rms_norm(x, np.ones(33), eps)
    ms = np.mean(x * x, axis=-1)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), ms / (ms + eps), rtol=1e-13)


def test_rmsnorm_offset_and_library():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 48))
    w = rng.standard_normal(48) * 0.1
    # rmsnorm_offset scales by 1 + w
    np.testing.assert_allclose(rms_norm(x, w, 1e-6, offset=True), rms_norm(x, 1.0 + w, 1e-6),
                               rtol=1e-14)
    # library routine: torch.nn.functional.rms_norm
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (48,), torch.from_numpy(w), eps=1e-6)
    np.testing.assert_allclose(rms_norm(x, w, 1e-6), ref.numpy(), rtol=1e-12, atol=1e-14)


def test_rmsnorm_float32_path():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 4096)).astype(np.float32)
    w = (1 + 0.1 * rng.standard_normal(4096)).astype(np.float32)
    y32 = rms_norm(x, w, 1e-6)
    assert y32.dtype == np.float32
    y64 = rms_norm(x.astype(np.float64), w.astype(np.float64), 1e-6)
    assert np.max(np.abs(y32 - y64)) / np.max(np.abs(y64)) < 1e-6


# -------------------------------------------------------------------- RoPE --
def test_rope_frequencies_hand_case():
    # hd = 4, base 10000: theta_0 = 1, theta_1 = 10000^(-1/2) = 0.01.
    cos, sin = rope_cos_sin(np.array([1, 3]), 4, 10000.0)
    np.testing.assert_allclose(cos, [[math.cos(1), math.cos(0.01)], [math.cos(3), math.cos(0.03)]],
                               rtol=1e-15)
    np.testing.assert_allclose(sin, [[math.sin(1), math.sin(0.01)], [math.sin(3), math.sin(0.03)]],
                               rtol=1e-15)


def test_rope_basis_vectors():
    # e_i -> cos(p th_i) e_i + sin(p th_i) e_{i+hd/2};  e_{i+hd/2} -> -sin e_i + cos e_{i+hd/2}
    hd, p, base = 8, 5, 100.0
    cos, sin = rope_cos_sin(np.array(p), hd, base)
    for i in range(hd // 2):
        th = base ** (-2.0 * i / hd)
        e = np.zeros(hd)
        e[i] = 1.0
        out = apply_rope(e, cos, sin)
        want = np.zeros(hd)
        want[i], want[i + hd // 2] = math.cos(p * th), math.sin(p * th)
        np.testing.assert_allclose(out, want, atol=1e-15)
        e = np.zeros(hd)
        e[i + hd // 2] = 1.0
        out = apply_rope(e, cos, sin)
        want = np.zeros(hd)
        want[i], want[i + hd // 2] = -math.sin(p * th), math.cos(p * th)
        np.testing.assert_allclose(out, want, atol=1e-15)


def test_rope_identity_norm_and_relative():
    rng = np.random.default_rng(3)
    hd = 16
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    c0, s0 = rope_cos_sin(np.array(0), hd, 1e4)
    np.testing.assert_array_equal(apply_rope(q, c0, s0), q)          # position 0 is the identity
    cp, sp = rope_cos_sin(np.array(37), hd, 1e4)
    r = apply_rope(q, cp, sp)
    h = hd // 2
    np.testing.assert_allclose(r[:h] ** 2 + r[h:] ** 2, q[:h] ** 2 + q[h:] ** 2, rtol=1e-13)
    # scores depend only on p - m (DantinoX page, RoPE relative-distance property)
    def score(p, m):
        a = apply_rope(q, *rope_cos_sin(np.array(p), hd, 1e4))
        b = apply_rope(k, *rope_cos_sin(np.array(m), hd, 1e4))
        return float(a @ b)
    assert abs(score(9, 4) - score(109, 104)) < 1e-12
    assert abs(score(9, 4) - score(12, 4)) > 1e-3


def test_rope_matches_page_interleaved_form():
    # The DantinoX page prints the rotation on interleaved pairs (2i, 2i+1):
    #   out[2i] = x[2i] cos - x[2i+1] sin ; out[2i+1] = x[2i] sin + x[2i+1] cos.
    # Rotate-half on u equals that form on the interleaved permutation of u.
    rng = np.random.default_rng(4)
    hd, p = 12, 11
    u = rng.standard_normal(hd)
    cos, sin = rope_cos_sin(np.array(p), hd, 1e4)
    perm = np.empty(hd, dtype=int)
    perm[0::2], perm[1::2] = np.arange(hd // 2), np.arange(hd // 2) + hd // 2
    x = u[perm]                                  # interleave: x[2i]=u[i], x[2i+1]=u[i+hd/2]
    inter = np.empty(hd)
    inter[0::2] = x[0::2] * cos - x[1::2] * sin
    inter[1::2] = x[0::2] * sin + x[1::2] * cos
    np.testing.assert_allclose(apply_rope(u, cos, sin)[perm], inter, rtol=1e-14, atol=1e-15)


def test_rope_matches_hf_helper():
    from transformers.models.llama.modeling_llama import apply_rotary_pos_emb
    rng = np.random.default_rng(5)
    hd, L, theta = 16, 9, 10000.0
    q = rng.standard_normal((1, 2, L, hd))
    k = rng.standard_normal((1, 1, L, hd))
    pos = np.arange(L)
    cos, sin = rope_cos_sin(pos, hd, theta)
    # HF expects cos/sin over the full head dim: [cos, cos]
    tc = torch.from_numpy(np.concatenate([cos, cos], -1))[None]
    ts = torch.from_numpy(np.concatenate([sin, sin], -1))[None]
    hq, hk = apply_rotary_pos_emb(torch.from_numpy(q), torch.from_numpy(k), tc, ts)
    np.testing.assert_allclose(apply_rope(q, cos[None, None], sin[None, None]), hq.numpy(),
                               rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(apply_rope(k, cos[None, None], sin[None, None]), hk.numpy(),
                               rtol=1e-13, atol=1e-14)


# -------------------------------------------------------------- activations --
def test_activation_closed_forms():
    z = np.array([0.0, 1.0, -2.0, 30.0])
    # silu(z) = z / (1 + e^-z)
    want = [0.0, 1 / (1 + math.exp(-1)), -2 / (1 + math.exp(2)), 30 / (1 + math.exp(-30))]
    np.testing.assert_allclose(silu(z), want, rtol=1e-15)
    # gelu_tanh(1) = 0.5 (1 + tanh(sqrt(2/pi) * 1.044715))
    g1 = 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * 1.044715))
    assert abs(gelu_tanh(np.array([1.0]))[0] - g1) < 1e-15
    assert gelu_tanh(np.array([0.0]))[0] == 0.0
    # large z: both tend to the identity, very negative z to 0
    assert abs(gelu_tanh(np.array([12.0]))[0] - 12.0) < 1e-12
    assert abs(silu(np.array([-60.0]))[0]) < 1e-20


def test_activations_match_library():
    rng = np.random.default_rng(6)
    z = rng.standard_normal(1000) * 4
    t = torch.from_numpy(z)
    np.testing.assert_allclose(silu(z), torch.nn.functional.silu(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(gelu_tanh(z), torch.nn.functional.gelu(t, approximate="tanh").numpy(),
                               rtol=1e-13, atol=1e-15)
    # and the tanh form stays within its known distance of the exact (erf) GELU
    exact = torch.nn.functional.gelu(t).numpy()
    assert np.max(np.abs(gelu_tanh(z) - exact)) < 1e-3
    # float32 inputs stay float32
    assert silu(z.astype(np.float32)).dtype == np.float32


# ---------------------------------------------------------------- attention --
def _brute_attention(q, k, v, q_pos, k_pos, window, softcap):
    """Triple loops in Python floats: for each (t, h): gather allowed keys,
    score, cap, exp-normalise, weight the values."""
    Lq, H, hd = q.shape
    KV = k.shape[1]
    G = H // KV
    out = np.zeros((Lq, H, hd))
    for t in range(Lq):
        for h in range(H):
            j = h // G
            idx = [s for s in range(k.shape[0])
                   if k_pos[s] <= q_pos[t] and (window == 0 or k_pos[s] > q_pos[t] - window)]
            sc = []
            for s in idx:
                dot = 0.0
                for e in range(hd):
                    dot += float(q[t, h, e]) * float(k[s, j, e])
                val = dot / math.sqrt(hd)
                if softcap:
                    val = softcap * math.tanh(val / softcap)
                sc.append(val)
            mx = max(sc)
            ws = [math.exp(a - mx) for a in sc]
            tot = sum(ws)
            for e in range(hd):
                out[t, h, e] = sum(w * float(v[s, j, e]) for w, s in zip(ws, idx)) / tot
    return out


@pytest.mark.parametrize("window,softcap,start", [(0, 0.0, 0), (3, 0.0, 0), (0, 2.5, 0),
                                                  (4, 1.5, 0), (0, 0.0, 5), (3, 0.0, 6)])
def test_attention_brute_force(window, softcap, start):
    rng = np.random.default_rng(7 + window)
    H, KV, hd, Lq = 4, 2, 4, 5
    Lk = start + Lq
    q = rng.standard_normal((Lq, H, hd)) * 2
    k = rng.standard_normal((Lk, KV, hd)) * 2
    v = rng.standard_normal((Lk, KV, hd))
    q_pos = np.arange(start, start + Lq)
    k_pos = np.arange(Lk)
    got = attention_row(q, k, v, q_pos, k_pos, window, softcap)
    want = _brute_attention(q, k, v, q_pos, k_pos, window, softcap)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_attention_hand_case():
    # hd = 2, scale 1/sqrt(2).  k0 = 0 gives score 0; k1 = [sqrt2 ln3, 0] with
    # q = [1, 0] gives score ln 3, so softmax = [1/4, 3/4].
    ln3 = math.log(3.0)
    q = np.array([[[1.0, 0.0]], [[1.0, 0.0]]])                # [2 tokens, 1 head, 2]
    k = np.array([[[0.0, 0.0]], [[math.sqrt(2) * ln3, 0.0]]])
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    pos = np.arange(2)
    out = attention_row(q, k, v, pos, pos, 0, 0.0)
    np.testing.assert_allclose(out[0, 0], [1.0, 0.0], atol=1e-15)     # token 0 sees only key 0
    np.testing.assert_allclose(out[1, 0], [0.25, 0.75], atol=1e-15)
    # window of 1 key: each token sees only itself
    out = attention_row(q, k, v, pos, pos, 1, 0.0)
    np.testing.assert_allclose(out[1, 0], [0.0, 1.0], atol=1e-15)
    # window of 2 keys (its own included) == full causal here
    np.testing.assert_allclose(attention_row(q, k, v, pos, pos, 2, 0.0), attention_row(q, k, v, pos, pos, 0, 0.0))
    # softcap 1: scores 0 and tanh(ln 3) = 0.8
    out = attention_row(q, k, v, pos, pos, 0, 1.0)
    p1 = math.exp(0.8) / (1 + math.exp(0.8))
    np.testing.assert_allclose(out[1, 0], [1 - p1, p1], atol=1e-15)


def test_attention_uniform_keys_average_values():
    # All keys equal -> uniform weights over the key set -> mean of the allowed values.
    rng = np.random.default_rng(8)
    L, H, KV, hd, W = 9, 2, 1, 3, 4
    q = rng.standard_normal((L, H, hd))
    k = np.tile(rng.standard_normal((1, KV, hd)), (L, 1, 1))
    v = rng.standard_normal((L, KV, hd))
    pos = np.arange(L)
    out = attention_row(q, k, v, pos, pos, W, 0.0)
    for t in range(L):
        lo = max(0, t - W + 1)
        np.testing.assert_allclose(out[t, 0], v[lo:t + 1, 0].mean(0), rtol=1e-13)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 4, 8))
    k = rng.standard_normal((1, 2, 8))
    v = rng.standard_normal((1, 2, 8))
    out = attention_row(q, k, v, np.array([0]), np.array([0]), 0, 3.0)
    np.testing.assert_array_equal(out[0, :2], v[0, [0, 0]])
    np.testing.assert_array_equal(out[0, 2:], v[0, [1, 1]])


def test_gqa_equals_mha_with_repeated_kv():
    # DantinoX page: GQA realised by repeating the kv heads (group of G query heads per kv head).
    rng = np.random.default_rng(10)
    L, H, KV, hd = 7, 6, 2, 8
    q = rng.standard_normal((L, H, hd))
    k = rng.standard_normal((L, KV, hd))
    v = rng.standard_normal((L, KV, hd))
    pos = np.arange(L)
    g = attention_row(q, k, v, pos, pos, 0, 0.0)
    m = attention_row(q, np.repeat(k, H // KV, axis=1), np.repeat(v, H // KV, axis=1), pos, pos, 0, 0.0)
    np.testing.assert_allclose(g, m, rtol=1e-14)


def test_attention_matches_torch_sdpa():
    # library routine: torch's scaled_dot_product_attention (math path, fp64) with enable_gqa
    rng = np.random.default_rng(11)
    L, H, KV, hd, W = 20, 8, 2, 16, 6
    q = rng.standard_normal((L, H, hd))
    k = rng.standard_normal((L, KV, hd))
    v = rng.standard_normal((L, KV, hd))
    pos = np.arange(L)
    for window in (0, W):
        allowed = pos[None, :] <= pos[:, None]
        if window:
            allowed &= pos[None, :] > pos[:, None] - window
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).transpose(0, 1)[None], torch.from_numpy(k).transpose(0, 1)[None],
            torch.from_numpy(v).transpose(0, 1)[None], attn_mask=torch.from_numpy(allowed),
            enable_gqa=True)[0].transpose(0, 1).numpy()
        np.testing.assert_allclose(attention_row(q, k, v, pos, pos, window, 0.0), ref, rtol=1e-12,
                                   atol=1e-13)


def test_attention_causal_invariance_and_limits():
    rng = np.random.default_rng(12)
    L, H, KV, hd = 12, 4, 2, 8
    q = rng.standard_normal((L, H, hd))
    k = rng.standard_normal((L, KV, hd))
    v = rng.standard_normal((L, KV, hd))
    pos = np.arange(L)
    base = attention_row(q, k, v, pos, pos, 0, 0.0)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[8:], k2[8:], v2[8:] = 99.0, -7.0, 123.0
    alt = attention_row(q2, k2, v2, pos, pos, 0, 0.0)
    np.testing.assert_array_equal(base[:8], alt[:8])           # future tokens change nothing
    assert not np.allclose(base[8:], alt[8:])
    # a window at least L wide is full causal attention
    np.testing.assert_allclose(attention_row(q, k, v, pos, pos, L, 0.0), base, rtol=1e-14)
    # a huge softcap is no cap
    np.testing.assert_allclose(attention_row(q, k, v, pos, pos, 0, 1e12), base, rtol=1e-9)
    # a small cap squeezes the scores: result differs
    assert not np.allclose(attention_row(q, k, v, pos, pos, 0, 0.5), base, rtol=1e-3)
