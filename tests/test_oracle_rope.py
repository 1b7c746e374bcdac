"""Pins of the oracle's RoPE options: ``rope_scaling`` (linear, Llama 3) and
partial rotary (``rope_dim``) of the mojolearn TransformerBlock parameter
list, with the rotation and frequencies of the DantinoX "Core Layers" page
(Positional Encoding / RoPE).

* Hugging Face's rope-init functions (the layer the mojolearn page says its
  block computes) give the inverse frequencies independently, in float32.
* Closed forms: linear scaling at position p equals plain RoPE at p / f; the
  Llama 3 ramp keeps short wavelengths, divides long ones by the factor and
  is continuous and monotone between.
* Partial rotary is checked against an explicit block-diagonal rotation
  matrix built here, against Hugging Face's partial-rotary attention step
  (StableLM's split / rotate / concatenate), and by the relative-position
  property of the rotated dot product.
* Whole block: Hugging Face's LlamaDecoderLayer with linear and Llama 3
  scaling; decode equals prefill bitwise with every option on.
"""
import math

import numpy as np
import pytest
import torch

from gqa_causal_attention_amd.workloads import random_block
from oracle import OracleState, apply_rope, block_forward, block_step, rope_cos_sin, rope_inv_freq
from tests.conftest import rel_err

LLAMA31 = {"type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
           "original_max_position_embeddings": 8192}


def _hf_inv_freq(rope_parameters, head_dim=128):
    from transformers import LlamaConfig
    from transformers.modeling_rope_utils import ROPE_INIT_FUNCTIONS
    hc = LlamaConfig(hidden_size=32 * head_dim, num_attention_heads=32, head_dim=head_dim,
                     rope_parameters=dict(rope_parameters), max_position_embeddings=131072)
    inv, attn_factor = ROPE_INIT_FUNCTIONS[rope_parameters["rope_type"]](hc, None)
    assert attn_factor == 1.0
    return inv.double().numpy()


@pytest.mark.parametrize("partial", [1.0, 0.5, 0.25])
@pytest.mark.parametrize("scaling", [{"type": "linear", "factor": 4.0}, LLAMA31,
                                     dict(LLAMA31, factor=32.0, low_freq_factor=2.0, high_freq_factor=8.0,
                                          original_max_position_embeddings=4096)])
def test_inv_freq_matches_hf_rope_init(scaling, partial):
    theta = 500000.0
    rp = {"rope_type": scaling["type"], "rope_theta": theta, "partial_rotary_factor": partial,
          **{k: v for k, v in scaling.items() if k != "type"}}
    ref = _hf_inv_freq(rp)
    rd = int(128 * partial)
    got = rope_inv_freq(rd, theta, scaling)
    assert got.shape == ref.shape == (rd // 2,)
    # Hugging Face forms the frequencies in float32
    assert np.max(np.abs(got - ref) / got) < 2e-6


def test_linear_scaling_is_position_over_factor():
    f = 4.0
    p = np.arange(0, 4096, 4)
    c1, s1 = rope_cos_sin(p, 64, 10000.0, {"type": "linear", "factor": f})
    c0, s0 = rope_cos_sin(p // 4, 64, 10000.0)
    np.testing.assert_allclose(c1, c0, atol=1e-12)
    np.testing.assert_allclose(s1, s0, atol=1e-12)


def test_llama3_ramp_closed_form():
    theta, rd = 500000.0, 128
    base = 500000.0 ** (-np.arange(0, rd, 2) / rd)
    got = rope_inv_freq(rd, theta, LLAMA31)
    wl = 2 * math.pi / base
    short, long_ = wl < 8192 / 4.0, wl > 8192 / 1.0
    mid = ~short & ~long_
    assert short.any() and long_.any() and mid.any()
    np.testing.assert_array_equal(got[short], base[short])          # high frequencies kept
    np.testing.assert_allclose(got[long_], base[long_] / 8.0, rtol=1e-15)  # low ones interpolated
    # between: strictly inside the two ends, and the blend's weight is linear
    # in n / wavelength (the ramp), so it reaches 0 and 1 at the two ends
    assert np.all(got[mid] < base[mid]) and np.all(got[mid] > base[mid] / 8.0)
    s = (got[mid] - base[mid] / 8.0) / (base[mid] - base[mid] / 8.0)
    np.testing.assert_allclose(s, (8192 / wl[mid] - 1.0) / (4.0 - 1.0), rtol=1e-12)
    # frequencies still fall with the pair index
    assert np.all(np.diff(got) < 0)


def _rotation_matrix(p, hd, rd, inv):
    R = np.eye(hd)
    h = rd // 2
    for i in range(h):
        a = p * inv[i]
        R[i, i], R[i, i + h] = math.cos(a), -math.sin(a)
        R[i + h, i], R[i + h, i + h] = math.sin(a), math.cos(a)
    return R


@pytest.mark.parametrize("hd,rd", [(16, 16), (16, 8), (64, 16), (128, 64), (24, 6)])
def test_partial_rotary_is_block_rotation(hd, rd):
    rng = np.random.default_rng(hd + rd)
    u = rng.standard_normal((5, hd))
    pos = np.array([0, 1, 7, 100, 4095])
    scaling = {"type": "linear", "factor": 2.0}
    inv = 10000.0 ** (-np.arange(0, rd, 2) / rd) / 2.0
    c, s = rope_cos_sin(pos, rd, 10000.0, scaling)
    got = apply_rope(u, c, s)
    for j, p in enumerate(pos):
        np.testing.assert_allclose(got[j], _rotation_matrix(p, hd, rd, inv) @ u[j], atol=1e-12)
    np.testing.assert_array_equal(got[:, rd:], u[:, rd:])              # pass-through exact
    # rotated dot products depend on the offset only
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    def dot(p, m):
        cp, sp = rope_cos_sin(np.array([p]), rd, 10000.0, scaling)
        cm, sm = rope_cos_sin(np.array([m]), rd, 10000.0, scaling)
        return float(apply_rope(q[None], cp, sp)[0] @ apply_rope(k[None], cm, sm)[0])
    assert abs(dot(10, 3) - dot(107, 100)) < 1e-9
    assert abs(dot(10, 3) - dot(11, 3)) > 1e-6


def test_partial_rotary_matches_hf_split_rotate_concat():
    from transformers import StableLmConfig
    from transformers.models.stablelm.modeling_stablelm import StableLmRotaryEmbedding, apply_rotary_pos_emb
    hd, H, L, partial = 64, 4, 12, 0.25
    hc = StableLmConfig(hidden_size=H * hd, num_attention_heads=H, max_position_embeddings=64,
                        rope_parameters={"rope_type": "default", "rope_theta": 10000.0,
                                         "partial_rotary_factor": partial})
    rd = int(hd * partial)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, H, L, hd))
    k = rng.standard_normal((1, H, L, hd))
    pos = torch.arange(3, 3 + L)[None]
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    cos, sin = StableLmRotaryEmbedding(hc)(qt, pos)
    qr, kr = apply_rotary_pos_emb(qt[..., :rd], kt[..., :rd], cos, sin)
    ref_q = torch.cat([qr, qt[..., rd:]], -1).numpy()
    ref_k = torch.cat([kr, kt[..., rd:]], -1).numpy()
    c, s = rope_cos_sin(np.arange(3, 3 + L), rd, 10000.0)
    got_q = apply_rope(q, c[None, None], s[None, None])
    got_k = apply_rope(k, c[None, None], s[None, None])
    assert np.max(np.abs(got_q - ref_q)) < 1e-5 and np.max(np.abs(got_k - ref_k)) < 1e-5


# with head_dim 16 and base 1e4 the wavelengths run from 6.3 to 2e4, so an
# original context of 64 puts pairs in all three regions of the Llama 3 ramp
@pytest.mark.parametrize("scaling", [{"type": "linear", "factor": 4.0},
                                     dict(LLAMA31, original_max_position_embeddings=64)])
def test_block_matches_hf_llama_layer_scaled_rope(scaling):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    from tests.test_oracle_block import _MLP_NAMES, _NORM_NAMES, _attn_names, _causal_mask, _hf_load
    cfg, W = random_block(11, rope_theta=10000.0, rope_scaling=scaling, max_positions=256)
    inv = rope_inv_freq(cfg["head_dim"], 10000.0, scaling)
    base = 10000.0 ** (-np.arange(0, cfg["head_dim"], 2) / cfg["head_dim"])
    assert np.any(inv != base)
    L = 40
    x = np.random.default_rng(3).standard_normal((1, L, cfg["d_model"])).astype(np.float32)
    rp = {"rope_type": scaling["type"], "rope_theta": 10000.0, **{k: v for k, v in scaling.items() if k != "type"}}
    hc = LlamaConfig(hidden_size=cfg["d_model"], intermediate_size=cfg["intermediate"],
                     num_attention_heads=cfg["n_heads"], num_key_value_heads=cfg["n_kv_heads"],
                     head_dim=cfg["head_dim"], rms_norm_eps=cfg["norm_eps"], rope_parameters=rp,
                     max_position_embeddings=256)
    hc._attn_implementation = "eager"
    layer = LlamaDecoderLayer(hc, layer_idx=0).double().eval()
    res = _hf_load(layer, W, {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES})
    assert not res.missing_keys and not res.unexpected_keys
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(L)[None]
    cos, sin = LlamaRotaryEmbedding(hc)(xt, pos)
    with torch.no_grad():
        ref = layer(xt, attention_mask=_causal_mask(L), position_ids=pos,
                    position_embeddings=(cos, sin)).numpy()
    got = block_forward(cfg, W, x, dtype=np.float64)
    # Hugging Face forms its rotary angles in float32
    assert rel_err(got, ref) < 2e-6
    assert rel_err(got - x, ref - x) < 2e-5
    # the scaling is visible in the output: plain RoPE gives a different block
    plain = block_forward(dict(cfg, rope_scaling=None), W, x, dtype=np.float64)
    assert rel_err(plain - x, ref - x) > 1e-3


@pytest.mark.parametrize("window", [0, 5])
def test_decode_equals_prefill_bitwise_scaled_partial(window):
    cfg, W = random_block(12, rope_dim=6, rope_scaling=dict(LLAMA31, original_max_position_embeddings=32),
                          qk_norm=True, qkv_bias=True, window=window)
    L = 11
    x = np.random.default_rng(4).standard_normal((2, L, cfg["d_model"])).astype(np.float32)
    full = block_forward(cfg, W, x, layout="rowwise")
    st = OracleState(cfg, 2, L)
    steps = np.concatenate([block_step(cfg, W, x[:, t], st, layout="rowwise") for t in range(L)], axis=1)
    np.testing.assert_array_equal(steps, full)
    # partial rotary: dimensions past rope_dim carry no position, so the
    # block with rope_dim=6 differs from the fully rotated one
    whole = block_forward(dict(cfg, rope_dim=None), W, x, layout="rowwise")
    assert rel_err(whole - x, full - x) > 1e-3
