"""Pins of the oracle's norm / MLP / bias / sandwich options: mojolearn
``norm='layernorm'`` + ``norm_bias``, ``mlp`` = gelu / gelu_tanh (ungated) and
geglu (gated, exact GELU), ``o_bias``, ``mlp_bias``, and Gemma's sandwich
norms (the dew DecoderBlock page's output norms; the gemma4 text page's block
equations).

* Closed forms: LayerNorm of a hand vector, its shift invariance; exact GELU
  at 0, the identity gelu(z) - gelu(-z) = z (Phi(z) + Phi(-z) = 1), and its
  distance from the tanh form.
* Library routines as independent implementations: torch ``layer_norm`` and
  ``gelu``; whole Hugging Face decoder layers, each with its own rotary table,
  norms and MLP: LlamaDecoderLayer with attention and MLP biases,
  GemmaDecoderLayer with the exact GELU, Gemma2DecoderLayer (sandwich norms,
  softcap, window), StableLmDecoderLayer (LayerNorm with bias, partial
  rotary, q/k/v biases) and Starcoder2DecoderLayer (LayerNorm with bias,
  ungated GELU MLP with biases, biased o_proj).
* Invariants with every option on: decode equals prefill bitwise (rowwise
  layout), chunked continuation equals the whole prefill.
"""
import math

import numpy as np
import pytest
import torch

from gqa_causal_attention_amd.workloads import random_block
from oracle import OracleState, block_forward, block_step, gelu_erf, gelu_tanh, layer_norm
from tests.conftest import rel_err
from tests.test_oracle_block import _MLP_NAMES, _NORM_NAMES, _attn_names, _causal_mask, _hf_load


def test_layer_norm_closed_form_and_library():
    x = np.array([1.0, 2.0, 3.0])
    # mean 2, population variance 2/3
    np.testing.assert_allclose(layer_norm(x, np.ones(3), None, 0.0), (x - 2.0) / math.sqrt(2.0 / 3.0), rtol=1e-15)
    w, b = np.array([2.0, -1.0, 0.5]), np.array([0.1, 0.2, 0.3])
    np.testing.assert_allclose(layer_norm(x, w, b, 0.0), (x - 2.0) / math.sqrt(2.0 / 3.0) * w + b, rtol=1e-15)
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 33))
    np.testing.assert_allclose(layer_norm(z + 7.0, w[:1].repeat(33), None, 1e-5),
                               layer_norm(z, w[:1].repeat(33), None, 1e-5), atol=1e-12)
    g, bb = rng.standard_normal(33), rng.standard_normal(33)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (33,), torch.from_numpy(g), torch.from_numpy(bb),
                                         eps=1e-5).numpy()
    np.testing.assert_allclose(layer_norm(z, g, bb, 1e-5), ref, atol=1e-12)


def test_gelu_erf_closed_forms():
    z = np.linspace(-6, 6, 241)
    g = gelu_erf(z)
    assert gelu_erf(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(g - gelu_erf(-z), z, atol=1e-14)
    # Phi(1) = 0.8413447460685429 (standard normal table)
    np.testing.assert_allclose(gelu_erf(np.array([1.0])), [0.8413447460685429], rtol=1e-13)
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="none").numpy()
    np.testing.assert_allclose(g, ref, atol=1e-14)
    # the two GELU forms are different functions, close to each other
    d = np.abs(g - gelu_tanh(z))
    assert 1e-5 < d.max() < 1e-3


def _run_hf(layer, rot_cls, hc, x, mask=None):
    L = x.shape[1]
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(L)[None].expand(x.shape[0], L)
    cos, sin = rot_cls(hc)(xt, pos)
    with torch.no_grad():
        out = layer(xt, attention_mask=_causal_mask(L) if mask is None else mask, position_ids=pos,
                    position_embeddings=(cos, sin))
    return (out[0] if isinstance(out, tuple) else out).numpy()


def test_block_matches_hf_llama_layer_attention_and_mlp_biases():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    cfg, W = random_block(41, qkv_bias=True, o_bias=True, mlp_bias=True)
    hc = LlamaConfig(hidden_size=64, intermediate_size=96, num_attention_heads=4, num_key_value_heads=2,
                     head_dim=16, rms_norm_eps=1e-6, attention_bias=True, mlp_bias=True,
                     rope_parameters={"rope_theta": 1e4, "rope_type": "default"}, max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = LlamaDecoderLayer(hc, layer_idx=0).double().eval()
    names = {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES,
             **{f"self_attn.{p}_proj.bias": f"{p}_proj.bias" for p in "qkvo"},
             **{f"mlp.{p}_proj.bias": f"{p}_proj.bias" for p in ("gate", "up", "down")}}
    res = _hf_load(layer, W, names)
    assert not res.missing_keys and not res.unexpected_keys
    x = np.random.default_rng(42).standard_normal((2, 12, 64)).astype(np.float32)
    ref = _run_hf(layer, LlamaRotaryEmbedding, hc, x)
    got = block_forward(cfg, W, x, dtype=np.float64)
    assert rel_err(got - x, ref - x) < 2e-5
    for name in ("o_proj.bias", "gate_proj.bias", "up_proj.bias", "down_proj.bias"):
        W2 = dict(W, **{name: np.zeros_like(W[name])})
        assert rel_err(block_forward(cfg, W2, x, dtype=np.float64) - x, ref - x) > 1e-3, name


def test_block_matches_hf_gemma_layer_exact_geglu():
    from transformers import GemmaConfig
    from transformers.models.gemma.modeling_gemma import GemmaDecoderLayer, GemmaRotaryEmbedding
    cfg, W = random_block(43, d_model=64, n_heads=4, n_kv_heads=1, head_dim=32, intermediate=96,
                          norm="rmsnorm_offset", mlp="geglu")
    # larger MLP pre-activations so the two GELU forms are told apart
    W["gate_proj.weight"] = W["gate_proj.weight"] * np.float32(60.0)
    hc = GemmaConfig(hidden_size=64, intermediate_size=96, num_attention_heads=4, num_key_value_heads=1,
                     head_dim=32, rms_norm_eps=1e-6, hidden_act="gelu",
                     rope_parameters={"rope_theta": 1e4, "rope_type": "default"}, max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = GemmaDecoderLayer(hc, layer_idx=0).double().eval()
    res = _hf_load(layer, W, {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES})
    assert not res.missing_keys and not res.unexpected_keys
    x = np.random.default_rng(44).standard_normal((1, 13, 64)).astype(np.float32)
    ref = _run_hf(layer, GemmaRotaryEmbedding, hc, x)
    got = block_forward(cfg, W, x, dtype=np.float64)
    # agreement ~1e-7 (Gemma's RMSNorm runs in float32); the tanh form is ~2e-5 away
    assert rel_err(got - x, ref - x) < 2e-6
    tanh_form = block_forward(dict(cfg, mlp="geglu_tanh"), W, x, dtype=np.float64)
    assert rel_err(tanh_form - x, ref - x) > 5e-6


@pytest.mark.parametrize("window", [0, 5])
def test_block_matches_hf_gemma2_layer_sandwich_norms(window):
    from transformers import Gemma2Config
    from transformers.models.gemma2.modeling_gemma2 import Gemma2DecoderLayer, Gemma2RotaryEmbedding
    cfg, W = random_block(45, d_model=64, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=64,
                          norm="rmsnorm_offset", mlp="geglu_tanh", attn_softcap=2.0, window=window,
                          sandwich_norms=True)
    W["q_proj.weight"] = W["q_proj.weight"] * np.float32(10.0)
    hc = Gemma2Config(hidden_size=64, intermediate_size=64, num_attention_heads=4, num_key_value_heads=2,
                      head_dim=32, rms_norm_eps=1e-6, query_pre_attn_scalar=32, attn_logit_softcapping=2.0,
                      sliding_window=window or None, hidden_act="gelu_pytorch_tanh",
                      rope_parameters={"rope_theta": 1e4, "rope_type": "default"}, max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = Gemma2DecoderLayer(hc, layer_idx=0).double().eval()
    names = {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES,
             "pre_feedforward_layernorm.weight": "pre_feedforward_layernorm.weight",
             "post_feedforward_layernorm.weight": "post_feedforward_layernorm.weight"}
    res = _hf_load(layer, W, names)
    assert not res.missing_keys and not res.unexpected_keys
    L = 14
    x = np.random.default_rng(46).standard_normal((1, L, 64)).astype(np.float32)
    ref = _run_hf(layer, Gemma2RotaryEmbedding, hc, x, mask=_causal_mask(L, window))
    got = block_forward(cfg, W, x, dtype=np.float64)
    assert rel_err(got - x, ref - x) < 5e-5
    plain = block_forward(dict(cfg, sandwich_norms=False), W, x, dtype=np.float64)
    assert rel_err(plain - x, ref - x) > 1e-2


def test_block_matches_hf_stablelm_layer_layernorm_partial_rotary():
    from transformers import StableLmConfig
    from transformers.models.stablelm.modeling_stablelm import StableLmDecoderLayer, StableLmRotaryEmbedding
    cfg, W = random_block(47, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                          norm="layernorm", norm_bias=True, qkv_bias=True, rope_dim=4, norm_eps=1e-5)
    hc = StableLmConfig(hidden_size=64, intermediate_size=96, num_attention_heads=4, num_key_value_heads=2,
                        layer_norm_eps=1e-5, use_qkv_bias=True, use_parallel_residual=False,
                        rope_parameters={"rope_type": "default", "rope_theta": 1e4, "partial_rotary_factor": 0.25},
                        max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = StableLmDecoderLayer(hc, layer_idx=0).double().eval()
    names = {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES,
             **{f"self_attn.{p}_proj.bias": f"{p}_proj.bias" for p in "qkv"},
             "input_layernorm.bias": "input_layernorm.bias",
             "post_attention_layernorm.bias": "post_attention_layernorm.bias"}
    res = _hf_load(layer, W, names)
    assert not res.missing_keys and not res.unexpected_keys
    x = np.random.default_rng(48).standard_normal((2, 11, 64)).astype(np.float32)
    ref = _run_hf(layer, StableLmRotaryEmbedding, hc, x)
    got = block_forward(cfg, W, x, dtype=np.float64)
    assert rel_err(got - x, ref - x) < 2e-5
    for over in (dict(norm="rmsnorm"), dict(rope_dim=None)):
        assert rel_err(block_forward(dict(cfg, **over), W, x, dtype=np.float64) - x, ref - x) > 1e-3
    W2 = dict(W, **{"post_attention_layernorm.bias": np.zeros(64, np.float32)})
    assert rel_err(block_forward(cfg, W2, x, dtype=np.float64) - x, ref - x) > 1e-3


@pytest.mark.parametrize("act", ["gelu_tanh", "gelu"])
def test_block_matches_hf_starcoder2_layer_ungated_mlp(act):
    from transformers import Starcoder2Config
    from transformers.models.starcoder2.modeling_starcoder2 import (Starcoder2DecoderLayer,
                                                                    Starcoder2RotaryEmbedding)
    cfg, W = random_block(49, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=96,
                          norm="layernorm", norm_bias=True, qkv_bias=True, o_bias=True, mlp_bias=True,
                          mlp=act, norm_eps=1e-5)
    assert "gate_proj.weight" not in W
    W["up_proj.weight"] = W["up_proj.weight"] * np.float32(60.0)
    hc = Starcoder2Config(hidden_size=64, intermediate_size=96, num_attention_heads=4, num_key_value_heads=2,
                          norm_epsilon=1e-5, use_bias=True,
                          hidden_act="gelu_pytorch_tanh" if act == "gelu_tanh" else "gelu",
                          rope_parameters={"rope_type": "default", "rope_theta": 1e4},
                          max_position_embeddings=64, residual_dropout=0.0, embedding_dropout=0.0)
    hc._attn_implementation = "eager"
    layer = Starcoder2DecoderLayer(hc, layer_idx=0).double().eval()
    names = {**_attn_names(), **_NORM_NAMES,
             **{f"self_attn.{p}_proj.bias": f"{p}_proj.bias" for p in "qkvo"},
             "mlp.c_fc.weight": "up_proj.weight", "mlp.c_fc.bias": "up_proj.bias",
             "mlp.c_proj.weight": "down_proj.weight", "mlp.c_proj.bias": "down_proj.bias",
             "input_layernorm.bias": "input_layernorm.bias",
             "post_attention_layernorm.bias": "post_attention_layernorm.bias"}
    res = _hf_load(layer, W, names)
    assert not res.missing_keys and not res.unexpected_keys
    x = np.random.default_rng(50).standard_normal((1, 12, 64)).astype(np.float32)
    ref = _run_hf(layer, Starcoder2RotaryEmbedding, hc, x)
    got = block_forward(cfg, W, x, dtype=np.float64)
    # agreement ~1e-7 (float32 rotary angles); the other GELU form is ~2e-5 away
    assert rel_err(got - x, ref - x) < 2e-6
    other = "gelu" if act == "gelu_tanh" else "gelu_tanh"
    assert rel_err(block_forward(dict(cfg, mlp=other), W, x, dtype=np.float64) - x, ref - x) > 5e-6


ALL_OPTIONS = [
    dict(norm="layernorm", norm_bias=True, sandwich_norms=True, mlp="geglu", o_bias=True, mlp_bias=True,
         qkv_bias=True, qk_norm=True),
    dict(norm="rmsnorm_offset", sandwich_norms=True, mlp="gelu", mlp_bias=True, window=5, attn_softcap=3.0),
    dict(norm="layernorm", mlp="gelu_tanh", o_bias=True, rope_dim=6),
]


@pytest.mark.parametrize("over", ALL_OPTIONS)
def test_decode_and_chunks_equal_prefill_with_options(over):
    cfg, W = random_block(51, **over)
    L = 10
    x = np.random.default_rng(52).standard_normal((2, L, 64)).astype(np.float32)
    full = block_forward(cfg, W, x, layout="rowwise")
    # the rowwise layout (matrix-vector per token) agrees with the batched one
    assert rel_err(full, block_forward(cfg, W, x)) < 1e-6
    st = OracleState(cfg, 2, L)
    parts = [block_forward(cfg, W, x[:, :4], st, layout="rowwise")]
    parts += [block_step(cfg, W, x[:, t], st, layout="rowwise") for t in range(4, L)]
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), full)
    st2 = OracleState(cfg, 2, L)
    chunks = [block_forward(cfg, W, x[:, a:b], st2) for a, b in ((0, 3), (3, 7), (7, L))]
    assert rel_err(np.concatenate(chunks, axis=1), block_forward(cfg, W, x)) < 1e-6
