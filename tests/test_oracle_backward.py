"""Pins of the oracle's backward (mojolearn ``TransformerBlock.backward``:
gradients of a zero-state prefill with respect to x and the nine weights).

* Brute force: central finite differences of the float64 forward along random
  directions, for x and every weight, with and without a window.
* A library routine as an independent implementation: torch autograd through
  Hugging Face's LlamaDecoderLayer (float64, its own rotary table, causal or
  sliding-window mask), the layer the mojolearn page says its block computes.
* The page's contract: non-default options raise; weight gradients are sums
  over the B * L tokens (two rows give the sum of their one-row gradients).
"""
import numpy as np
import pytest
import torch

from gqa_causal_attention_amd.workloads import random_block
from oracle import BACKWARD_WEIGHTS, block_backward, block_forward
from tests.conftest import rel_err
from tests.test_oracle_block import _MLP_NAMES, _NORM_NAMES, _attn_names, _causal_mask, _hf_load


def _tiny(seed, **over):
    return random_block(seed, d_model=16, n_heads=4, n_kv_heads=2, head_dim=8, intermediate=24, **over)


@pytest.mark.parametrize("window", [0, 3])
def test_backward_matches_finite_differences(window):
    cfg, W = _tiny(61, window=window)
    W = {k: v.astype(np.float64) for k, v in W.items()}
    rng = np.random.default_rng(62)
    x = rng.standard_normal((2, 6, 16))
    dy = rng.standard_normal((2, 6, 16))
    grads = block_backward(cfg, W, x, dy)
    loss = lambda xx, WW: float(np.sum(block_forward(cfg, WW, xx, dtype=np.float64) * dy))
    eps = 1e-6
    for name in ("x",) + BACKWARD_WEIGHTS:
        base = x if name == "x" else W[name]
        for trial in range(2):
            dirn = rng.standard_normal(base.shape)
            if name == "x":
                fp, fm = loss(x + eps * dirn, W), loss(x - eps * dirn, W)
            else:
                fp = loss(x, dict(W, **{name: W[name] + eps * dirn}))
                fm = loss(x, dict(W, **{name: W[name] - eps * dirn}))
            fd = (fp - fm) / (2 * eps)
            an = float(np.sum(grads[name] * dirn))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, trial, fd, an)
        assert grads[name].shape == base.shape


@pytest.mark.parametrize("window", [0, 5])
def test_backward_matches_hf_llama_autograd(window):
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    cfg, W = random_block(63, window=window)
    hc = LlamaConfig(hidden_size=64, intermediate_size=96, num_attention_heads=4, num_key_value_heads=2,
                     head_dim=16, rms_norm_eps=1e-6, rope_parameters={"rope_theta": 1e4, "rope_type": "default"},
                     max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = LlamaDecoderLayer(hc, layer_idx=0).double()
    names = {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES}
    res = _hf_load(layer, W, names)
    assert not res.missing_keys and not res.unexpected_keys
    rng = np.random.default_rng(64)
    L = 12
    x = rng.standard_normal((2, L, 64))
    dy = rng.standard_normal((2, L, 64))
    xt = torch.tensor(x, requires_grad=True)
    pos = torch.arange(L)[None].expand(2, L)
    cos, sin = LlamaRotaryEmbedding(hc)(xt, pos)
    out = layer(xt, attention_mask=_causal_mask(L, window), position_ids=pos, position_embeddings=(cos, sin))
    out = out[0] if isinstance(out, tuple) else out
    (out * torch.from_numpy(dy)).sum().backward()
    got = block_backward(cfg, W, x, dy)
    assert rel_err(got["x"], xt.grad.numpy()) < 2e-6
    params = dict(layer.named_parameters())
    for hf_name, ours in names.items():
        assert rel_err(got[ours], params[hf_name].grad.numpy()) < 2e-6, ours


def test_backward_sums_over_tokens_and_rows():
    cfg, W = _tiny(65)
    rng = np.random.default_rng(66)
    x = rng.standard_normal((2, 5, 16))
    dy = rng.standard_normal((2, 5, 16))
    both = block_backward(cfg, W, x, dy)
    one = [block_backward(cfg, W, x[i:i + 1], dy[i:i + 1]) for i in range(2)]
    for name in BACKWARD_WEIGHTS:
        np.testing.assert_allclose(both[name], one[0][name] + one[1][name], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(both["x"], np.concatenate([one[0]["x"], one[1]["x"]]), rtol=1e-12)


@pytest.mark.parametrize("over", [dict(qkv_bias=True), dict(attn_softcap=5.0), dict(norm="rmsnorm_offset"),
                                  dict(mlp="geglu_tanh"), dict(qk_norm=True), dict(rope_dim=4),
                                  dict(sandwich_norms=True)])
def test_backward_refuses_other_options(over):
    cfg, W = _tiny(67, **over)
    with pytest.raises(ValueError):
        block_backward(cfg, W, np.zeros((1, 3, 16)), np.zeros((1, 3, 16)))
