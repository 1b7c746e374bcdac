"""Whole-block pins of the CPU oracle.

* Library routines run on the CPU as independent implementations of the same
  layer: Hugging Face's LlamaDecoderLayer (the formulation the mojolearn page
  says its block computes), Qwen3DecoderLayer (q/k/v biases with qk_norm
  before RoPE), GemmaDecoderLayer ((1 + w) RMSNorm and the tanh-GELU gated
  MLP) and Gemma2Attention (tanh softcap of the scores).  Each gets its own
  rotary table and its own softmax; the oracle's helpers are not used on the
  library side.
* The page's invariants: token-by-token decode equals one prefill (bitwise in
  the oracle's rowwise layout), chunked continuation equals the whole
  prefill, batch rows are independent, per-row cache lengths.
"""
import numpy as np
import pytest
import torch

from gqa_causal_attention_amd.workloads import make_workload, random_block
from oracle import OracleState, block_forward, block_step
from tests.conftest import rel_err


def _hf_load(layer, W, names):
    sd = {}
    for hf_name, ours in names.items():
        sd[hf_name] = torch.from_numpy(np.asarray(W[ours], dtype=np.float64))
    missing = layer.load_state_dict(sd, strict=False)
    return missing


def _attn_names(prefix="self_attn."):
    return {f"{prefix}{p}_proj.weight": f"{p}_proj.weight" for p in "qkvo"}


_MLP_NAMES = {f"mlp.{p}_proj.weight": f"{p}_proj.weight" for p in ("gate", "up", "down")}
_NORM_NAMES = {"input_layernorm.weight": "input_layernorm.weight",
               "post_attention_layernorm.weight": "post_attention_layernorm.weight"}


def _causal_mask(L, window=0, dtype=torch.float64):
    pos = torch.arange(L)
    allowed = pos[None, :] <= pos[:, None]
    if window:
        allowed &= pos[None, :] > pos[:, None] - window
    m = torch.zeros(L, L, dtype=dtype)
    m[~allowed] = float("-inf")
    return m[None, None]


def test_block_matches_hf_llama_layer():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaDecoderLayer, LlamaRotaryEmbedding
    wl = make_workload("tiny_llama_f32")
    cfg, W, x = wl["cfg"], wl["weights"], wl["x"]
    hc = LlamaConfig(hidden_size=64, intermediate_size=172, num_attention_heads=4,
                     num_key_value_heads=2, head_dim=16, rms_norm_eps=1e-6,
                     rope_parameters={"rope_theta": 1e4, "rope_type": "default"},
                     max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = LlamaDecoderLayer(hc, layer_idx=0).double().eval()
    res = _hf_load(layer, W, {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES})
    assert not res.missing_keys and not res.unexpected_keys
    L = x.shape[1]
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(L)[None]
    cos, sin = LlamaRotaryEmbedding(hc)(xt, pos)
    with torch.no_grad():
        ref = layer(xt, attention_mask=_causal_mask(L), position_ids=pos,
                    position_embeddings=(cos, sin)).numpy()
    got = block_forward(cfg, W, x, dtype=np.float64)
    # HF forms its rotary angles and softmax in float32: agreement to ~1e-7
    assert rel_err(got, ref) < 2e-6
    assert rel_err(got - x, ref - x) < 2e-5


def test_block_matches_hf_qwen3_layer_bias_qknorm():
    from transformers import Qwen3Config
    from transformers.models.qwen3.modeling_qwen3 import Qwen3DecoderLayer, Qwen3RotaryEmbedding
    cfg, W = random_block(21, d_model=64, n_heads=4, n_kv_heads=2, head_dim=16, intermediate=80,
                          qkv_bias=True, qk_norm=True)
    hc = Qwen3Config(hidden_size=64, intermediate_size=80, num_attention_heads=4,
                     num_key_value_heads=2, head_dim=16, rms_norm_eps=1e-6, attention_bias=True,
                     rope_parameters={"rope_theta": 1e4, "rope_type": "default"},
                     max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = Qwen3DecoderLayer(hc, layer_idx=0).double().eval()
    names = {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES,
             "self_attn.q_proj.bias": "q_proj.bias", "self_attn.k_proj.bias": "k_proj.bias",
             "self_attn.v_proj.bias": "v_proj.bias", "self_attn.q_norm.weight": "q_norm.weight",
             "self_attn.k_norm.weight": "k_norm.weight"}
    res = _hf_load(layer, W, names)
    assert res.missing_keys == ["self_attn.o_proj.bias"]
    with torch.no_grad():
        layer.self_attn.o_proj.bias.zero_()
    x = np.random.default_rng(22).standard_normal((2, 11, 64)).astype(np.float32)
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(11)[None].expand(2, 11)
    cos, sin = Qwen3RotaryEmbedding(hc)(xt, pos)
    with torch.no_grad():
        ref = layer(xt, attention_mask=_causal_mask(11), position_ids=pos,
                    position_embeddings=(cos, sin)).numpy()
    got = block_forward(cfg, W, x, dtype=np.float64)
    assert rel_err(got - x, ref - x) < 2e-5
    # and the biases / q-k norms matter
    W2 = dict(W, **{"k_proj.bias": np.zeros_like(W["k_proj.bias"])})
    assert rel_err(block_forward(cfg, W2, x, dtype=np.float64) - x, ref - x) > 1e-3


def test_block_matches_hf_gemma_layer_offset_norm_geglu():
    from transformers import GemmaConfig
    from transformers.models.gemma.modeling_gemma import GemmaDecoderLayer, GemmaRotaryEmbedding
    cfg, W = random_block(23, d_model=64, n_heads=4, n_kv_heads=1, head_dim=32, intermediate=96,
                          norm="rmsnorm_offset", mlp="geglu_tanh")
    hc = GemmaConfig(hidden_size=64, intermediate_size=96, num_attention_heads=4,
                     num_key_value_heads=1, head_dim=32, rms_norm_eps=1e-6,
                     hidden_activation="gelu_pytorch_tanh",
                     rope_parameters={"rope_theta": 1e4, "rope_type": "default"},
                     max_position_embeddings=64)
    hc._attn_implementation = "eager"
    layer = GemmaDecoderLayer(hc, layer_idx=0).double().eval()
    res = _hf_load(layer, W, {**_attn_names(), **_MLP_NAMES, **_NORM_NAMES})
    assert not res.missing_keys and not res.unexpected_keys
    x = np.random.default_rng(24).standard_normal((1, 13, 64)).astype(np.float32)
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(13)[None]
    cos, sin = GemmaRotaryEmbedding(hc)(xt, pos)
    with torch.no_grad():
        ref = layer(xt, attention_mask=_causal_mask(13), position_ids=pos,
                    position_embeddings=(cos, sin)).numpy()
    got = block_forward(cfg, W, x, dtype=np.float64)
    # Gemma's RMSNorm computes in float32
    assert rel_err(got - x, ref - x) < 5e-5


@pytest.mark.parametrize("window", [0, 5])
def test_attention_sublayer_matches_hf_gemma2_softcap(window):
    from transformers import Gemma2Config
    from transformers.models.gemma2.modeling_gemma2 import (Gemma2Attention, Gemma2RMSNorm,
                                                             Gemma2RotaryEmbedding)
    cfg, W = random_block(25, d_model=64, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=64,
                          norm="rmsnorm_offset", mlp="geglu_tanh", attn_softcap=1.5,
                          window=window)
    # scale q up so the softcap bites: scores of several units before capping
    W["q_proj.weight"] = W["q_proj.weight"] * np.float32(20.0)
    W["down_proj.weight"] = np.zeros_like(W["down_proj.weight"])   # y = x + attention sublayer
    hc = Gemma2Config(hidden_size=64, intermediate_size=64, num_attention_heads=4,
                      num_key_value_heads=2, head_dim=32, rms_norm_eps=1e-6,
                      query_pre_attn_scalar=32, attn_logit_softcapping=1.5,
                      sliding_window=window or None,
                      rope_parameters={"rope_theta": 1e4, "rope_type": "default"},
                      max_position_embeddings=64)
    hc._attn_implementation = "eager"
    attn = Gemma2Attention(hc, layer_idx=0).double().eval()
    res = _hf_load(attn, W, _attn_names(prefix=""))
    assert not res.missing_keys and not res.unexpected_keys
    norm = Gemma2RMSNorm(64, eps=1e-6).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(W["input_layernorm.weight"].astype(np.float64)))
    L = 14
    x = np.random.default_rng(26).standard_normal((1, L, 64)).astype(np.float32)
    xt = torch.from_numpy(x.astype(np.float64))
    pos = torch.arange(L)[None]
    cos, sin = Gemma2RotaryEmbedding(hc)(xt, pos)
    with torch.no_grad():
        ref, _ = attn(norm(xt), position_embeddings=(cos, sin),
                      attention_mask=_causal_mask(L, window))
    got = block_forward(cfg, W, x, dtype=np.float64) - x
    assert rel_err(got, ref.numpy()) < 5e-5
    # without the cap the result is clearly different (the cap is exercised)
    cfg_nocap = dict(cfg, attn_softcap=0.0)
    assert rel_err(block_forward(cfg_nocap, W, x, dtype=np.float64) - x, ref.numpy()) > 1e-2


# ------------------------------------------------------------ invariants ----
@pytest.mark.parametrize("window", [0, 5])
def test_decode_equals_prefill_bitwise_rowwise(window):
    cfg, W = random_block(31, window=window, attn_softcap=3.0 if window else 0.0)
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, 14, 64)).astype(np.float32)
    st_full = OracleState(cfg, 2, 16)
    y_full = block_forward(cfg, W, x, st_full, layout="rowwise")
    st = OracleState(cfg, 2, 16)
    ys = [block_forward(cfg, W, x[:, :6], st, layout="rowwise")]
    for t in range(6, 14):
        ys.append(block_step(cfg, W, x[:, t], st, layout="rowwise"))
    y_inc = np.concatenate(ys, axis=1)
    np.testing.assert_array_equal(y_inc, y_full)
    np.testing.assert_array_equal(st.k, st_full.k)
    np.testing.assert_array_equal(st.lengths, [14, 14])
    # batched layout agrees to rounding
    y_b = block_forward(cfg, W, x)
    assert rel_err(y_b, y_full) < 1e-6


@pytest.mark.parametrize("window", [0, 4])
def test_chunked_continuation_equals_whole(window):
    cfg, W = random_block(33, window=window)
    x = np.random.default_rng(34).standard_normal((1, 12, 64))
    y = block_forward(cfg, W, x, OracleState(cfg, 1, 12), dtype=np.float64)
    st = OracleState(cfg, 1, 12, dtype=np.float64)
    y1 = block_forward(cfg, W, x[:, :7], st, dtype=np.float64)
    y2 = block_forward(cfg, W, x[:, 7:], st, dtype=np.float64)
    np.testing.assert_allclose(np.concatenate([y1, y2], 1), y, rtol=1e-12, atol=1e-12)


def test_ring_holds_last_window_positions():
    cfg, W = random_block(35, window=4)
    x = np.random.default_rng(36).standard_normal((1, 10, 64))
    st = OracleState(cfg, 1, 32, dtype=np.float64)
    block_forward(cfg, W, x, st, dtype=np.float64)
    st_ref = OracleState(cfg, 1, 32, dtype=np.float64)
    for t in range(10):                                   # one token at a time
        block_step(cfg, W, x[:, t], st_ref, dtype=np.float64)
    np.testing.assert_allclose(st.k, st_ref.k, rtol=1e-12, atol=1e-13)
    assert st.capacity == 4 and st.lengths[0] == 10


def test_batch_rows_independent_and_per_row_lengths():
    cfg, W = random_block(37)
    rng = np.random.default_rng(38)
    xa = rng.standard_normal((1, 5, 64))
    xb = rng.standard_normal((1, 9, 64))
    steps = rng.standard_normal((2, 64))
    # rows with different cached lengths, one decode step together
    st = OracleState(cfg, 2, 16, dtype=np.float64)
    sa, sb = OracleState(cfg, 1, 16, dtype=np.float64), OracleState(cfg, 1, 16, dtype=np.float64)
    block_forward(cfg, W, xa, sa, dtype=np.float64)
    block_forward(cfg, W, xb, sb, dtype=np.float64)
    st.k[0], st.v[0], st.lengths[0] = sa.k[0], sa.v[0], 5
    st.k[1], st.v[1], st.lengths[1] = sb.k[0], sb.v[0], 9
    y = block_step(cfg, W, steps, st, dtype=np.float64)
    ya = block_step(cfg, W, steps[:1], sa, dtype=np.float64)
    yb = block_step(cfg, W, steps[1:], sb, dtype=np.float64)
    np.testing.assert_allclose(y[0], ya[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(y[1], yb[0], rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(st.lengths, [6, 10])


def test_block_causal_invariance_rowwise():
    cfg, W = random_block(39)
    x = np.random.default_rng(40).standard_normal((1, 10, 64)).astype(np.float32)
    y = block_forward(cfg, W, x, layout="rowwise")
    x2 = x.copy()
    x2[:, 6:] = 5.0
    y2 = block_forward(cfg, W, x2, layout="rowwise")
    np.testing.assert_array_equal(y[:, :6], y2[:, :6])


def test_float32_oracle_error_bound():
    wl = make_workload("tiny_llama_f32")
    y32 = block_forward(wl["cfg"], wl["weights"], wl["x"])
    y64 = block_forward(wl["cfg"], wl["weights"], wl["x"], dtype=np.float64)
    assert y32.dtype == np.float32
    assert rel_err(y32, y64) < 1e-6
    assert rel_err(y32 - wl["x"], y64 - wl["x"]) < 1e-5


def test_oracle_refuses_out_of_range_positions():
    cfg, W = random_block(41, max_positions=8)
    x = np.zeros((1, 9, 64), dtype=np.float32)
    with pytest.raises(ValueError):
        block_forward(cfg, W, x)
    st = OracleState(cfg, 1, 6)
    with pytest.raises(ValueError):
        block_forward(cfg, W, x[:, :7], st)
    with pytest.raises(ValueError):
        block_forward(cfg, W, np.zeros((2, 1, 64)), st)


def test_ring_slot_layout():
    # Keys do not depend on the window; the ring keeps position p at slot p mod W
    # (mojolearn TransformerState, sliding-window layout), the full cache at slot p.
    cfg, W = random_block(42, window=4)
    x = np.random.default_rng(43).standard_normal((1, 10, 64))
    ring = OracleState(cfg, 1, 32, dtype=np.float64)
    block_forward(cfg, W, x, ring, dtype=np.float64)
    cfg_full = dict(cfg, window=0)
    full = OracleState(cfg_full, 1, 32, dtype=np.float64)
    block_forward(cfg_full, W, x, full, dtype=np.float64)
    for p in range(6, 10):
        np.testing.assert_array_equal(ring.k[:, :, p % 4], full.k[:, :, p])
        np.testing.assert_array_equal(ring.v[:, :, p % 4], full.v[:, :, p])
    assert np.all(full.k[:, :, 10:] == 0)


@pytest.mark.parametrize("over", [dict(), dict(window=5, attn_softcap=2.0, norm="rmsnorm_offset",
                                               mlp="geglu_tanh"), dict(qkv_bias=True, qk_norm=True)])
def test_rows_form_matches_full_form(over):
    from oracle import block_forward_rows
    cfg, W = random_block(50, **over)
    rng = np.random.default_rng(51)
    x = rng.standard_normal((2, 13, 64))
    rows = [(0, 0), (1, 12), (0, 7), (1, 3)]
    full = block_forward(cfg, W, x, dtype=np.float64)
    got = block_forward_rows(cfg, W, x, rows, dtype=np.float64)
    np.testing.assert_allclose(got, np.stack([full[b, t] for b, t in rows]), rtol=1e-12, atol=1e-12)
    # continuation from a carried state (ring included)
    st = OracleState(cfg, 2, 40, dtype=np.float64)
    block_forward(cfg, W, rng.standard_normal((2, 9, 64)), st, dtype=np.float64)
    x2 = rng.standard_normal((2, 6, 64))
    ref = block_forward(cfg, W, x2, st.copy(), dtype=np.float64)
    got = block_forward_rows(cfg, W, x2, [(0, 5), (1, 0)], st, dtype=np.float64)
    np.testing.assert_allclose(got, np.stack([ref[0, 5], ref[1, 0]]), rtol=1e-12, atol=1e-12)


def test_page_worked_example_golden():
    """The oracle on the mojolearn page's usage example (TransformerBlock,
    Examples) reproduces the stored output in tests/golden (written by the
    committed script from the float64 oracle; the page prints the example's
    inputs, not its output).  Also checks the example's documented shape
    contract: the output has the input's shape (B, L, d_model)."""
    from tests.golden.make_mojolearn_example import oracle_output, read
    y = np.asarray(oracle_output(), dtype=np.float64)
    assert y.shape == (2, 16, 64)
    ref = read()
    assert abs(y.sum() - ref["sum"]) <= 1e-9 * max(1.0, abs(ref["sum"]))
    assert abs(np.square(y).sum() - ref["sumsq"]) <= 1e-9 * ref["sumsq"]
    for (b, t), row in ref["rows"].items():
        np.testing.assert_allclose(y[b, t], row, rtol=0, atol=1e-12)


def test_ragged_lengths_reading_and_pins():
    """mojolearn forward(x, lengths=...): the page's ragged batch.  Pins that do
    not restate the definition: (a) lengths all equal to L is the plain
    batched forward; (b) by causality, a row's real positions equal the first
    lengths[i] positions of the same row run unragged at full L; (c) padding
    outputs are exactly +0.0 (positive zero) and the padding inputs change
    nothing; (d) a state is refused, as are lengths outside [1, L]."""
    cfg, W = random_block(31, window=0)
    rng = np.random.default_rng(5)
    B, L = 3, 9
    x = rng.standard_normal((B, L, cfg["d_model"]), dtype=np.float32)
    full = block_forward(cfg, W, x, dtype=np.float64)
    np.testing.assert_allclose(block_forward(cfg, W, x, dtype=np.float64, lengths=[L] * B), full, rtol=0,
                               atol=1e-12)
    lens = [4, 9, 1]
    y = block_forward(cfg, W, x, dtype=np.float64, lengths=lens)
    for i, n in enumerate(lens):
        np.testing.assert_allclose(y[i, :n], full[i, :n], rtol=0, atol=1e-12)
        pad = y[i, n:]
        assert np.all(pad == 0.0) and not np.any(np.signbit(pad))
    x2 = x.copy()
    for i, n in enumerate(lens):
        x2[i, n:] = rng.standard_normal((L - n, cfg["d_model"]), dtype=np.float32) * 5
    np.testing.assert_array_equal(block_forward(cfg, W, x2, dtype=np.float64, lengths=lens), y)
    with pytest.raises(ValueError):
        block_forward(cfg, W, x, OracleState(cfg, B, 16), lengths=lens)
    with pytest.raises(ValueError):
        block_forward(cfg, W, x, lengths=[0, 9, 1])
    with pytest.raises(ValueError):
        block_forward(cfg, W, x, lengths=[10, 9, 1])


def test_ragged_window_softcap_pin():
    """The ragged reading under a window, softcap and GQA: still the causal
    prefix of the unragged run (windowed keys are never later positions)."""
    cfg, W = random_block(32, window=3, attn_softcap=5.0, n_heads=4, n_kv_heads=1, mlp="geglu_tanh")
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 7, cfg["d_model"]), dtype=np.float32)
    full = block_forward(cfg, W, x, dtype=np.float64)
    y = block_forward(cfg, W, x, dtype=np.float64, lengths=[5, 2])
    np.testing.assert_allclose(y[0, :5], full[0, :5], rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[1, :2], full[1, :2], rtol=0, atol=1e-12)
    assert np.all(y[0, 5:] == 0) and np.all(y[1, 2:] == 0)
