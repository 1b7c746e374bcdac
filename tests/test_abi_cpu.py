"""The C-ABI library loads and exports every function include/gqa_block.h
declares, and create-time validation (which runs on the host before any HIP
call) returns the documented error codes.  No GPU needed."""
import ctypes
import os
import re

import pytest

from gqa_causal_attention_amd import binding
from gqa_causal_attention_amd.binding import Config, Tensor, make_config
from gqa_causal_attention_amd.workloads import random_block, weight_shapes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.load_library()


def test_header_symbols_exported():
    lib = _lib()
    hdr = open(os.path.join(ROOT, "include", "gqa_block.h")).read()
    names = set(re.findall(r"\b(gqa_[a-z_]+)\s*\(", hdr))
    assert names == set(binding.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.gqa_version()


def _records(cfg, W, drop=None, rename=None, reshape=None, redtype=None, extra=None):
    recs = []
    fake = 0x1000
    for name, a in W.items():
        if name == drop:
            continue
        nm = rename[1] if rename and rename[0] == name else name
        shape = list(a.shape)
        if reshape and reshape[0] == name:
            shape = list(reshape[1])
        matrix = a.ndim == 2
        dt = 1 if (matrix and cfg["dtype"] == "bf16") else 0
        if redtype == name:
            dt = 1 - dt
        recs.append(Tensor(nm.encode(), ctypes.c_void_p(fake), dt, len(shape),
                           (ctypes.c_int64 * 2)(*(shape + [0, 0])[:2])))
    if extra:
        recs.append(Tensor(extra.encode(), ctypes.c_void_p(fake), 0, 1, (ctypes.c_int64 * 2)(64, 0)))
    return (Tensor * len(recs))(*recs), len(recs)


def _create(cfg, arr, n):
    lib = _lib()
    h = ctypes.c_void_p()
    c = make_config(cfg)
    rc = lib.gqa_block_create(ctypes.byref(c), arr, n, ctypes.byref(h))
    return rc, lib.gqa_last_error().decode()


@pytest.mark.parametrize("case,code", [
    ("missing", -2), ("extra", -2), ("badshape", -2), ("dtype", -3), ("bias_without_option", -2),
])
def test_weight_table_errors(case, code):
    cfg, W = random_block(1)
    kw = {}
    if case == "missing":
        kw["drop"] = "up_proj.weight"
    elif case == "extra":
        kw["extra"] = "o_proj.bias"
    elif case == "badshape":
        kw["reshape"] = ("k_proj.weight", (64, 64))
    elif case == "dtype":
        kw["redtype"] = "down_proj.weight"
    elif case == "bias_without_option":
        kw["extra"] = "q_proj.bias"
    arr, n = _records(cfg, W, **kw)
    rc, msg = _create(cfg, arr, n)
    assert rc == code, msg
    assert msg


@pytest.mark.parametrize("field,value,code", [
    ("n_kv_heads", 3, -2), ("head_dim", 15, -2), ("head_dim", 512, -11), ("window", -1, -1),
    ("max_positions", 0, -1), ("rope_theta", 0.0, -1), ("attn_softcap", -1.0, -1),
    ("rope_dim", 3, -1), ("rope_dim", 18, -1), ("rope_dim", -2, -1),
    ("rope_scaling", {"type": "linear", "factor": 0.0}, -1),
    ("rope_scaling", {"type": "llama3", "factor": 8.0, "low_freq_factor": 4.0, "high_freq_factor": 1.0,
                      "original_max_position_embeddings": 8192}, -1),
    ("rope_scaling", {"type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                      "original_max_position_embeddings": 0}, -1),
    ("norm_bias", True, -1),
])
def test_config_errors(field, value, code):
    cfg, W = random_block(2)
    cfg[field] = value
    arr, n = _records(cfg, W)
    rc, msg = _create(cfg, arr, n)
    assert rc == code, msg


def test_rope_scaling_kind_is_checked():
    cfg, W = random_block(2, rope_scaling={"type": "yarn", "factor": 2.0})
    with pytest.raises(ValueError):
        make_config(cfg)
    c = make_config(dict(cfg, rope_scaling=None))
    c.rope_scaling = 7
    lib = _lib()
    arr, n = _records(cfg, W)
    h = ctypes.c_void_p()
    assert lib.gqa_block_create(ctypes.byref(c), arr, n, ctypes.byref(h)) == -1
    assert "rope_scaling" in lib.gqa_last_error().decode()


@pytest.mark.parametrize("case,code", [("gate_for_ungated", -2), ("missing_sandwich", -2),
                                       ("missing_norm_bias", -2), ("norm_bias_unasked", -2)])
def test_option_weight_tables(case, code):
    if case == "gate_for_ungated":
        cfg, W = random_block(5, mlp="gelu")
        arr, n = _records(cfg, W, extra="gate_proj.weight")
    elif case == "missing_sandwich":
        cfg, W = random_block(5, sandwich_norms=True)
        arr, n = _records(cfg, W, drop="post_feedforward_layernorm.weight")
    elif case == "missing_norm_bias":
        cfg, W = random_block(5, norm="layernorm", norm_bias=True)
        arr, n = _records(cfg, W, drop="input_layernorm.bias")
    else:
        cfg, W = random_block(5, norm="layernorm")
        arr, n = _records(cfg, W, extra="post_attention_layernorm.bias")
    rc, msg = _create(cfg, arr, n)
    assert rc == code, msg


@pytest.mark.parametrize("field,value", [("o_bias", 2), ("sandwich_norms", -1), ("mlp", 5), ("norm", 3)])
def test_option_fields_checked_by_the_library(field, value):
    cfg, W = random_block(2)
    c = make_config(cfg)
    setattr(c, field, value)
    lib = _lib()
    arr, n = _records(cfg, W)
    h = ctypes.c_void_p()
    assert lib.gqa_block_create(ctypes.byref(c), arr, n, ctypes.byref(h)) == -1
    assert lib.gqa_last_error().decode()


def test_unknown_option_names():
    for key, val in (("norm", "batchnorm"), ("mlp", "relu")):
        cfg, _ = random_block(6, **{key: val})
        with pytest.raises(ValueError):
            make_config(cfg)


def test_bf16_shape_rule():
    cfg, W = random_block(3, dtype="bf16", d_model=96, intermediate=128)
    arr, n = _records(cfg, W)
    rc, msg = _create(cfg, arr, n)
    assert rc == -11 and "multiples of 64" in msg


def test_valid_table_passes_validation():
    # A valid table passes every host check; without a GPU the first device
    # call then fails with GQA_ERR_HIP, with a GPU it succeeds (fake pointers
    # would fault, so only run this where no device is visible).
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake device pointers must not reach a GPU")
    for over in ({}, dict(rope_dim=6, rope_scaling={"type": "linear", "factor": 4.0}),
                 dict(rope_dim=16, rope_scaling={"type": "llama3", "factor": 8.0, "low_freq_factor": 1.0,
                                                 "high_freq_factor": 4.0,
                                                 "original_max_position_embeddings": 8192}),
                 dict(norm="layernorm", norm_bias=True, sandwich_norms=True, o_bias=True, mlp_bias=True,
                      mlp="geglu"),
                 dict(mlp="gelu_tanh", mlp_bias=True, sandwich_norms=True, norm="rmsnorm_offset"),
                 dict(mlp="gelu")):
        cfg, W = random_block(4, qkv_bias=True, qk_norm=True, **over)
        arr, n = _records(cfg, W)
        rc, msg = _create(cfg, arr, n)
        assert rc == -10, msg


def test_null_arguments():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.gqa_block_create(None, None, 0, ctypes.byref(h)) == -1
    n = ctypes.c_size_t()
    assert lib.gqa_workspace_bytes(None, 1, 1, ctypes.byref(n)) == -1
    assert lib.gqa_block_forward(None, None, None, None, 1, 1, None, 0, None) == -1
    assert lib.gqa_block_step(None, None, None, None, 1, None, 0, None) == -7
    n = ctypes.c_size_t()
    assert lib.gqa_block_describe_plan(None, 0, 1, 1, None, 0, ctypes.byref(n)) == -1
    assert "NULL" in lib.gqa_last_error().decode()
