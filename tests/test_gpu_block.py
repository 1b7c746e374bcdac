"""Parity of the HIP block against the CPU oracle on small shapes that still
span several GEMM / attention tiles with ragged tails, every block option,
carried state, chunked continuation and decode steps.

Bar: max|gpu - oracle| / max|oracle| on y and on y - x, 1e-4 for float32
blocks and 2e-2 for bf16-weight blocks (bf16 GEMM operands, activations and
KV cache; float32 accumulation, softmax and residual stream)."""
import numpy as np
import pytest

from gqa_causal_attention_amd.workloads import make_workload, random_block, round_bf16
from tests.helpers import (OracleState, block_forward, block_step, check_close, fill_state_gpu, rel_err,
                           oracle_dtype, to_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _block(cfg, W):
    from gqa_causal_attention_amd import Block
    return Block(cfg, W)


def test_tiny_llama_prefill_then_decode(torch_cuda):
    """The tiny fp32 workload: prefill 16 tokens, then 8 single-token steps."""
    wl = make_workload("tiny_llama_f32")
    cfg, W, x, xs = wl["cfg"], wl["weights"], wl["x"], wl["x_steps"]
    blk = _block(cfg, W)
    st = blk.allocate_state(1, wl["capacity"])
    ost = OracleState(cfg, 1, wl["capacity"], dtype=np.float64)
    y = blk.forward(to_gpu(x), st).cpu().numpy()
    yr = block_forward(cfg, W, x, ost, dtype=np.float64)
    check_close(y, yr, x, "f32", "prefill")
    for i in range(xs.shape[0]):
        y = blk.step(to_gpu(xs[i]), st).cpu().numpy()
        yr = block_step(cfg, W, xs[i], ost, dtype=np.float64)
        check_close(y, yr, xs[i], "f32", f"step {i}")
    np.testing.assert_array_equal(st.lengths.cpu().numpy(), [24])
    np.testing.assert_array_equal(st.host_lengths(), [24])
    # the cache holds post-RoPE keys and raw values at slot = position
    np.testing.assert_allclose(st.k.cpu().numpy(), ost.k, rtol=1e-4, atol=1e-5)
    np.testing.assert_allclose(st.v.cpu().numpy(), ost.v, rtol=1e-4, atol=1e-5)
    # self-contained prefill (no state)
    y0 = blk.forward(to_gpu(x)).cpu().numpy()
    check_close(y0, block_forward(cfg, W, x, dtype=np.float64), x, "f32", "stateless")


LLAMA31_ROPE = {"type": "llama3", "factor": 8.0, "low_freq_factor": 1.0, "high_freq_factor": 4.0,
                "original_max_position_embeddings": 8192}

BF16_CASES = {
    # name: (block overrides, B, prefill L, continuation L, decode steps)
    "llama_g4_hd128": (dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=512,
                            rope_theta=5e5), 2, 150, 37, 3),
    "hd64_g4": (dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, intermediate=320), 1, 200, 0, 2),
    "gemma_window_softcap_hd256": (dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=256,
                                        intermediate=384, window=64, attn_softcap=50.0,
                                        mlp="geglu_tanh", norm="rmsnorm_offset"), 2, 150, 20, 3),
    "qwen_bias_qknorm_g5": (dict(d_model=640, n_heads=10, n_kv_heads=2, head_dim=128,
                                 intermediate=640, qkv_bias=True, qk_norm=True), 1, 130, 5, 2),
    "mha_g1": (dict(d_model=256, n_heads=2, n_kv_heads=2, head_dim=128, intermediate=256), 1, 70, 0, 2),
    # qk_norm with the (1 + w) norm weights, whole-head RoPE (the prefill
    # attention kernel normalises and rotates q itself)
    "qknorm_offset_hd64": (dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=64, intermediate=384,
                                qk_norm=True, norm="rmsnorm_offset", mlp="geglu_tanh"), 2, 150, 20, 2),
    "big_m_tiles": (dict(d_model=512, n_heads=4, n_kv_heads=1, head_dim=128, intermediate=768,
                         rope_theta=5e5), 1, 1100, 0, 1),
    # RoPE options: the Llama 3.1 ramp; partial rotary with linear scaling and
    # qk_norm (vector RoPE form: rotated and pass-through lanes); a rope_dim
    # that is not a multiple of 8 (wave-per-head form)
    "llama31_rope_scaling": (dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=512,
                                  rope_theta=5e5, rope_scaling=LLAMA31_ROPE), 2, 150, 37, 3),
    "partial_rotary_linear_qknorm": (dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                                          intermediate=256, rope_dim=32, qk_norm=True, qkv_bias=True,
                                          rope_scaling={"type": "linear", "factor": 4.0}), 2, 90, 10, 3),
    "partial_rotary_rd20_hd64": (dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=256,
                                      rope_dim=20, qk_norm=True), 1, 70, 6, 2),
    # norm / MLP / bias options: Gemma 2 sandwich norms (128x128 tiles, then
    # decode); LayerNorm with every bias and an ungated exact-GELU MLP on the
    # pipelined large-M tiles; exact GeGLU with MLP biases under LayerNorm
    # sandwich norms; ungated tanh-GELU; a 10240-wide row (register norm form)
    "gemma2_sandwich": (dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=128, intermediate=384, window=64,
                             attn_softcap=50.0, mlp="geglu_tanh", norm="rmsnorm_offset", sandwich_norms=True),
                        2, 150, 20, 3),
    "layernorm_biases_gelu": (dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=512,
                                   norm="layernorm", norm_bias=True, qkv_bias=True, o_bias=True, mlp_bias=True,
                                   mlp="gelu"), 1, 600, 10, 3),
    "geglu_sandwich_layernorm": (dict(d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, intermediate=768,
                                      mlp="geglu", mlp_bias=True, o_bias=True, sandwich_norms=True,
                                      norm="layernorm", norm_bias=True), 1, 700, 0, 2),
    "gelu_tanh_ungated": (dict(d_model=256, n_heads=4, n_kv_heads=1, head_dim=128, intermediate=256,
                               mlp="gelu_tanh"), 2, 90, 0, 2),
    "wide_row_10240": (dict(d_model=10240, n_heads=2, n_kv_heads=1, head_dim=128, intermediate=256,
                            norm="layernorm"), 1, 40, 0, 1),
}


@pytest.mark.parametrize("name", list(BF16_CASES))
def test_bf16_block_variants(torch_cuda, name):
    over, B, L0, L1, steps = BF16_CASES[name]
    cfg, W = random_block(100 + list(BF16_CASES).index(name), dtype="bf16", **over)
    rng = np.random.default_rng(7)
    cap = L0 + L1 + steps
    blk = _block(cfg, W)
    st = blk.allocate_state(B, cap)
    ost = OracleState(cfg, B, cap, dtype=np.float32)
    x0 = rng.standard_normal((B, L0, cfg["d_model"]), dtype=np.float32)
    check_close(blk.forward(to_gpu(x0), st).cpu().numpy(), block_forward(cfg, W, x0, ost), x0, "bf16",
                f"{name} prefill")
    if L1:
        x1 = rng.standard_normal((B, L1, cfg["d_model"]), dtype=np.float32)
        check_close(blk.forward(to_gpu(x1), st).cpu().numpy(), block_forward(cfg, W, x1, ost), x1, "bf16",
                    f"{name} continuation")
    for i in range(steps):
        xt = rng.standard_normal((B, cfg["d_model"]), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, "bf16",
                    f"{name} step {i}")
    np.testing.assert_array_equal(st.lengths.cpu().numpy(), ost.lengths)


def test_bf16_decode_ragged_rows_prefilled_cache(torch_cuda):
    """Rows at different positions (one still empty), a cache pre-filled with
    N(0, 1) keys/values, several chunks of the split-K decode per row."""
    cfg, W = random_block(200, dtype="bf16", d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=256, max_positions=8192)
    # 0 and 1 cached keys, a split boundary crossed during the steps (2047),
    # three splits (4097) and one split with a ragged end (700)
    B, cap = 5, 4400
    lengths = np.array([0, 1, 2047, 4097, 700], dtype=np.int32)
    rng = np.random.default_rng(8)
    kf = round_bf16(rng.standard_normal((B, 2, cap, 128), dtype=np.float32))
    vf = round_bf16(rng.standard_normal((B, 2, cap, 128), dtype=np.float32))
    used = np.arange(cap)[None, None, :, None] < lengths[:, None, None, None]
    kf, vf = np.where(used, kf, 0).astype(np.float32), np.where(used, vf, 0).astype(np.float32)
    blk = _block(cfg, W)
    st = blk.allocate_state(B, cap)
    fill_state_gpu(st, kf, vf, lengths)
    ost = OracleState.from_fill(cfg, kf, vf, lengths)
    for i in range(3):
        xt = rng.standard_normal((B, 1, 256), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, "bf16", f"step {i}")
    np.testing.assert_array_equal(st.lengths.cpu().numpy(), lengths + 3)


DECODE_GEMM_BLOCKS = {
    # q/k/v, o_proj and gate/up K-split in two (1024 deep); down unsplit, 1280
    # deep (10 chunks), fused residual
    "split": dict(d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128, intermediate=1280, qkv_bias=True),
    # no split: the fused bias / residual / gated epilogues (4- and 6-chunk depths)
    "fused": dict(d_model=512, n_heads=8, n_kv_heads=2, head_dim=64, intermediate=768, qkv_bias=True,
                  mlp="geglu_tanh"),
    # split q/k/v GEMM with partial rotary: the RoPE kernel sums the partials
    # of rotated and pass-through columns alike
    "split_partial_rotary": dict(d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128, intermediate=1280,
                                 qkv_bias=True, rope_dim=64, rope_theta=5e5, rope_scaling=LLAMA31_ROPE),
    # sandwich norms with biases: the norm kernels sum the o_proj and down
    # K-split partials (+ bias) before the output norm and the residual add
    "split_sandwich_biases": dict(d_model=2048, n_heads=16, n_kv_heads=4, head_dim=128, intermediate=2560,
                                  sandwich_norms=True, o_bias=True, mlp_bias=True, mlp="geglu",
                                  norm="rmsnorm_offset"),
    # ungated MLP: the up GEMM stores act(up + bias)
    "ungated_biases": dict(d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=1280,
                           mlp="gelu_tanh", mlp_bias=True, o_bias=True, norm="layernorm", norm_bias=True),
    # o_proj and down K-split around an unsplit gate/up: the norm kernel sums
    # o_proj's partials (+ bias), down's reduce kernel adds bias and residual
    # (offset RMSNorm weights)
    "split_o_down_offset_biases": dict(d_model=1024, n_heads=16, n_kv_heads=4, head_dim=128,
                                       intermediate=2048, o_bias=True, mlp_bias=True, mlp="geglu",
                                       norm="rmsnorm_offset"),
}


@pytest.mark.parametrize("B", [1, 7, 20, 33, 64])
@pytest.mark.parametrize("kind", list(DECODE_GEMM_BLOCKS))
def test_bf16_decode_gemm_batch_sizes(torch_cuda, kind, B):
    """Decode steps at every activation-row tiling of the decode GEMMs (1, 2
    and 4 groups of 16 rows, ragged last group), split and unsplit K."""
    cfg, W = random_block(210 + list(DECODE_GEMM_BLOCKS).index(kind), dtype="bf16", **DECODE_GEMM_BLOCKS[kind])
    rng = np.random.default_rng(12 + B)
    blk = _block(cfg, W)
    plan = blk.describe_plan(B, 1)
    splits = {ln.split()[0]: int(ln.split("splits=")[1].split()[0]) for ln in plan.splitlines() if "splits=" in ln}
    if kind.startswith("split") and kind != "split_o_down_offset_biases":   # the K-split partial paths
        assert "gemm_qkv tile=6" in plan and "gemm_o tile=6" in plan, plan
        assert splits["gemm_qkv"] >= 2 and splits["gemm_o"] >= 2, plan
    if kind == "split_sandwich_biases":
        assert "gemm_down tile=6" in plan and splits["gemm_down"] >= 2, plan
    if kind == "split_o_down_offset_biases":
        assert "gemm_o tile=6" in plan and "gemm_down tile=6" in plan, plan
        assert splits["gemm_o"] >= 2 and splits["gemm_down"] >= 2 and splits["gemm_gate_up"] == 1, plan
    st = blk.allocate_state(B, 8)
    ost = OracleState(cfg, B, 8)
    x = rng.standard_normal((B, 5, cfg["d_model"]), dtype=np.float32)
    check_close(blk.forward(to_gpu(x), st).cpu().numpy(), block_forward(cfg, W, x, ost), x, "bf16", "prefill")
    for i in range(2):
        xt = rng.standard_normal((B, cfg["d_model"]), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, "bf16",
                    f"{kind} B={B} step {i}")


@pytest.mark.parametrize("B", [100, 520, 2048, 2100])
def test_bf16_decode_many_rows(torch_cuda, B):
    """Decode batches past the weight-streaming GEMM's 64 rows: 64x128 tiles
    (M = 100), the pipelined large-M tiles (M = 520), the split-K decode
    attention at its largest row table (2048), and more rows than that table
    holds (2100: the matrix-core prefill attention at L = 1 over the cache);
    each after a short prefill, against the oracle."""
    cfg, W = random_block(215, dtype="bf16", d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=512)
    rng = np.random.default_rng(16 + B)
    blk = _block(cfg, W)
    plan = blk.describe_plan(B, 1)
    want = {100: "gemm_o tile=2", 520: "gemm_o tile=7", 2048: "gemm_o tile=7", 2100: "attention=prefill_mfma"}[B]
    assert want in plan, plan
    if B <= 2048:   # (2048: the split-K decode attention's largest row table)
        assert "attention=decode_splitk" in plan, plan
    st = blk.allocate_state(B, 8)
    ost = OracleState(cfg, B, 8)
    x = rng.standard_normal((B, 3, cfg["d_model"]), dtype=np.float32)
    check_close(blk.forward(to_gpu(x), st).cpu().numpy(), block_forward(cfg, W, x, ost), x, "bf16",
                f"B={B} prefill")
    for i in range(2):
        xt = rng.standard_normal((B, cfg["d_model"]), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, "bf16",
                    f"B={B} step {i}")


@pytest.mark.parametrize("dtype,window", [("bf16", 1), ("bf16", 2), ("f32", 1), ("bf16", 31)])
def test_degenerate_windows(torch_cuda, dtype, window):
    """The smallest windows: W = 1 (every position attends itself only, so the
    attention output is its own value row) and W = 2, plus a window one
    short of the prefill, through prefill, continuation and decode steps over
    the ring, against the oracle."""
    cfg, W = random_block(216 + window, dtype=dtype, d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=256, window=window)
    rng = np.random.default_rng(30 + window)
    blk = _block(cfg, W)
    st = blk.allocate_state(2, 64)
    ost = OracleState(cfg, 2, 64)
    for L in (32, 5):
        x = rng.standard_normal((2, L, 256), dtype=np.float32)
        check_close(blk.forward(to_gpu(x), st).cpu().numpy(), block_forward(cfg, W, x, ost), x, dtype,
                    f"W={window} L={L}")
    for i in range(3):
        xt = rng.standard_normal((2, 256), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, dtype,
                    f"W={window} step {i}")


def test_last_position(torch_cuda):
    """Positions up to max_positions - 1 (the RoPE table's last row) match the
    oracle; one more step is refused before any launch and leaves the state
    unchanged."""
    from gqa_causal_attention_amd.binding import GqaError
    cfg, W = random_block(220, dtype="bf16", d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=256, max_positions=40)
    rng = np.random.default_rng(40)
    blk = _block(cfg, W)
    st = blk.allocate_state(1, 64)
    ost = OracleState(cfg, 1, 64)
    x = rng.standard_normal((1, 36, 256), dtype=np.float32)
    check_close(blk.forward(to_gpu(x), st).cpu().numpy(), block_forward(cfg, W, x, ost), x, "bf16", "prefill")
    for i in range(4):   # positions 36 .. 39
        xt = rng.standard_normal((1, 256), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost), xt, "bf16",
                    f"position {36 + i}")
    with pytest.raises(GqaError) as e:
        blk.step(to_gpu(rng.standard_normal((1, 256), dtype=np.float32)), st)
    assert e.value.name == "POSITION"
    assert st.host_lengths().tolist() == [40]


def test_bf16_window_ring_wraps(torch_cuda):
    """Prefill longer than the window (in-call keys from the fresh K/V), then
    decode steps through the ring's wrap-around."""
    cfg, W = random_block(201, dtype="bf16", d_model=256, n_heads=4, n_kv_heads=2, head_dim=128,
                          intermediate=256, window=48)
    rng = np.random.default_rng(9)
    blk = _block(cfg, W)
    st = blk.allocate_state(2, 400)
    ost = OracleState(cfg, 2, 400)
    x = rng.standard_normal((2, 130, 256), dtype=np.float32)
    check_close(blk.forward(to_gpu(x), st).cpu().numpy(), block_forward(cfg, W, x, ost), x, "bf16", "prefill")
    for i in range(60):
        xt = rng.standard_normal((2, 1, 256), dtype=np.float32)
        y = blk.step(to_gpu(xt), st).cpu().numpy()
        if i % 7 == 0 or i == 59:
            check_close(y, block_step(cfg, W, xt, ost), xt, "bf16", f"step {i}")
        else:
            block_step(cfg, W, xt, ost)
    got_k = st.k.float().cpu().numpy()
    np.testing.assert_allclose(got_k, ost.k, rtol=2e-2, atol=2e-2 * np.abs(ost.k).max())


F32_CASES = {
    "window_softcap_geglu": (dict(window=7, attn_softcap=5.0, mlp="geglu_tanh", norm="rmsnorm_offset"),
                             2, 19, 6, 10),
    "bias_qknorm_g3": (dict(n_heads=6, n_kv_heads=2, head_dim=12, d_model=48, qkv_bias=True,
                            qk_norm=True), 3, 9, 4, 3),
    "odd_dims": (dict(d_model=50, n_heads=5, n_kv_heads=5, head_dim=10, intermediate=37), 1, 13, 0, 2),
    "partial_rotary_llama3_window_qknorm": (dict(rope_dim=6, window=5, qk_norm=True,
                                                 rope_scaling=dict(LLAMA31_ROPE,
                                                                   original_max_position_embeddings=32)),
                                            2, 19, 6, 5),
    "partial_rotary_odd_linear": (dict(d_model=50, n_heads=5, n_kv_heads=5, head_dim=10, intermediate=37,
                                       rope_dim=4, rope_scaling={"type": "linear", "factor": 2.5}), 1, 13, 3, 2),
    "layernorm_sandwich_all_biases": (dict(norm="layernorm", norm_bias=True, sandwich_norms=True, o_bias=True,
                                           mlp_bias=True, qkv_bias=True, mlp="geglu"), 2, 15, 5, 3),
    "odd_dims_layernorm_gelu_sandwich": (dict(d_model=50, n_heads=5, n_kv_heads=5, head_dim=10, intermediate=37,
                                              norm="layernorm", norm_bias=True, mlp="gelu",
                                              sandwich_norms=True), 1, 13, 0, 2),
    "odd_wide_row_9002": (dict(d_model=9002, n_heads=2, n_kv_heads=1, head_dim=8, intermediate=40,
                               mlp="gelu_tanh", mlp_bias=True), 1, 6, 0, 1),
}


@pytest.mark.parametrize("name", list(F32_CASES))
def test_f32_block_variants(torch_cuda, name):
    over, B, L0, L1, steps = F32_CASES[name]
    cfg, W = random_block(300 + list(F32_CASES).index(name), **over)
    rng = np.random.default_rng(10)
    cap = L0 + L1 + steps
    blk = _block(cfg, W)
    st = blk.allocate_state(B, cap)
    ost = OracleState(cfg, B, cap, dtype=np.float64)
    d = cfg["d_model"]
    x0 = rng.standard_normal((B, L0, d), dtype=np.float32)
    check_close(blk.forward(to_gpu(x0), st).cpu().numpy(), block_forward(cfg, W, x0, ost, dtype=np.float64),
                x0, "f32", f"{name} prefill")
    if L1:
        x1 = rng.standard_normal((B, L1, d), dtype=np.float32)
        check_close(blk.forward(to_gpu(x1), st).cpu().numpy(), block_forward(cfg, W, x1, ost, dtype=np.float64),
                    x1, "f32", f"{name} continuation")
    for i in range(steps):
        xt = rng.standard_normal((B, d), dtype=np.float32)
        check_close(blk.step(to_gpu(xt), st).cpu().numpy(), block_step(cfg, W, xt, ost, dtype=np.float64),
                    xt, "f32", f"{name} step {i}")
    np.testing.assert_allclose(st.k.cpu().numpy(), ost.k, rtol=1e-4, atol=1e-4 * np.abs(ost.k).max())


@pytest.mark.gpu
@pytest.mark.parametrize("window,softcap", [(0, 0.0), (200, 30.0)])
def test_ragged_prefill_packed_multiblock(torch_cuda, window, softcap):
    """The packed ragged path at a size that runs the large-M GEMM tiles (1278
    real tokens of 2800 padded) and several attention query blocks per row,
    rows of 700, 513, 64 and 1 tokens, with and without a window and softcap:
    against the oracle, padding +0.0, and that the packed path ran (its
    gather / scatter launches appear in the library's timing table)."""
    cfg, W = random_block(43 + window, dtype="bf16", d_model=512, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=1024, window=window, attn_softcap=softcap)
    B, L, lens = 4, 700, [700, 513, 64, 1]
    rng = np.random.default_rng(18)
    x = rng.standard_normal((B, L, cfg["d_model"]), dtype=np.float32)
    blk = _block(cfg, W)
    y = blk.forward(to_gpu(x), lengths=lens).cpu().numpy()
    ref = block_forward(cfg, W, x, dtype=np.float32, lengths=lens)
    for i, n in enumerate(lens):
        check_close(y[i, :n], ref[i, :n], x[i, :n], "bf16", f"packed ragged row {i} (length {n})")
        assert np.all(y[i, n:] == 0.0) and not np.any(np.signbit(y[i, n:]))
    # the packed path ran: its gather / scatter launches are in the timing table
    blk.set_timing(True)
    blk.forward(to_gpu(x), lengths=lens)
    names = set(blk.kernel_times())
    blk.set_timing(False)
    assert {"ragged_gather", "ragged_scatter"} <= names, names


def test_bf16_gemm_tail_split(torch_cuda, monkeypatch):
    """Large-M GEMMs whose last wave of tiles is at most half full run that
    tail as a separate K-split launch plus ordered reduce.  Counting waves in
    8 CUs (the tuning override) makes o_proj and down at M = 1100 take that
    path (rows from 1024, 2 splits), checked in the library's plan, against
    the oracle and against the same prefill without tail splits."""
    cfg, W = random_block(44, dtype="bf16", d_model=1024, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=2048)
    rng = np.random.default_rng(19)
    x = rng.standard_normal((1, 1100, 1024), dtype=np.float32)
    blk = _block(cfg, W)
    monkeypatch.setenv("GQA_GEMM_TAIL_CUS", "0")
    plain = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.setenv("GQA_GEMM_TAIL_CUS", "8")
    plan = blk.describe_plan(1, 1100)
    assert "gemm_o tile=7 splits=1 waves=0 tail_rows_from=1024 tail_splits=2" in plan, plan
    assert "gemm_down tile=7 splits=1 waves=0 tail_rows_from=1024 tail_splits=2" in plan, plan
    y = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.delenv("GQA_GEMM_TAIL_CUS")
    check_close(y, block_forward(cfg, W, x, dtype=np.float32), x, "bf16", "tail-split GEMMs")
    check_close(y, plain, x, "bf16", "tail-split vs whole-wave GEMMs")


def test_bf16_gemm_column_tail_split(torch_cuda, monkeypatch):
    """When the full waves hold whole columns of tiles rather than whole rows,
    the tail is the remaining columns.  Counting waves in 32 CUs, o_proj and
    down (N = 3072, 4 x 12 tiles at M = 1024) run columns [0, 2048) as one
    wave and columns [2048, 3072) in 2 K splits; checked in the plan, against
    the oracle and against the same prefill without tail splits."""
    cfg, W = random_block(45, dtype="bf16", d_model=3072, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=1024, o_bias=True, mlp_bias=True)
    rng = np.random.default_rng(23)
    x = rng.standard_normal((2, 512, 3072), dtype=np.float32)
    blk = _block(cfg, W)
    monkeypatch.setenv("GQA_GEMM_TILE192", "0")  # 256-wide tiles (the shape would take 256 x 192)
    monkeypatch.setenv("GQA_GEMM_TAIL_CUS", "0")
    plain = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.setenv("GQA_GEMM_TAIL_CUS", "32")
    plan = blk.describe_plan(2, 512)
    assert "gemm_o tile=7 splits=1 waves=0 tail_cols_from=2048 tail_splits=2" in plan, plan
    assert "gemm_down tile=7 splits=1 waves=0 tail_cols_from=2048 tail_splits=2" in plan, plan
    y = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.delenv("GQA_GEMM_TAIL_CUS")
    monkeypatch.delenv("GQA_GEMM_TILE192")
    check_close(y, block_forward(cfg, W, x, dtype=np.float32), x, "bf16", "column-tail GEMMs")
    check_close(y, plain, x, "bf16", "column-tail vs whole-wave GEMMs")


@pytest.mark.parametrize("qk_norm", [False, True])
def test_bf16_rope_q_in_attention_matches_rope_kernel(torch_cuda, monkeypatch, qk_norm):
    """The prefill attention kernel's own q norm + RoPE against the same
    prefill with q rotated by the RoPE kernel (GQA_ROPE_Q_IN_ATTN=0): both round
    float32 rotations of the same values to bf16 (contraction and the norm's
    order of summation may differ in the last bits), so the sublayer outputs
    agree far inside the bf16 tolerance, where a wrong rotation partner, sign or
    position would not; the fused path also against the oracle."""
    cfg, W = random_block(47 + qk_norm, dtype="bf16", d_model=512, n_heads=8, n_kv_heads=2, head_dim=128,
                          intermediate=768, qk_norm=qk_norm, norm="rmsnorm_offset" if qk_norm else "rmsnorm")
    rng = np.random.default_rng(31)
    x = rng.standard_normal((2, 300, 512), dtype=np.float32)
    blk = _block(cfg, W)
    y = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.setenv("GQA_ROPE_Q_IN_ATTN", "0")
    y0 = blk.forward(to_gpu(x)).cpu().numpy()
    monkeypatch.delenv("GQA_ROPE_Q_IN_ATTN")
    assert rel_err(y - x, y0 - x) < 2e-3
    check_close(y, block_forward(cfg, W, x, dtype=np.float32), x, "bf16", "q RoPE in attention")


def test_page_worked_example_golden(torch_cuda):
    """The HIP block on the mojolearn page's usage example (float32 weights,
    TransformerBlock(weights, n_heads=4) on x of shape (2, 16, 64)) against the
    stored float64 oracle output in tests/golden: sampled rows (y and y - x)
    and the whole-output sum, within the float32 tolerance."""
    from tests.golden.make_mojolearn_example import CFG, example_inputs, read
    W, x = example_inputs()
    y = _block(CFG, W).forward(to_gpu(x)).cpu().numpy().astype(np.float64)
    assert y.shape == x.shape
    ref = read()
    got = np.stack([y[b, t] for (b, t) in ref["rows"]])
    exp = np.stack(list(ref["rows"].values()))
    xs = np.stack([x[b, t] for (b, t) in ref["rows"]]).astype(np.float64)
    # The example's norm gains are 0.02-scale, so y - x is ~1e-3 of |y| and the
    # float32 output's own rounding (half an ulp of y, which the float64
    # reference does not have) is ~1e-4 of max|y - x|: the y - x bar adds two
    # ulps of max|y| to the float32 tolerance.
    e1 = rel_err(got, exp)
    dev = np.max(np.abs(got - exp))
    bar = 1e-4 * np.max(np.abs(exp - xs)) + 2.0 ** -22 * np.max(np.abs(exp))
    print(f"[parity] page example: err(y)={e1:.3e} max|dy|={dev:.3e} bar(y-x)={bar:.3e}")
    assert e1 <= 1e-4 and dev <= bar
    assert abs(y.sum() - ref["sum"]) <= 1e-4 * np.abs(y).sum()


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_ragged_prefill_lengths(torch_cuda, dtype):
    """mojolearn forward(x, lengths=...): a ragged batch against the oracle's
    reading of it (each row alone at its own length, padding +0.0), padding
    exactly positive zero, real positions equal to the unragged run's
    (causality: bitwise on the float32 padded path; to the bf16 bar on the
    packed path, whose GEMMs see 258 rows instead of 600 and so run other
    tiles), padding inputs changing nothing (bitwise), and the argument
    errors."""
    import torch
    from gqa_causal_attention_amd.binding import GqaError
    if dtype == "bf16":
        cfg, W = random_block(41, dtype="bf16", d_model=256, n_heads=8, n_kv_heads=2, head_dim=128,
                              intermediate=384)
        B, L, lens = 3, 200, [200, 57, 1]
    else:
        cfg, W = random_block(42, dtype="f32", window=6, attn_softcap=20.0)
        B, L, lens = 3, 13, [13, 5, 1]
    rng = np.random.default_rng(17)
    x = rng.standard_normal((B, L, cfg["d_model"]), dtype=np.float32)
    blk = _block(cfg, W)
    y = blk.forward(to_gpu(x), lengths=lens).cpu().numpy()
    ref = block_forward(cfg, W, x, dtype=oracle_dtype(cfg), lengths=lens)
    check_close(y, ref, x, dtype, f"ragged {dtype}")
    full = blk.forward(to_gpu(x)).cpu().numpy()
    x2 = x.copy()
    for i, n in enumerate(lens):
        pad = y[i, n:]
        assert np.all(pad == 0.0) and not np.any(np.signbit(pad)), f"row {i}: padding not +0.0"
        if dtype == "f32":
            np.testing.assert_array_equal(y[i, :n], full[i, :n])
        else:
            check_close(y[i, :n], full[i, :n], x[i, :n], dtype, f"ragged row {i} vs unragged")
        x2[i, n:] = rng.standard_normal((L - n, cfg["d_model"]), dtype=np.float32) * 3
    np.testing.assert_array_equal(blk.forward(to_gpu(x2), lengths=lens).cpu().numpy(), y)
    with pytest.raises(GqaError):
        blk.forward(to_gpu(x), lengths=[0] + lens[1:])
    with pytest.raises(GqaError):
        blk.forward(to_gpu(x), lengths=[L + 1] + lens[1:])
    with pytest.raises(ValueError):
        blk.forward(to_gpu(x), blk.allocate_state(B, L), lengths=lens)
    torch.cuda.synchronize()
