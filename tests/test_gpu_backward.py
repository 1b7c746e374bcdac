"""Parity of the HIP backward (mojolearn TransformerBlock.backward: gradients of
a zero-state prefill for x and the nine weights) with the float64 oracle.

Bar: max|gpu - oracle| / max|oracle| per gradient tensor, the forward's bars:
1e-4 for float32 blocks, 2e-2 for bf16 blocks.  The bf16 backward rounds both
operands of every gradient product (dy, dgate | dup, dx1, dq | dk | dv as well
as the weights and activations) and measures 5e-3 .. 1e-2 (printed), so the
forward's bar still holds with a factor 2 to spare.
"""
import numpy as np
import pytest

from gqa_causal_attention_amd.workloads import random_block
from oracle import BACKWARD_WEIGHTS, block_backward
from tests.helpers import rel_err, to_gpu

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _check(cfg, W, x, dy, dtype, what):
    from gqa_causal_attention_amd import Block
    blk = Block(cfg, W)
    got = blk.backward(to_gpu(x), to_gpu(dy))
    ref = block_backward(cfg, W, x, dy, dtype=np.float64)
    worst = 0.0
    for name in ("x",) + BACKWARD_WEIGHTS:
        g = got[name].cpu().numpy()
        assert g.shape == ref[name].shape, name
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        e = rel_err(g, ref[name])
        worst = max(worst, e)
        assert e <= TOL[dtype], f"{what} {name}: err {e:.3e} > {TOL[dtype]}"
    print(f"[parity] backward {what}: worst err {worst:.3e} (tol {TOL[dtype]})")
    return got


CASES = {
    # name: (dtype, block overrides, B, L)
    "f32_tiny": ("f32", dict(), 2, 13),
    "f32_window": ("f32", dict(window=5), 2, 19),
    "f32_odd_dims": ("f32", dict(d_model=50, n_heads=5, n_kv_heads=5, head_dim=10, intermediate=37), 1, 9),
    # bf16 (matrix-core attention backward for head_dim 64 / 128): 128x128 GEMM tiles over
    # T = 300 (ragged), weight-gradient depth padded to 512
    "bf16_hd128_g4": ("bf16", dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=512,
                                   rope_theta=5e5), 1, 300),
    # T = 40: decode-sized products (weight-streaming kernel, K split), window
    "bf16_small_t_window": ("bf16", dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=320,
                                         window=16), 2, 20),
    # T = 700: the pipelined large-M tiles; q/k/v width 640 + 2 * 64 padded to the GEMM depth
    "bf16_large_t": ("bf16", dict(d_model=512, n_heads=5, n_kv_heads=1, head_dim=128, intermediate=768), 1, 700),
    # the attention backward's wave-kernel form: head_dim 256, and L = 1
    "bf16_hd256_wave_form": ("bf16", dict(d_model=256, n_heads=2, n_kv_heads=1, head_dim=256, intermediate=256,
                                          window=24), 1, 90),
    "bf16_single_position": ("bf16", dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=256), 3, 1),
    # T = 768 (a multiple of 64, above 512): every product reads its operands in
    # place (weights K-major for the input gradients, activations along the
    # token axis for the weight gradients), the small grids split along K; the
    # dk / dv weight gradients have M = 128 rows (a ragged 256-row tile)
    "bf16_in_place_t768": ("bf16", dict(d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=512), 2, 384),
    # the same with head_dim 128 (q width 1024 != d), a window, and the dk / dv
    # weight gradients split along K; both cases run SwiGLU's backward in the
    # epilogue of the da product (a single K split)
    "bf16_in_place_window": ("bf16", dict(d_model=256, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024,
                                          window=100), 1, 640),
}


@pytest.mark.parametrize("name", list(CASES))
def test_backward_parity(torch_cuda, name):
    dtype, over, B, L = CASES[name]
    cfg, W = random_block(400 + list(CASES).index(name), dtype=dtype, **over)
    rng = np.random.default_rng(401)
    x = rng.standard_normal((B, L, cfg["d_model"]), dtype=np.float32)
    dy = rng.standard_normal((B, L, cfg["d_model"]), dtype=np.float32)
    _check(cfg, W, x, dy, dtype, name)


@pytest.mark.parametrize("L", [128, 256])
def test_backward_llama3_8b_widths_short_sequence(torch_cuda, L):
    """The 8B block's widths (d 4096, 32/8 heads of 128, IT 14336) at L = 128
    (transposed copies) and L = 256 (weight gradients read in place)."""
    from gqa_causal_attention_amd.workloads import LLAMA3_8B_BLOCK, draw_weights
    cfg = dict(LLAMA3_8B_BLOCK)
    W = draw_weights(cfg, np.random.default_rng(402))
    rng = np.random.default_rng(403)
    x = rng.standard_normal((1, L, 4096), dtype=np.float32)
    dy = rng.standard_normal((1, L, 4096), dtype=np.float32)
    _check(cfg, W, x, dy, "bf16", f"llama3_8b_L{L}")


def test_backward_deterministic_and_overwrites(torch_cuda):
    import torch
    from gqa_causal_attention_amd import Block
    cfg, W = random_block(404, dtype="bf16", d_model=256, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=256)
    blk = Block(cfg, W)
    rng = np.random.default_rng(405)
    x = to_gpu(rng.standard_normal((1, 70, 256), dtype=np.float32))
    dy = to_gpu(rng.standard_normal((1, 70, 256), dtype=np.float32))
    g1 = blk.backward(x, dy)
    g1 = {k: v.clone() for k, v in g1.items()}
    prefilled = {k: torch.full_like(v, 7.0) for k, v in g1.items()}
    g2 = blk.backward(x, dy, grads=prefilled)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_errors(torch_cuda):
    import torch
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.binding import GqaError
    cfg, W = random_block(406, qkv_bias=True)
    blk = Block(cfg, W)
    x = torch.zeros(1, 4, 64, device="cuda")
    with pytest.raises(GqaError) as e:
        blk.backward(x, torch.zeros_like(x))
    assert e.value.name == "UNSUPPORTED"
    cfg, W = random_block(407, max_positions=8)
    blk = Block(cfg, W)
    x = torch.zeros(1, 9, 64, device="cuda")
    with pytest.raises(GqaError) as e:
        blk.backward(x, torch.zeros_like(x))
    assert e.value.name == "POSITION"


@pytest.mark.timeout(900)
def test_backward_llama3_8b_same_plan_as_4k(torch_cuda):
    """The 8B block's backward in the launch plan the bench times at B=1,
    L=4096: B=2 rows of L=2048 make the same T=4096 tokens, so every gradient
    product runs the same tiles, transposed-operand modes, K splits and fused
    SwiGLU epilogue (asserted from the library's own plan), while the float64
    oracle's attention stays at 2048 x 2048 per head."""
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.workloads import LLAMA3_8B_BLOCK, draw_weights
    cfg = dict(LLAMA3_8B_BLOCK)
    W = draw_weights(cfg, np.random.default_rng(402))
    blk = Block(cfg, W)
    plan = blk.describe_plan(2, 2048, backward=True)
    assert plan == blk.describe_plan(1, 4096, backward=True), plan
    assert "tr_dx=1 tr_dw=1 fuse_swiglu=1 mfma_attention=1" in plan, plan
    del blk
    rng = np.random.default_rng(408)
    x = rng.standard_normal((2, 2048, 4096), dtype=np.float32)
    dy = rng.standard_normal((2, 2048, 4096), dtype=np.float32)
    _check(cfg, W, x, dy, "bf16", "llama3_8b_B2_L2048 (the 4k plan)")
