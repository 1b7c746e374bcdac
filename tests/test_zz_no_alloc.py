"""The no-allocation decode step (gqa_block_step_noalloc): called through the
C ABI, it must produce exactly what gqa_block_step produces on the same state
and inputs -- two calls in a row, the second with fewer rows (the shared
scratch keeps the first call's contents) -- and refuse a step whose workspace
exceeds its fixed scratch before launching anything."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _filled_states(torch, blk, B, cap, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    lengths = np.random.default_rng(seed).integers(cap // 4, cap - 1, size=B).astype(np.int32)
    states = []
    k = torch.randn((B, blk.cfg["n_kv_heads"], cap, blk.cfg["head_dim"]), generator=g, device="cuda")
    v = torch.randn(k.shape, generator=g, device="cuda")
    for _ in range(2):
        st = blk.allocate_state(B, cap)
        st.k.copy_(k.to(st.k.dtype))
        st.v.copy_(v.to(st.v.dtype))
        st.set_lengths(lengths)
        states.append(st)
    return states, lengths


def test_step_noalloc_equals_step(torch_cuda):
    torch = torch_cuda
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.binding import GqaError
    from gqa_causal_attention_amd.workloads import LLAMA3_8B_BLOCK, draw_weights
    cfg = dict(LLAMA3_8B_BLOCK)
    blk = Block(cfg, draw_weights(cfg, np.random.default_rng(600)))
    rng = np.random.default_rng(601)
    for B, cap in ((64, 2048), (16, 1024)):          # the second call: a smaller input
        (st_ref, st), lengths = _filled_states(torch, blk, B, cap, 602 + B)
        x = torch.from_numpy(rng.standard_normal((B, 1, 4096), dtype=np.float32)).cuda()
        y_ref = blk.step(x, st_ref)
        y = torch.full_like(y_ref, float("nan"))
        blk.step_noalloc(x, st, out=y)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"B={B}: max |diff| {(y - y_ref).abs().max().item():.3e}"
        assert torch.equal(st.k, st_ref.k) and torch.equal(st.v, st_ref.v)
        assert st.host_lengths().tolist() == (lengths + 1).tolist() == st_ref.host_lengths().tolist()
        assert torch.equal(st.lengths, st_ref.lengths)
        blk.status()
    # a step whose workspace exceeds the fixed scratch is refused before any launch
    B = 2048
    st = blk.allocate_state(B, 2)
    x = torch.zeros((B, 1, 4096), device="cuda")
    y = torch.full((B, 1, 4096), 7.0, device="cuda")
    with pytest.raises(GqaError) as e:
        blk.step_noalloc(x, st, out=y)
    assert e.value.name == "WORKSPACE" and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert st.host_lengths().tolist() == [0] * B and int(st.lengths.abs().sum().item()) == 0
    assert bool((y == 7.0).all())
