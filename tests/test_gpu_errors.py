"""Error paths on the GPU: the binding's argument checks (raised before any
pointer reaches the library, so nothing is launched) and the optional
non-finite scan of the cached keys/values (mojolearn TransformerBlock: cache
values are checked like inputs), whose count is checked against the same
count taken on the host copy of the cache."""
import os

import numpy as np
import pytest

from gqa_causal_attention_amd.workloads import random_block

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def test_binding_rejects_bad_arguments(torch_cuda):
    torch = torch_cuda
    from gqa_causal_attention_amd import Block
    cfg, W = random_block(500, dtype="bf16", d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=256)
    blk = Block(cfg, W)
    other = Block(cfg, W)
    st = blk.allocate_state(2, 16)
    good = torch.zeros(2, 3, 128, device="cuda")
    bad = [
        (lambda: blk.forward(torch.zeros(2, 3, 127, device="cuda")), "shape"),        # wrong d_model
        (lambda: blk.forward(torch.zeros(2, 3, 128)), "on cpu"),                        # host tensor
        (lambda: blk.forward(torch.zeros(2, 3, 128, device="cuda", dtype=torch.float16)), "float32"),
        (lambda: blk.forward(torch.zeros(2, 128, 3, device="cuda").transpose(1, 2)), "contiguous"),
        (lambda: blk.forward(good, out=torch.zeros(2, 3, 64, device="cuda")), "shape"),
        (lambda: blk.forward(good, out=torch.zeros(2, 3, 128)), "on cpu"),
        (lambda: blk.forward(good, other.allocate_state(2, 16)), "state"),
        (lambda: blk.forward(good, lengths=[1, 2, 3]), "lengths"),
        (lambda: blk.step(torch.zeros(2, 2, 128, device="cuda"), st), "x must be"),
        (lambda: blk.step(torch.zeros(2, 127, device="cuda"), st), "shape"),
        (lambda: blk.step(torch.zeros(2, 128, device="cuda"), st, out=torch.zeros(3, 128, device="cuda")), "out"),
        (lambda: blk.backward(good, torch.zeros(2, 3, 64, device="cuda")), "shape"),
        (lambda: blk.backward(good, torch.zeros_like(good), grads={"x": torch.zeros_like(good)}), "grads"),
    ]
    for fn, what in bad:
        with pytest.raises(ValueError) as e:
            fn()
        assert what.split()[0] in str(e.value) or what in str(e.value).lower(), (what, str(e.value))
    torch.cuda.synchronize()
    assert st.host_lengths().tolist() == [0, 0]       # nothing ran on the state


def _host_count(st, lengths, window):
    k = st.k.float().cpu().numpy()
    v = st.v.float().cpu().numpy()
    n = 0
    for b, ln in enumerate(lengths):
        used = min(int(ln), window) if window else int(ln)
        n += int(np.count_nonzero(~np.isfinite(k[b, :, :used])) + np.count_nonzero(~np.isfinite(v[b, :, :used])))
    return n


@pytest.mark.parametrize("dtype,window", [("bf16", 0), ("f32", 0), ("bf16", 8)])
def test_check_finite_counts_cached_values(torch_cuda, dtype, window, monkeypatch):
    """GQA_CHECK_FINITE=1 at create: each call with a state counts the
    non-finite values in the rows' used cache slots; values in unused slots
    (at or past a row's length) are not counted; without the option nothing
    is reported."""
    torch = torch_cuda
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.binding import GqaError
    cfg, W = random_block(501, dtype=dtype, d_model=128, n_heads=4, n_kv_heads=2, head_dim=32, intermediate=256,
                          window=window)
    lengths = [10, 12, 3]
    cap = 24
    rng = np.random.default_rng(502)
    x = torch.from_numpy(rng.standard_normal((3, 1, 128), dtype=np.float32)).cuda()
    for on in (True, False):
        if on:
            monkeypatch.setenv("GQA_CHECK_FINITE", "1")
        else:
            monkeypatch.delenv("GQA_CHECK_FINITE", raising=False)
        blk = Block(cfg, W)
        st = blk.allocate_state(3, cap)
        st.k.copy_(torch.from_numpy(rng.standard_normal(tuple(st.k.shape), dtype=np.float32)))
        st.v.copy_(torch.from_numpy(rng.standard_normal(tuple(st.v.shape), dtype=np.float32)))
        st.k[0, 1, 4, 7] = float("nan")        # used (row 0 holds 10, or the last W of them)
        st.v[1, 0, 7, 0] = float("inf")        # used
        st.k[1, 0, 5, 1] = float("-inf")       # used
        if not window:
            st.k[2, 1, 20, 3] = float("nan")   # row 2 holds 3: unused slot, not counted
            st.v[0, 0, 11, 5] = float("nan")   # row 0 holds 10: unused slot
        st.set_lengths(lengths)
        expect = _host_count(st, lengths, window)
        assert expect == 3
        blk.step(x, st)
        if on:
            with pytest.raises(GqaError) as e:
                blk.status()
            assert e.value.name == "NONFINITE" and f"{expect} non-finite cached" in str(e.value), str(e.value)
            blk.status()        # cleared
        else:
            blk.status()
    monkeypatch.delenv("GQA_CHECK_FINITE", raising=False)


@pytest.mark.parametrize("dtype,window,L,dev_len", [
    ("bf16", 0, 1, 16 + 5),     # decode step, device start past the capacity
    ("bf16", 0, 1, -7),         # decode step, negative device start
    ("f32", 0, 3, 15),          # continuation: start + L past the capacity
    ("bf16", 0, 5, 14),         # bf16 continuation (matrix-core prefill attention)
    ("bf16", 8, 5, 8192 + 1),   # window ring: start past the RoPE tables (max_positions)
])
def test_device_position_guard(torch_cuda, dtype, window, L, dev_len):
    """A device start position the host mirror does not know of (what a replayed
    captured step leaves when it does not restore the lengths), outside the
    cache or the RoPE tables, is clamped by the kernels and reported by
    status() as a position error; restoring the lengths recovers."""
    torch = torch_cuda
    from gqa_causal_attention_amd import Block
    from gqa_causal_attention_amd.binding import GqaError
    cfg, W = random_block(503, dtype=dtype, d_model=128, n_heads=4, n_kv_heads=2, head_dim=64, intermediate=256,
                          window=window, max_positions=8192)
    if dtype == "bf16":     # the matrix-core attention kernels take these shapes
        plan = blk_plan = Block(cfg, W).describe_plan(2, L)
        assert ("decode_splitk" if L == 1 else "prefill_mfma") in blk_plan, plan
    rng = np.random.default_rng(504)
    blk = Block(cfg, W)
    st = blk.allocate_state(2, 16)
    blk.forward(torch.from_numpy(rng.standard_normal((2, 4, 128), dtype=np.float32)).cuda(), st)
    blk.status()
    shape = (2, 128) if L == 1 else (2, L, 128)
    x = torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).cuda()
    st.lengths.fill_(dev_len)           # device copy only; the host mirror still says 4
    y = blk.step(x, st) if L == 1 else blk.forward(x, st)
    torch.cuda.synchronize()
    with pytest.raises(GqaError) as e:
        blk.status()
    assert e.value.name == "POSITION" and "restore" in str(e.value), str(e.value)
    blk.status()                        # cleared
    st.set_lengths([4, 4])
    y = blk.step(x, st) if L == 1 else blk.forward(x, st)
    blk.status()
    assert torch.isfinite(y).all()
