"""Invariants of the GPU block (the page's guarantees and the structure of the
method), checked on the HIP path itself, plus the host-side error contract
exercised with a live device.

* run-to-run determinism (bitwise) and causal invariance (bitwise for
  tokens past a 32-position boundary: no kernel reads later tokens);
* decode token by token == one prefill, chunked continuation == whole
  prefill, a window at least L wide == full causal, GQA == MHA with the kv
  heads repeated (all within the bf16 bar: different kernels, different
  summation orders);
* state snapshot / restore: copying the cache and lengths out and back
  resumes the sequence exactly;
* errors raised before any launch: batch mismatch, capacity, max_positions,
  step without a state, short workspace; non-finite input reported by
  status()."""
import numpy as np
import pytest

from gqa_causal_attention_amd.workloads import random_block
from tests.helpers import check_close, rel_err, to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _blk(cfg, W):
    from gqa_causal_attention_amd import Block
    return Block(cfg, W)


LLAMA_SMALL = dict(d_model=512, n_heads=8, n_kv_heads=2, head_dim=128, intermediate=1024, rope_theta=5e5)


def test_determinism_and_causal_invariance(torch_cuda):
    cfg, W = random_block(400, dtype="bf16", **LLAMA_SMALL)
    blk = _blk(cfg, W)
    x = np.random.default_rng(1).standard_normal((2, 1024, 512), dtype=np.float32)
    y1 = blk.forward(to_gpu(x)).cpu().numpy()
    y2 = blk.forward(to_gpu(x)).cpu().numpy()
    np.testing.assert_array_equal(y1, y2)
    x2 = x.copy()
    x2[:, 640:] = np.random.default_rng(2).standard_normal((2, 384, 512))
    y3 = blk.forward(to_gpu(x2)).cpu().numpy()
    np.testing.assert_array_equal(y3[:, :640], y1[:, :640])
    assert not np.allclose(y3[:, 640:], y1[:, 640:])


@pytest.mark.parametrize("window", [0, 96])
def test_decode_and_chunks_equal_prefill(torch_cuda, window):
    cfg, W = random_block(401, dtype="bf16", window=window, **LLAMA_SMALL)
    blk = _blk(cfg, W)
    x = np.random.default_rng(3).standard_normal((2, 300, 512), dtype=np.float32)
    whole = blk.forward(to_gpu(x), blk.allocate_state(2, 300)).cpu().numpy()
    st = blk.allocate_state(2, 300)
    parts = [blk.forward(to_gpu(x[:, :170]), st), blk.forward(to_gpu(x[:, 170:290]), st)]
    for t in range(290, 300):
        parts.append(blk.step(to_gpu(x[:, t]), st))
    inc = np.concatenate([p.cpu().numpy() for p in parts], axis=1)
    check_close(inc, whole, x, "bf16", "incremental vs whole")


def test_window_at_least_L_is_full_causal(torch_cuda):
    cfg, W = random_block(402, dtype="bf16", **LLAMA_SMALL)
    x = np.random.default_rng(4).standard_normal((1, 200, 512), dtype=np.float32)
    full = _blk(cfg, W).forward(to_gpu(x)).cpu().numpy()
    wide = _blk(dict(cfg, window=200), W).forward(to_gpu(x)).cpu().numpy()
    check_close(wide, full, x, "bf16", "window >= L")


def test_gqa_equals_mha_with_repeated_kv(torch_cuda):
    cfg, W = random_block(403, dtype="bf16", **LLAMA_SMALL)
    G = cfg["n_heads"] // cfg["n_kv_heads"]
    hd = cfg["head_dim"]
    mha = dict(cfg, n_kv_heads=cfg["n_heads"])
    Wm = dict(W)
    for n in ("k_proj.weight", "v_proj.weight"):
        w = W[n].reshape(cfg["n_kv_heads"], hd, -1)
        Wm[n] = np.repeat(w, G, axis=0).reshape(cfg["n_heads"] * hd, -1)
    x = np.random.default_rng(5).standard_normal((2, 150, 512), dtype=np.float32)
    a = _blk(cfg, W).forward(to_gpu(x)).cpu().numpy()
    b = _blk(mha, Wm).forward(to_gpu(x)).cpu().numpy()
    check_close(b, a, x, "bf16", "GQA vs MHA")


def test_state_snapshot_restore(torch_cuda):
    torch = torch_cuda
    cfg, W = random_block(404, dtype="bf16", **LLAMA_SMALL)
    blk = _blk(cfg, W)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 40, 512), dtype=np.float32)
    steps = rng.standard_normal((6, 3, 512), dtype=np.float32)
    st = blk.allocate_state(3, 64)
    blk.forward(to_gpu(x), st)
    for i in range(3):
        blk.step(to_gpu(steps[i]), st)
    snap = (st.k.clone(), st.v.clone(), st.host_lengths())
    ref = [blk.step(to_gpu(steps[i]), st).cpu().numpy() for i in range(3, 6)]
    st2 = blk.allocate_state(3, 64)
    st2.k.copy_(snap[0])
    st2.v.copy_(snap[1])
    st2.set_lengths(snap[2])
    got = [blk.step(to_gpu(steps[i]), st2).cpu().numpy() for i in range(3, 6)]
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    assert torch.equal(st.k, st2.k)


def test_error_contract(torch_cuda):
    torch = torch_cuda
    from gqa_causal_attention_amd import GqaError
    cfg, W = random_block(405, dtype="bf16", max_positions=100, **dict(LLAMA_SMALL))
    blk = _blk(cfg, W)
    st = blk.allocate_state(2, 50)
    x = to_gpu(np.zeros((2, 10, 512), dtype=np.float32))
    with pytest.raises(GqaError) as e:
        blk.forward(to_gpu(np.zeros((3, 10, 512), dtype=np.float32)), st)
    assert e.value.name == "STATE"
    with pytest.raises(GqaError) as e:
        blk.forward(to_gpu(np.zeros((2, 51, 512), dtype=np.float32)), st)
    assert e.value.name == "CAPACITY"
    with pytest.raises(GqaError) as e:
        blk.forward(to_gpu(np.zeros((1, 101, 512), dtype=np.float32)))
    assert e.value.name == "POSITION"
    with pytest.raises(GqaError) as e:
        blk.step(to_gpu(np.zeros((2, 512), dtype=np.float32)), None)
    assert e.value.name == "STATE"
    with pytest.raises(GqaError) as e:
        st.set_lengths([60, 0])
    assert e.value.name == "CAPACITY"
    # a failed call leaves the state untouched
    assert st.host_lengths().tolist() == [0, 0]
    blk.forward(x, st)
    assert st.host_lengths().tolist() == [10, 10]
    # workspace too small: call the ABI directly
    import ctypes
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    rc = blk.lib.gqa_block_forward(blk.handle, st.handle, ctypes.c_void_p(x.data_ptr()),
                                   ctypes.c_void_p(y.data_ptr()), 2, 10, ctypes.c_void_p(ws.data_ptr()),
                                   16, None)
    assert rc == -8
    assert st.host_lengths().tolist() == [10, 10]
    # a non-finite input is reported by status() (and the flag then clears)
    xb = np.zeros((2, 1, 512), dtype=np.float32)
    xb[1, 0, 7] = np.inf
    blk.step(to_gpu(xb), st)
    with pytest.raises(GqaError) as e:
        blk.status()
    assert e.value.name == "NONFINITE"
    blk.status()


def test_nonfinite_weights_refused(torch_cuda):
    from gqa_causal_attention_amd import GqaError
    cfg, W = random_block(406, dtype="bf16", **LLAMA_SMALL)
    W = dict(W)
    bad = W["gate_proj.weight"].copy()
    bad[3, 5] = np.nan
    W["gate_proj.weight"] = bad
    with pytest.raises(GqaError) as e:
        _blk(cfg, W)
    assert e.value.name == "NONFINITE"


def test_empty_inputs(torch_cuda):
    torch = torch_cuda
    cfg, W = random_block(407, dtype="bf16", **LLAMA_SMALL)
    blk = _blk(cfg, W)
    st = blk.allocate_state(2, 8)
    y = blk.forward(torch.zeros((2, 0, 512), dtype=torch.float32, device="cuda"), st)
    assert y.shape == (2, 0, 512)
    assert st.host_lengths().tolist() == [0, 0]


def test_decode_step_graph_replays_match_eager(torch_cuda):
    """The decode step captured in a HIP graph (positions restored on the device
    inside the graph): every replay equals the eager step bit for bit, with
    eager work and synchronisations between the replays."""
    torch = torch_cuda
    cfg, W = random_block(408, dtype="bf16", **LLAMA_SMALL)
    blk = _blk(cfg, W)
    rng = np.random.default_rng(11)
    B = 4
    st = blk.allocate_state(B, 600)
    blk.forward(to_gpu(rng.standard_normal((B, 500, 512), dtype=np.float32)), st)
    lengths = st.host_lengths().copy()
    x = to_gpu(rng.standard_normal((B, 1, 512), dtype=np.float32))
    y = torch.empty_like(x)
    k0, v0 = st.k.clone(), st.v.clone()
    ref = blk.step(x, st).clone()
    st.set_lengths(lengths)
    blk.step(x, st, out=y)
    torch.cuda.synchronize()
    lengths_dev = torch.from_numpy(lengths.astype(np.int32)).cuda()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.lengths.copy_(lengths_dev)
        blk.step(x, st, out=y)
    other = _blk(cfg, W)  # unrelated eager work on its own workspace (the graph holds blk's)
    for i in range(4):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref.cpu().numpy())
        assert st.lengths.cpu().tolist() == (lengths + 1).tolist()
        _ = other.forward(to_gpu(rng.standard_normal((1, 8, 512), dtype=np.float32)))
        torch.cuda.synchronize()
    assert torch.equal(st.v[:, :, :500], v0[:, :, :500])


def test_prefill_graph_replays_match_eager(torch_cuda):
    """A self-contained prefill on the large-M GEMM and flash paths (M > 512),
    captured in a HIP graph: every replay equals the eager forward bit for bit,
    with eager work and synchronisations between the replays."""
    torch = torch_cuda
    cfg, W = random_block(409, dtype="bf16", **LLAMA_SMALL)
    blk = _blk(cfg, W)
    rng = np.random.default_rng(12)
    x = to_gpu(rng.standard_normal((1, 700, 512), dtype=np.float32))
    y = torch.empty_like(x)
    ref = blk.forward(x).clone()
    blk.forward(x, out=y)  # workspace allocated before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        blk.forward(x, out=y)
    for i in range(3):
        y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref.cpu().numpy())
        # unrelated eager work (a smaller call: blk's captured workspace is kept)
        _ = blk.forward(to_gpu(rng.standard_normal((2, 9, 512), dtype=np.float32)))
        torch.cuda.synchronize()
