"""Parity at the full workload sizes, in the launch configuration the bench
times, on sampled outputs the oracle computes row by row
(``block_forward_rows`` for prefills; ``block_step`` on a sub-batch of rows
for decode, rows being independent).  Bar: 2e-2 (bf16 weights) on y and y - x
over the sampled rows."""
import numpy as np
import pytest

from gqa_causal_attention_amd.workloads import make_workload
from oracle import OracleState, block_forward_rows, block_step
from tests.helpers import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _sample_rows(B, L, extra, seed):
    rng = np.random.default_rng(seed)
    ts = set(int(t) for t in extra if t < L) | set(int(t) for t in rng.integers(0, L, 6))
    return [(b, t) for b in range(B) for t in sorted(ts)]


def _attention_only(W):
    """The block's weights with down_proj zeroed: the MLP then adds exactly
    0, so y - x is the attention sublayer's output (o_proj of the attention)
    alone, in the GPU run and in the oracle alike."""
    W = dict(W)
    W["down_proj.weight"] = np.zeros_like(W["down_proj.weight"])
    return W


def _prefill_case(torch, name, extra_rows, with_state, attention_only=False):
    from gqa_causal_attention_amd import Block
    wl = make_workload(name)
    cfg, W, x = wl["cfg"], wl["weights"], wl["x"]
    if attention_only:
        W = _attention_only(W)
    B, L = x.shape[:2]
    blk = Block(cfg, W)
    xg = torch.from_numpy(x).cuda()
    if with_state:
        st = blk.allocate_state(B, wl["capacity"])
        y = blk.forward(xg, st)
        assert st.host_lengths().tolist() == [L] * B
    else:
        y = blk.forward(xg)
    rows = _sample_rows(B, L, extra_rows, 99)
    idx_b = torch.tensor([b for b, _ in rows], device="cuda")
    idx_t = torch.tensor([t for _, t in rows], device="cuda")
    yg = y[idx_b, idx_t].cpu().numpy()
    del y, xg
    ref = block_forward_rows(cfg, W, x, rows)
    xs = np.stack([x[b, t] for b, t in rows])
    check_close(yg, ref, xs, "bf16", name + (" attention sublayer" if attention_only else ""))


def test_llama3_8b_prefill_4k(torch_cuda):
    _prefill_case(torch_cuda, "llama3_8b_prefill_4k", [0, 1, 31, 32, 63, 64, 2047, 2048, 4094, 4095], False)


def test_llama3_8b_prefill_4k_with_cache(torch_cuda):
    _prefill_case(torch_cuda, "llama3_8b_prefill_4k", [0, 255, 256, 4095], True)


def test_gemma2_window_prefill_8k(torch_cuda):
    _prefill_case(torch_cuda, "gemma2_window_prefill_8k", [0, 4094, 4095, 4096, 4097, 6000, 8191], True)


def test_qwen_long_prefill_32k(torch_cuda):
    _prefill_case(torch_cuda, "qwen_long_prefill_32k", [0, 1, 16383, 32766, 32767], False)


def _decode_case(torch, name, rows, attention_only=False):
    from gqa_causal_attention_amd import Block
    wl = make_workload(name)
    cfg, W, x, lengths = wl["cfg"], wl["weights"], wl["x"], wl["lengths"]
    if attention_only:
        W = _attention_only(W)
    B, cap = wl["batch"], wl["capacity"]
    blk = Block(cfg, W)
    st = blk.allocate_state(B, cap)
    st.k.copy_(torch.from_numpy(wl["k_fill"]).cuda().to(torch.bfloat16))
    st.v.copy_(torch.from_numpy(wl["v_fill"]).cuda().to(torch.bfloat16))
    st.set_lengths(lengths)
    y = blk.step(torch.from_numpy(x).cuda(), st).cpu().numpy()
    assert st.host_lengths().tolist() == (lengths + 1).tolist()
    rows = sorted(set(rows) | {int(np.argmax(lengths)), int(np.argmin(lengths))})
    ost = OracleState.from_fill(cfg, wl["k_fill"][rows], wl["v_fill"][rows], lengths[rows])
    ref = block_step(cfg, W, x[rows], ost)
    check_close(y[rows], ref, x[rows], "bf16", name + (" attention sublayer" if attention_only else ""))
    # the new token's key/value landed in slot p_b (post-RoPE key, bf16)
    kc = st.k.float().cpu().numpy()
    for i, b in enumerate(rows):
        np.testing.assert_allclose(kc[b, :, lengths[b]], ost.k[i, :, lengths[b]], rtol=2e-2,
                                   atol=2e-2 * np.abs(ost.k[i, :, lengths[b]]).max())


def test_llama3_8b_decode_b64(torch_cuda):
    _decode_case(torch_cuda, "llama3_8b_decode_b64", [0, 21, 42, 63])


def test_qwen_long_decode_b16(torch_cuda):
    _decode_case(torch_cuda, "qwen_long_decode_b16", [0, 15])


# The attention sublayer alone (down_proj zeroed, so y - x = o_proj(attention)),
# checked row by row: at these sizes the MLP's output is several times the
# attention's, so a whole-block bar alone would not see a wrong attention on
# long rows.
def test_attention_only_llama3_8b_prefill_4k(torch_cuda):
    _prefill_case(torch_cuda, "llama3_8b_prefill_4k", [0, 1, 63, 64, 2047, 4095], True, attention_only=True)


def test_attention_only_gemma2_window_prefill_8k(torch_cuda):
    _prefill_case(torch_cuda, "gemma2_window_prefill_8k", [0, 4095, 4096, 8191], True, attention_only=True)


def test_attention_only_qwen_long_prefill_32k(torch_cuda):
    _prefill_case(torch_cuda, "qwen_long_prefill_32k", [0, 16383, 32767], False, attention_only=True)


def test_attention_only_llama3_8b_decode_b64(torch_cuda):
    _decode_case(torch_cuda, "llama3_8b_decode_b64", [0, 21, 42, 63], attention_only=True)


def test_attention_only_qwen_long_decode_b16(torch_cuda):
    _decode_case(torch_cuda, "qwen_long_decode_b16", [0, 7, 15], attention_only=True)


def test_llama3_8b_continuation_2k_2k_then_steps(torch_cuda):
    """Continuation from a carried cache at the 8B shape: prefill the first
    2048 tokens of the 4k workload into a state, forward the other 2048 on
    that state, then 4 single-token steps, each against the oracle carrying
    its own state (sampled rows of the prefills, every step)."""
    torch = torch_cuda
    from gqa_causal_attention_amd import Block
    wl = make_workload("llama3_8b_prefill_4k")
    cfg, W, x = wl["cfg"], wl["weights"], wl["x"]
    steps = np.random.default_rng(77).standard_normal((4, 1, 1, cfg["d_model"]), dtype=np.float32)
    cap = 4096 + 4
    blk = Block(cfg, W)
    st = blk.allocate_state(1, cap)
    ost = OracleState(cfg, 1, cap)
    for i, (lo, hi) in enumerate(((0, 2048), (2048, 4096))):
        xc = np.ascontiguousarray(x[:, lo:hi])
        y = blk.forward(torch.from_numpy(xc).cuda(), st)
        assert st.host_lengths().tolist() == [hi]
        ts = sorted({0, 1, 63, 64, 1023, 2046, 2047} | set(np.random.default_rng(i).integers(0, 2048, 5).tolist()))
        idx = torch.tensor(ts, device="cuda")
        yg = y[0, idx].cpu().numpy()
        ref = block_forward_rows(cfg, W, xc, [(0, t) for t in ts], state=ost)
        check_close(yg, ref, xc[0, ts], "bf16", f"8B continuation chunk {i} (positions {lo}..{hi - 1})")
        if i == 0:
            # the oracle's state after the first chunk (the second chunk's rows read it)
            from oracle import block_forward as oracle_forward
            oracle_forward(cfg, W, xc, ost)
    # the oracle state must hold the second chunk too before the steps
    from oracle import block_forward as oracle_forward
    oracle_forward(cfg, W, np.ascontiguousarray(x[:, 2048:]), ost)
    assert ost.lengths.tolist() == [4096]
    for j in range(4):
        yg = blk.step(torch.from_numpy(steps[j]).cuda(), st).cpu().numpy()
        ref = block_step(cfg, W, steps[j], ost)
        check_close(yg, ref, steps[j], "bf16", f"8B continuation step {j} (position {4096 + j})")
    assert st.host_lengths().tolist() == [4100]
