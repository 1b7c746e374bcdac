"""Shared helpers of the GPU tests: run the HIP block and the CPU oracle on the
same seeded inputs and compare them."""
import numpy as np

from oracle import OracleState, block_forward, block_step

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(got - ref)) / (den if den > 0 else 1.0))


def row_err(got, ref):
    """Worst row of max|got - ref| / max|ref|, each token row (last axis)
    normalised by its own largest reference value."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, np.shape(got)[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    den = np.max(np.abs(ref), axis=1)
    num = np.max(np.abs(got - ref), axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def check_close(y_gpu, y_ref, x, dtype, what=""):
    """The parity bar: max|g - r| / max|r| on y and on y - x (the sublayers'
    sum), and on y - x row by row (each token row normalised by its own
    largest value, so rows whose sublayer output is small are held to the bar
    as well)."""
    tol = TOL[dtype]
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite GPU output"
    e1 = rel_err(y_gpu, y_ref)
    e2 = rel_err(y_gpu - x, y_ref - x)
    e3 = row_err(y_gpu - x, y_ref - x)
    print(f"[parity] {what}: err(y)={e1:.3e} err(y-x)={e2:.3e} worst row of y-x={e3:.3e} tol={tol}")
    assert e1 <= tol and e2 <= tol and e3 <= tol, \
        f"{what}: err(y)={e1:.3e} err(y-x)={e2:.3e} worst row of y-x={e3:.3e} tol={tol}"
    return e1, e2


def to_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def fill_state_gpu(st, k_fill, v_fill, lengths):
    import torch
    st.k.copy_(torch.from_numpy(k_fill).to(st.k.dtype))
    st.v.copy_(torch.from_numpy(v_fill).to(st.v.dtype))
    st.set_lengths(lengths)


def oracle_dtype(cfg):
    return np.float64 if cfg["dtype"] == "f32" else np.float32


__all__ = ["TOL", "rel_err", "row_err", "check_close", "to_gpu", "fill_state_gpu", "oracle_dtype", "OracleState",
           "block_forward", "block_step"]
