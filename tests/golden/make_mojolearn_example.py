"""Writes mojolearn_example.txt: the oracle's output on the usage example of the
mojolearn.transformer page (TransformerBlock, "Examples": d = 64, it = 128,
n_heads = 4, weights and x drawn from numpy default_rng(0) in the order the
example lists them, weights scaled by 0.02, x of shape (2, 16, 64)).

The page prints the example's inputs but not its output, so the stored values
are the float64 oracle's (this script calls only oracle/ and numpy).  They are
a fixed expected output for the GPU path on the page's own worked example and
a regression record for the oracle.

    python tests/golden/make_mojolearn_example.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import block_forward  # noqa: E402

D, IT, H = 64, 128, 4
# the example's `shapes` dict, in its order
SHAPES = {"input_layernorm.weight": (D,), "post_attention_layernorm.weight": (D,),
          "q_proj.weight": (D, D), "k_proj.weight": (D, D), "v_proj.weight": (D, D),
          "o_proj.weight": (D, D), "gate_proj.weight": (IT, D), "up_proj.weight": (IT, D),
          "down_proj.weight": (D, IT)}
# TransformerBlock(weights, n_heads=4) with the page's defaults: n_kv_heads = n_heads,
# head_dim = d / n_heads, rope_theta 10000, RMSNorm eps 1e-6, SwiGLU, full causal
CFG = dict(d_model=D, n_heads=H, n_kv_heads=H, head_dim=D // H, intermediate=IT, window=0,
           rope_theta=10000.0, norm_eps=1e-6, attn_softcap=0.0, norm="rmsnorm", mlp="swiglu",
           qkv_bias=False, qk_norm=False, max_positions=64, dtype="f32")
# sampled outputs stored in full: (row, position) pairs
SAMPLES = [(0, 0), (0, 7), (0, 15), (1, 0), (1, 9), (1, 15)]


def example_inputs():
    rng = np.random.default_rng(0)
    weights = {k: rng.standard_normal(s, dtype=np.float32) * 0.02 for k, s in SHAPES.items()}
    x = rng.standard_normal((2, 16, D), dtype=np.float32)
    return weights, x


def oracle_output():
    weights, x = example_inputs()
    return block_forward(CFG, weights, x, dtype=np.float64)


def write(path=os.path.join(HERE, "mojolearn_example.txt")):
    y = np.asarray(oracle_output(), dtype=np.float64)
    with open(path, "w") as f:
        f.write("# mojolearn.transformer page, TransformerBlock Examples: output of the float64 oracle\n")
        f.write("# (written by tests/golden/make_mojolearn_example.py; the page prints no output values)\n")
        f.write(f"sum {y.sum():.17g}\n")
        f.write(f"sumsq {np.square(y).sum():.17g}\n")
        for b, t in SAMPLES:
            f.write(f"y {b} {t} " + " ".join(f"{v:.17g}" for v in y[b, t]) + "\n")


def read(path=os.path.join(HERE, "mojolearn_example.txt")):
    out = {"rows": {}}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            parts = line.split()
            if parts[0] in ("sum", "sumsq"):
                out[parts[0]] = float(parts[1])
            else:
                out["rows"][(int(parts[1]), int(parts[2]))] = np.array([float(v) for v in parts[3:]])
    return out


if __name__ == "__main__":
    write()
