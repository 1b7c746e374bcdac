"""MI355X-native (gfx950) Llama-shaped decoder block: HIP kernels behind a C
ABI (include/gqa_block.h) with a thin ctypes binding.

    from gqa_causal_attention_amd import Block
    blk = Block(cfg, weights)            # cfg: dict of block options, weights: HF names
    st = blk.allocate_state(batch, max_tokens)
    y = blk.forward(x, st)               # x: float32 CUDA tensor [B, L, d]
    y_t = blk.step(x_t, st)

The library is built in-tree by ``python -m gqa_causal_attention_amd.build``;
importing the binding does not build it and there is no fallback path.
"""
from .binding import Block, GqaError, State, load_library  # noqa: F401

__all__ = ["Block", "GqaError", "State", "load_library"]
