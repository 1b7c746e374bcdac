"""CPU oracle of the decoder block.  TEST INFRASTRUCTURE ONLY: imported by the
tests, the smoke check and the bench's CPU baseline leg, never by the product
path.  See ``oracle.block`` for what it computes and the passages it follows."""
from .block import (BACKWARD_WEIGHTS, MLP_KINDS, backward_supported, block_backward, OracleState, apply_rope, attention_row, block_forward, block_forward_rows,
                    block_step, gelu_erf, gelu_tanh, layer_norm, rms_norm, rope_cos_sin, rope_inv_freq, silu)

__all__ = ["BACKWARD_WEIGHTS", "MLP_KINDS", "backward_supported", "block_backward", "OracleState", "apply_rope", "attention_row", "block_forward", "block_forward_rows",
           "block_step", "gelu_erf", "gelu_tanh", "layer_norm", "rms_norm", "rope_cos_sin", "rope_inv_freq",
           "silu"]
