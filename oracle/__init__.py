"""CPU oracle of the prefill forward -- test infrastructure only.

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of `bench.py` may
import this package. The product path (the HIP library and its Python binding) never
imports, calls or falls back to it.
"""
from .oracle import (  # noqa: F401
    layer_norm, rms_norm, rope_frequencies, apply_rope, alibi_slopes, silu, gelu_tanh,
    causal_attention, split_fused_qkv, attention, mlp, block, embed, forward, next_token_probs,
    quantize_q8_0, dequantize_q8_0, q8_0_weights, Q8_BLOCK, Q8_MATRICES,
)
