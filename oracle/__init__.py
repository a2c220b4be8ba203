"""CPU oracle for the decode step. TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the bench's CPU-baseline leg may import this package.
The HIP path never calls it and shares no code with it.

Pinned functions (each checked against something other than itself in tests/test_oracle_pins.py):
rmsnorm, apply_rope / rope_cos_sin, softmax, silu, attend, argmax_lowest, float_to_bf16,
bf16_to_float, Decoder.step (brute-force full recompute, closed forms, GQA/int8/tied identities,
an independent torch forward). The full-size end-to-end logits are "parity unpinned" by any
closed form: the pinned pieces plus brute force on small shapes are what pin them.
"""
from .decoder import (Decoder, apply_rope, argmax_lowest, attend, bf16_to_float, dequant_int4,
                      float_to_bf16, unpack_int4,
                      rmsnorm, rope_cos_sin, silu, softmax, top2_margin)

__all__ = ["Decoder", "apply_rope", "argmax_lowest", "attend", "bf16_to_float", "dequant_int4",
           "float_to_bf16", "unpack_int4",
           "rmsnorm", "rope_cos_sin", "silu", "softmax", "top2_margin"]
