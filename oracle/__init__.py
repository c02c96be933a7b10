"""CPU oracle for the Llama-2/3 decoder forward pass.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition that the HIP library is checked against.  Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it; the product path
never calls it, and it shares no code with the HIP library or its binding.

Every function is pinned by a CPU test to something other than itself (closed
forms, invariants, brute force on tiny inputs, library routines), see
``tests/test_oracle_pins.py``.  The RoPE pairing convention (interleaved pairs)
is a reading of the pages and is documented as such; no other part is unpinned.
"""
from .llama import (  # noqa: F401
    OracleConfig,
    OracleModel,
    apply_rope,
    causal_gqa_attention,
    decoder_layer,
    feed_forward,
    greedy_argmax,
    rms_norm,
    rope_cos_sin,
    rope_inv_freq,
    silu,
    softmax,
)
