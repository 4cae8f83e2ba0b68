"""CPU oracle for the decoder-only transformer prefill (test infrastructure only).

This package is the reference that the HIP library is checked against. It is NOT
part of the product: only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import it. The library never calls it and must
fail loudly rather than fall back to it.

Every operation follows the plain definition given on the source pages, written
out in numpy with float64 arithmetic on float32 tensors and one rounding to
float32 at each operation's output (the "float64-accumulated f32" reference of
the metalgemm page, Theorem 1 proof). Matrix products use numpy's matmul as a
library primitive; nothing is blocked, fused or reordered beyond that.

Parity pins: every function here is pinned by closed forms, invariants or brute
force in tests/test_oracle_pins.py. The whole forward's values are pinned in
tests/test_oracle_vs_transformers.py against an independent implementation of the
same published architectures (the transformers library's llama, qwen3, gemma3,
phi3 and qwen3moe models, built locally in float64 with these weights), every
hidden slot and the logits within 2e-6 of scale. The pages' own printed end-to-end
numbers come from trained weights that do not exist here and stay unreproduced.
"""
from .forward import (  # noqa: F401
    argmax,
    attention,
    attention_probs,
    embed,
    embed_scale,
    forward,
    gated_ffn,
    gelu_tanh,
    gemm,
    greedy,
    moe_ffn,
    moe_route,
    rmsnorm,
    round_bf16,
    rope,
    rope_frequencies,
    rotate,
    silu,
    softcap,
    swiglu,
)

import sys as _sys

# the module itself (its name is shadowed by the forward() function above), for tests
# that reach its diagnostic helpers
forward_module = _sys.modules[__name__ + ".forward"]
