"""fp64 CPU oracle for cross-layer KV sharing (YOCO / YOCO++).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline
leg of the benchmark may import it; the product path never does. It shares
no code with the HIP library. Every function here is pinned by CPU tests to
closed forms, library routines or exact arithmetic (no function is left
with its parity unpinned).
"""
from .yoco_oracle import (  # noqa: F401
    LAMBDA,
    bf16_nearest,
    causal_prefill,
    compose,
    compose_backward,
    compose_kv,
    compose_magnitude,
    decode_attention,
    self_attn_decode,
    softmax_attend,
    to_f64,
)
