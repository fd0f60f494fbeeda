"""Float64 CPU oracle of the Liger Attention layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. It shares no code with the GPU library.
"""
from .liger_ref import (  # noqa: F401
    SCALAR_MEAN,
    VECTOR_AVGPOOL4,
    decode_step,
    full_attention,
    full_attention_rows,
    gate,
    pool_scalar_mean,
    pool_vector_avg4,
    prefill,
    prefill_backward,
    prefill_continue,
    ring_fill,
    sigmoid,
    softmax,
)
