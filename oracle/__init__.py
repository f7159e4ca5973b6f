"""fp64 CPU oracle for the hybrid GQA attention layer (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package; the GPU library never does.
"""
from .attention import (  # noqa: F401
    FULL,
    SLIDING,
    LayerSpec,
    cached_positions,
    decode,
    kv_append,
    llama3_frequencies,
    prefill,
    prefill_rows,
    rope,
    round_bf16,
    sigmoid,
    visible,
)
