"""Hybrid sliding/full grouped-query attention for MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI declared in
include/hgqa.h (library libhgqa.so, built in this package directory). The
Python binding `full_gqa_attention_layer_amd.hgqa` only marshals tensors,
pointers and streams; it loads the library on first use.
"""
from . import accounting, synth, workloads  # noqa: F401
