"""Hybrid sliding/full grouped-query attention for MI355X (gfx950).

The compute runs in hand-written HIP kernels behind the C ABI declared in
include/hgqa.h (library libhgqa.so, built in this package directory). The
Python side in `hgqa` only marshals tensors, pointers and streams.
"""
from . import accounting, synth, workloads  # noqa: F401


def __getattr__(name):
    # The binding loads the shared library; import it only when asked for so
    # that host-only helpers work without a built library.
    if name == "hgqa":
        from . import hgqa
        return hgqa
    raise AttributeError(name)
