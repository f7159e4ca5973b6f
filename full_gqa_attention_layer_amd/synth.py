"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and nothing else: it holds none of the
attention arithmetic. Every tensor is keyed by (seed, workload id, layer id,
tensor id) so each draw is reproducible on its own.

Tensor ids: 0 Q, 1 K, 2 V, 3 gate logits, 4 sequence lengths, 5 new K,
6 new V, 7 cached K, 8 cached V.

Host draws use NumPy's PCG64 seeded by SeedSequence(key), as float32 standard
normals, then round to bfloat16 (ties to even) when a bf16 tensor is asked
for. Device draws (only for multi-GB caches) use torch's Philox generator on
the GPU, seeded from the same SeedSequence; any CPU check of such a tensor
copies the drawn bits back rather than drawing again.
"""
from __future__ import annotations

import numpy as np
import torch

Q, K, V, GATE, SEQ_LENS, NEW_K, NEW_V, CACHE_K, CACHE_V = range(9)


def _seed_sequence(key):
    return np.random.SeedSequence([int(x) for x in key])


def host_normal(shape, key, dtype=torch.bfloat16) -> torch.Tensor:
    """Standard normals drawn on the host, returned as a CPU tensor of dtype."""
    gen = np.random.Generator(np.random.PCG64(_seed_sequence(key)))
    x = gen.standard_normal(size=tuple(shape), dtype=np.float32)
    return torch.from_numpy(x).to(dtype)


def device_seed(key) -> int:
    """A 63-bit torch generator seed derived from the key."""
    a, b = _seed_sequence(key).generate_state(2, dtype=np.uint32)
    return ((int(a) << 32) | int(b)) & ((1 << 63) - 1)


DEVICE_CHUNK = 1 << 28  # elements drawn per generator call


def device_normal_(out: torch.Tensor, key) -> torch.Tensor:
    """Fill a contiguous device tensor in place with standard normals from
    torch's Philox generator, drawn in float32 and rounded to out.dtype. The
    flattened tensor is drawn in chunks of DEVICE_CHUNK elements, chunk i
    keyed by (key..., i)."""
    assert out.is_cuda and out.is_contiguous()
    flat = out.view(-1)
    for i, lo in enumerate(range(0, flat.numel(), DEVICE_CHUNK)):
        hi = min(flat.numel(), lo + DEVICE_CHUNK)
        g = torch.Generator(device=out.device)
        g.manual_seed(device_seed(tuple(key) + (i,)))
        flat[lo:hi].copy_(torch.randn(hi - lo, generator=g, device=out.device,
                                      dtype=torch.float32))
    return out


def host_uniform_int(low: int, high_inclusive: int, size: int, key) -> np.ndarray:
    """Integers uniform on [low, high_inclusive], drawn on the host."""
    gen = np.random.Generator(np.random.PCG64(_seed_sequence(key)))
    return gen.integers(low, high_inclusive + 1, size=size, dtype=np.int64)
