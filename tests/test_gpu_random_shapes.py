"""Seeded random layer shapes on the GPU against the fp64 oracle.

Each case draws a layer (sliding or full, window, G, KV heads, head_dim, RoPE
base and rotary dims, softmax scale), a batch and lengths from its own seed,
and compares the HIP path with the oracle on every output element: prefill,
cache appends followed by decode, and chunked prefill over a cache. The draws
cover combinations the hand-picked cases do not, such as odd G, three KV
heads, windows of every size against ragged lengths, and both RoPE paths of
the bf16 kernel (r/2 a multiple of 16, or an odd multiple of 8).
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth
from full_gqa_attention_layer_amd.workloads import FULL, SLIDING, LayerShape
from tests.gpu_helpers import DEV, assert_close, f64, prefill_inputs, require_gpu, spec
from tests.test_gpu_chunk import _chunk_case
from tests.test_gpu_decode import build_caches

pytestmark = pytest.mark.gpu


def random_shape(rng, dtype, max_window=300):
    D = int(rng.choice([64, 128]))
    hkv = int(rng.choice([1, 2, 3]))
    G = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16]))
    sliding = bool(rng.random() < 0.5)
    window = int(rng.integers(1, max_window)) if sliding else 0
    theta = float(rng.choice([0.0, 1e4, 5e5, 5e6]))
    # rotary dims: bf16 layers take multiples of 16, fp32 layers any even count
    step = 16 if dtype == hgqa.BF16 else 2
    r = int(rng.choice(np.arange(step, D + 1, step)))
    scale = float(rng.choice([0.0, 0.0, 0.05]))
    return LayerShape(SLIDING if sliding else FULL, window, G * hkv, hkv, D, theta, r / D, scale)


def case_rng(kind, idx):
    return np.random.default_rng([7, kind, idx])


N_PREFILL, N_DECODE, N_CHUNK = 16, 10, 10


@pytest.mark.parametrize("idx", range(N_PREFILL))
def test_random_prefill(idx):
    require_gpu()
    rng = case_rng(0, idx)
    dtype = hgqa.FP32 if idx % 5 == 4 else hgqa.BF16
    shape = random_shape(rng, dtype)
    B, T = int(rng.integers(1, 3)), int(rng.integers(1, 350))
    what = f"random prefill[{idx}] {shape} B{B} T{T} {'fp32' if dtype == hgqa.FP32 else 'bf16'}"
    print(what, flush=True)
    q, k, v, g = prefill_inputs(shape, B, T, dtype, (0, 600 + idx, 0))
    L = hgqa.layer_from_shape(shape, dtype)
    out = hgqa.attn_prefill(L, q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
    assert_close(out, ref, dtype, what)


@pytest.mark.parametrize("idx", range(N_DECODE))
def test_random_append_then_decode(idx):
    require_gpu()
    rng = case_rng(1, idx)
    dtype = hgqa.FP32 if idx % 5 == 4 else hgqa.BF16
    shape = random_shape(rng, dtype, max_window=700)
    lens = [int(x) for x in rng.integers(1, 3000, size=int(rng.integers(1, 4)))]
    what = f"random decode[{idx}] {shape} lengths {lens}"
    print(what, flush=True)
    key = (0, 650 + idx, 0)
    kc, vc, okc, ovc, _ = build_caches(shape, dtype, lens, key)
    B = len(lens)
    td = torch.bfloat16 if dtype == hgqa.BF16 else torch.float32
    q = synth.host_normal((B, shape.num_q_heads, shape.head_dim), key + (synth.Q,), td)
    g = synth.host_normal((B, shape.num_q_heads), key + (synth.GATE,), td)
    L = hgqa.layer_from_shape(shape, dtype)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = hgqa.attn_decode(L, q.to(DEV), g.to(DEV), kc, vc, seq, max(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(g), okc, ovc, lens, spec(shape))
    assert_close(out, ref, dtype, what)


@pytest.mark.parametrize("idx", range(N_CHUNK))
def test_random_chunk(idx):
    require_gpu()
    rng = case_rng(2, idx)
    dtype = hgqa.FP32 if idx % 5 == 4 else hgqa.BF16
    shape = random_shape(rng, dtype)
    p0, n = int(rng.integers(0, 600)), int(rng.integers(1, 150))
    _chunk_case(shape, dtype, p0, n, 500 + idx)
