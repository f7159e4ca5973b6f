"""Chunked prefill on the GPU against the fp64 oracle.

A chunk of n tokens at positions p0..p0+n-1 continues a sequence whose first
p0 positions sit in the layer's cache. Its output must equal the plain prefill
definition of the whole sequence at the chunk's rows (the oracle evaluates
exactly those rows), and afterwards the cache must hold what kv_append of the
whole sequence leaves (bit-exact). Chunks with n = 4 are the multi-token
decode step (one token plus three drafts, causal among themselves).
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth
from full_gqa_attention_layer_amd.workloads import FULL, SLIDING, LayerShape
from tests.gpu_helpers import DEV, assert_close, f64, prefill_inputs, require_gpu, spec, tdtype

pytestmark = pytest.mark.gpu

CASES = [
    # shape, dtype, p0, n
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), hgqa.BF16, 100, 50),    # ring, chunk < W
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), hgqa.BF16, 30, 90),     # p0 < W < n
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), hgqa.BF16, 0, 70),      # empty cache
    (LayerShape(FULL, 0, 8, 1, 128, 5e6, 0.5), hgqa.BF16, 300, 77),
    (LayerShape(FULL, 0, 12, 1, 128, 0.0, 1.0), hgqa.BF16, 1000, 4),       # 1 + 3 drafts
    (LayerShape(SLIDING, 512, 96, 8, 128, 1e4, 1.0), hgqa.BF16, 700, 4),   # Step sliding, drafts
    (LayerShape(SLIDING, 2048, 32, 2, 128, 5e5, 1.0), hgqa.BF16, 2500, 129),
    (LayerShape(FULL, 0, 8, 2, 64, 1e4, 0.25), hgqa.BF16, 129, 200),
    (LayerShape(SLIDING, 64, 4, 1, 64, 1e4, 1.0), hgqa.FP32, 70, 40),
    (LayerShape(FULL, 0, 6, 2, 128, 5e6, 0.5), hgqa.FP32, 50, 20),
    (LayerShape(FULL, 0, 8, 1, 128, 1e4, 1.0, 0.0, (2.0, 1.0, 4.0, 256)), hgqa.BF16, 300, 100),
]
B = 2


def _cap(shape, total):
    return shape.window if shape.layer_type == SLIDING else total + 5


def _chunk_case(shape, dtype, p0, n, idx):
    total = p0 + n
    what = f"chunk[{idx}] {shape} p0 {p0} n {n}"
    print(what, flush=True)
    q, k, v, g = prefill_inputs(shape, B, total, dtype, (0, 300 + idx, 0))
    L = hgqa.layer_from_shape(shape, dtype)
    cap = _cap(shape, total)
    kc = torch.zeros(B, shape.num_kv_heads, cap, shape.head_dim, dtype=tdtype(dtype), device=DEV)
    vc = torch.zeros_like(kc)
    zeros = torch.zeros(B, dtype=torch.int32, device=DEV)
    if p0 > 0:
        hgqa.kv_append(L, zeros, p0, k[:, :p0].contiguous().to(DEV), v[:, :p0].contiguous().to(DEV),
                       kc, vc)
    out = hgqa.attn_prefill_chunk(L, p0, q[:, p0:].contiguous().to(DEV),
                                  k[:, p0:].contiguous().to(DEV), v[:, p0:].contiguous().to(DEV),
                                  g[:, p0:].contiguous().to(DEV), kc, vc)
    # the cache the whole sequence leaves through kv_append
    kw = torch.zeros_like(kc)
    vw = torch.zeros_like(vc)
    hgqa.kv_append(L, zeros, total, k.to(DEV), v.to(DEV), kw, vw)
    torch.cuda.synchronize()
    assert torch.equal(kc, kw) and torch.equal(vc, vw), f"{what}: cache differs from kv_append"

    rows = [(b, t, h) for b in range(B) for t in range(p0, total) for h in range(shape.num_q_heads)]
    ref = oracle.prefill_rows(f64(q), f64(k), f64(v), f64(g), spec(shape), rows)
    got = f64(out).reshape(B, n, shape.num_q_heads, shape.head_dim)
    got = np.stack([got[b, t - p0, h] for (b, t, h) in rows])
    assert_close(got, ref, dtype, what)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_chunk_matches_whole_sequence_prefill(idx):
    require_gpu()
    shape, dtype, p0, n = CASES[idx]
    _chunk_case(shape, dtype, p0, n, idx)


# Both workgroup shapes of the bf16 kernel (4 and 8 waves) on chunks over a
# ring and over a full cache, whatever the launcher would pick.
WAVE_CASES = [1, 3, 6]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("idx", WAVE_CASES)
def test_chunk_both_workgroup_shapes(idx, waves, monkeypatch):
    require_gpu()
    monkeypatch.setenv("HGQA_PREFILL_WAVES", str(waves))
    shape, dtype, p0, n = CASES[idx]
    _chunk_case(shape, dtype, p0, n, idx)


def test_chunks_in_sequence_equal_one_prefill():
    """A prompt fed as three chunks gives the single-call prefill's output
    (same kernel arithmetic, so up to rounding order of the softmax)."""
    require_gpu()
    shape = LayerShape(SLIDING, 128, 16, 2, 128, 1e4, 1.0)
    dtype = hgqa.BF16
    T, cuts = 400, [0, 130, 260, 400]
    q, k, v, g = prefill_inputs(shape, B, T, dtype, (0, 399, 0))
    L = hgqa.layer_from_shape(shape, dtype)
    whole = hgqa.attn_prefill(L, q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV))
    kc = torch.zeros(B, shape.num_kv_heads, shape.window, shape.head_dim, dtype=torch.bfloat16,
                     device=DEV)
    vc = torch.zeros_like(kc)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        parts.append(hgqa.attn_prefill_chunk(L, a, q[:, a:b].contiguous().to(DEV),
                                             k[:, a:b].contiguous().to(DEV),
                                             v[:, a:b].contiguous().to(DEV),
                                             g[:, a:b].contiguous().to(DEV), kc, vc))
    chunked = torch.cat(parts, dim=1)
    torch.cuda.synchronize()
    err = (chunked.float() - whole.float()).abs()
    print(f"chunked vs one call: max-abs {float(err.max()):.3e}", flush=True)
    assert float(err.max()) <= 1e-2
