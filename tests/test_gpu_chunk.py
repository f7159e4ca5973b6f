"""Chunked prefill on the GPU against the fp64 oracle.

A chunk of n tokens at positions p0..p0+n-1 continues a sequence whose first
p0 positions sit in the layer's cache; each sequence of a batch may have its
own p0. Its output must equal the plain prefill
definition of the whole sequence at the chunk's rows (the oracle evaluates
exactly those rows), and afterwards the cache must hold what kv_append of the
whole sequence leaves (bit-exact). Chunks with n = 4 are the multi-token
decode step (one token plus three drafts, causal among themselves). At the
benchmark's sizes (a 2048-token chunk over 30720 cached tokens, the verify
step over the batched decode's caches) sampled tokens are compared with
one-token decodes of the oracle over the same history.
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth, workloads
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
    # every sequence at its own position: a 1 + 3 verify step over full caches
    # and over rings, ragged chunks over a full cache with partial rotary, a
    # ring with one sequence still inside its first window, and fp32
    (LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5), hgqa.BF16, [1000, 3, 2500, 777], 4),
    (LayerShape(SLIDING, 512, 96, 8, 128, 1e4, 1.0), hgqa.BF16, [1300, 20, 600], 4),
    (LayerShape(FULL, 0, 16, 2, 128, 5e6, 0.5), hgqa.BF16, [0, 513, 64], 300),
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), hgqa.BF16, [10, 200], 90),
    (LayerShape(FULL, 0, 8, 1, 128, 0.0, 1.0), hgqa.BF16, [5, 4000], 2100),
    (LayerShape(FULL, 0, 6, 2, 128, 5e6, 0.5), hgqa.FP32, [50, 0, 7], 20),
]
B = 2


def _cap(shape, total):
    return shape.window if shape.layer_type == SLIDING else total + 5


def _chunk_case(shape, dtype, p0, n, idx):
    """p0: the start position of every sequence, or a list with one per sequence."""
    starts = list(p0) if isinstance(p0, (list, tuple)) else [p0] * B
    nb = len(starts)
    total = max(starts) + n
    what = f"chunk[{idx}] {shape} p0 {p0} n {n}"
    print(what, flush=True)
    q, k, v, g = prefill_inputs(shape, nb, total, dtype, (0, 300 + idx, 0))
    L = hgqa.layer_from_shape(shape, dtype)
    cap = _cap(shape, total)
    kc = torch.zeros(nb, shape.num_kv_heads, cap, shape.head_dim, dtype=tdtype(dtype), device=DEV)
    vc = torch.zeros_like(kc)
    zero = torch.zeros(1, dtype=torch.int32, device=DEV)
    for b, s0 in enumerate(starts):
        if s0 > 0:
            hgqa.kv_append(L, zero, s0, k[b:b + 1, :s0].contiguous().to(DEV),
                           v[b:b + 1, :s0].contiguous().to(DEV), kc[b:b + 1], vc[b:b + 1])
    pick = lambda t: torch.stack([t[b, s0:s0 + n] for b, s0 in enumerate(starts)]).contiguous()
    sp = torch.tensor(starts, dtype=torch.int32, device=DEV)
    out = hgqa.attn_prefill_chunk(L, sp, pick(q).to(DEV), pick(k).to(DEV), pick(v).to(DEV),
                                  pick(g).to(DEV), kc, vc, max_end_pos=total)
    # the cache each whole sequence leaves through kv_append
    kw = torch.zeros_like(kc)
    vw = torch.zeros_like(vc)
    for b, s0 in enumerate(starts):
        hgqa.kv_append(L, zero, s0 + n, k[b:b + 1, :s0 + n].contiguous().to(DEV),
                       v[b:b + 1, :s0 + n].contiguous().to(DEV), kw[b:b + 1], vw[b:b + 1])
    torch.cuda.synchronize()
    assert torch.equal(kc, kw) and torch.equal(vc, vw), f"{what}: cache differs from kv_append"

    rows = [(b, t, h) for b, s0 in enumerate(starts) for t in range(s0, s0 + n)
            for h in range(shape.num_q_heads)]
    ref = oracle.prefill_rows(f64(q), f64(k), f64(v), f64(g), spec(shape), rows)
    got = f64(out).reshape(nb, n, shape.num_q_heads, shape.head_dim)
    got = np.stack([got[b, t - starts[b], h] for (b, t, h) in rows])
    assert_close(got, ref, dtype, what)


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_chunk_matches_whole_sequence_prefill(idx):
    require_gpu()
    shape, dtype, p0, n = CASES[idx]
    _chunk_case(shape, dtype, p0, n, idx)


# Both workgroup shapes of the bf16 kernel (4 and 8 waves) on chunks over a
# ring and over a full cache, whatever the launcher would pick.
WAVE_CASES = [1, 3, 6, 13, 15]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("idx", WAVE_CASES)
def test_chunk_both_workgroup_shapes(idx, waves, tuning):
    require_gpu()
    tuning(hgqa.TUNE_PREFILL_WAVES, waves)
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


# Key splits: each case again with the tiles per split forced small, so the
# splits, the empty trailing splits of the shorter sequences and the merge
# all run; results must match the oracle as without splits.
SPLIT_CASES = [0, 3, 6, 11, 13, 14]


@pytest.mark.parametrize("split_tiles", [1, 3, 7])
@pytest.mark.parametrize("idx", SPLIT_CASES)
def test_chunk_key_splits(idx, split_tiles, tuning):
    require_gpu()
    shape, dtype, p0, n = CASES[idx]
    if dtype != hgqa.BF16:
        pytest.skip("key splits are a bf16 path")
    tuning(hgqa.TUNE_CHUNK_SPLIT_TILES, split_tiles)
    _chunk_case(shape, dtype, p0, n, idx)


def test_verify_step_automatic_splits():
    """A 1 + 3 verify step of three sequences over a full cache of up to 9000
    keys: 24 blocks, so the automatic plan splits the keys."""
    require_gpu()
    shape = LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    base = hgqa.attn_prefill_chunk_workspace_bytes(L, 3, 4, 4)  # no split for 4 keys
    assert hgqa.attn_prefill_chunk_workspace_bytes(L, 3, 4, 9000) > base
    _chunk_case(shape, hgqa.BF16, [8996, 5000, 123], 4, 40)


# ------------------------------------------------------------ full size
#
# The benchmark's chunk and verify legs at their own sizes. The caches hold
# seeded random (already rotated) keys, so the reference for a new token is a
# one-token decode at its position over the oracle's cache: the slots below
# the chunk's start as given, then the oracle's own append of the chunk.

def _oracle_cache(kc, vc, b, p0, k_new, v_new, shape):
    """Sequence b's cache for the oracle: slots [0, p0) copied from the GPU
    cache (inputs the call leaves alone), the new tokens appended by the
    oracle at p0.."""
    n = k_new.shape[1]
    okc = np.zeros((1, kc.shape[1], p0 + n, kc.shape[3]))
    ovc = np.zeros_like(okc)
    okc[:, :, :p0] = f64(kc[b:b + 1, :, :p0])
    ovc[:, :, :p0] = f64(vc[b:b + 1, :, :p0])
    return oracle.kv_append(okc, ovc, f64(k_new[b:b + 1]), f64(v_new[b:b + 1]), [p0], spec(shape))


def test_chunked_prefill_full_size():
    """2048 new tokens at positions 30720.. of the Step full layer (64 Q / 8 KV,
    base 5e6, rotary 0.5), the benchmark's chunk: sampled tokens (the first
    and last, both sides of 64-key tile edges, seeded others), every head."""
    require_gpu()
    shape = workloads.STEP_FULL.layers[0]
    Hq, Hkv, D = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    p0, n = 30720, 2048
    key = (0, 970, 0)
    kc = torch.empty(1, Hkv, p0 + n, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    synth.device_normal_(kc, key + (synth.CACHE_K,))
    synth.device_normal_(vc, key + (synth.CACHE_V,))
    q = synth.host_normal((1, n, Hq, D), key + (synth.Q,))
    k = synth.host_normal((1, n, Hkv, D), key + (synth.K,))
    v = synth.host_normal((1, n, Hkv, D), key + (synth.V,))
    g = synth.host_normal((1, n, Hq), key + (synth.GATE,))
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    out = hgqa.attn_prefill_chunk(L, p0, q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV), kc, vc)
    torch.cuda.synchronize()
    okc, ovc = _oracle_cache(kc, vc, 0, p0, k, v, shape)
    rng = np.random.default_rng(11)
    rows = sorted({0, 1, 63, 64, 65, 1023, 1024, n - 2, n - 1} |
                  {int(t) for t in rng.integers(0, n, 7)})
    got = np.stack([f64(out[0, t]) for t in rows])
    ref = np.stack([oracle.decode(f64(q[:, t]), f64(g[:, t]), okc, ovc, [p0 + t + 1],
                                  spec(shape))[0] for t in rows])
    assert_close(got, ref, hgqa.BF16, f"chunk of {n} over {p0}: tokens {rows}")


def test_verify_step_full_size():
    """The benchmark's verify step: 64 sequences over the batched decode's
    full-layer caches (lengths U[65536, 131072]), 4 new tokens each (1 + 3
    drafts) ending at position L_b - 1. The shortest and the longest sequence
    and four seeded others, every token and head, one sequence at a time so
    host memory stays bounded."""
    require_gpu()
    wl = workloads.BATCHED_DECODE
    shape = wl.layers[0]
    B, Hq, Hkv, D, n = wl.batch, shape.num_q_heads, shape.num_kv_heads, shape.head_dim, 4
    lens = synth.host_uniform_int(wl.min_seq_len, wl.seq_len, B, (0, wl.wid, 0, synth.SEQ_LENS))
    key = (0, 971, 0)
    kc = torch.empty(B, Hkv, wl.seq_len, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(B):
        synth.device_normal_(kc[b], key + (synth.CACHE_K, b))
        synth.device_normal_(vc[b], key + (synth.CACHE_V, b))
    q = synth.host_normal((B, n, Hq, D), key + (synth.Q,))
    g = synth.host_normal((B, n, Hq), key + (synth.GATE,))
    kn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_K,))
    vn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_V,))
    starts = lens - n
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    out = hgqa.attn_prefill_chunk(L, torch.tensor(starts, dtype=torch.int32, device=DEV),
                                  q.to(DEV), kn.to(DEV), vn.to(DEV), g.to(DEV), kc, vc,
                                  max_end_pos=int(lens.max()))
    torch.cuda.synchronize()
    order = np.argsort(lens)
    rng = np.random.default_rng(12)
    picks = sorted({int(order[0]), int(order[-1])} |
                   {int(b) for b in rng.permutation(order[1:-1])[:4]})
    got, ref = [], []
    for b in picks:
        p0 = int(starts[b])
        okc, ovc = _oracle_cache(kc, vc, b, p0, kn, vn, shape)
        for t in range(n):
            ref.append(oracle.decode(f64(q[b:b + 1, t]), f64(g[b:b + 1, t]), okc, ovc,
                                     [p0 + t + 1], spec(shape))[0])
            got.append(f64(out[b, t]))
        del okc, ovc
    assert_close(np.stack(got), np.stack(ref), hgqa.BF16,
                 f"verify step over lengths {int(lens.min())}..{int(lens.max())}: sequences {picks}")
