"""kv_append and decode parity: the HIP path through the C ABI against the
fp64 oracle. Cache indexing is checked bit-exactly (slot map, every V byte,
K bytes when nothing rotates); rotated K is checked to one bf16 ulp of the
oracle's exact rotation; decode outputs to the bf16/fp32 bars."""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth, workloads
from full_gqa_attention_layer_amd.workloads import FULL, SLIDING, LayerShape
from tests.gpu_helpers import DEV, assert_close, f64, require_gpu, spec, tdtype

pytestmark = pytest.mark.gpu


def _kv(shape, B, n, dtype, key):
    dt = tdtype(dtype)
    k = synth.host_normal((B, n, shape.num_kv_heads, shape.head_dim), key + (synth.NEW_K,), dt)
    v = synth.host_normal((B, n, shape.num_kv_heads, shape.head_dim), key + (synth.NEW_V,), dt)
    return k, v


def _cap(shape, lens):
    return shape.window if shape.layer_type == SLIDING else max(lens) + 3


def build_caches(shape, dtype, lens, key):
    """History of len(lens) sequences appended position by position range on
    the GPU (one kv_append per sequence, as a serving engine would after its
    prefill) and by the oracle. Returns GPU caches, oracle caches, raw K/V."""
    B = len(lens)
    cap = _cap(shape, lens)
    n = max(lens)
    k, v = _kv(shape, B, n, dtype, key)
    L = hgqa.layer_from_shape(shape, dtype)
    dt = tdtype(dtype)
    kc = torch.zeros(B, shape.num_kv_heads, cap, shape.head_dim, dtype=dt, device=DEV)
    vc = torch.zeros_like(kc)
    okc = np.zeros(tuple(kc.shape))
    ovc = np.zeros(tuple(kc.shape))
    for b, Lb in enumerate(lens):
        kb = k[b:b + 1, :Lb].contiguous().to(DEV)
        vb = v[b:b + 1, :Lb].contiguous().to(DEV)
        hgqa.kv_append(L, torch.zeros(1, dtype=torch.int32, device=DEV), Lb, kb, vb,
                       kc[b:b + 1], vc[b:b + 1])
        okb, ovb = oracle.kv_append(okc[b:b + 1], ovc[b:b + 1], f64(k[b:b + 1, :Lb]),
                                    f64(v[b:b + 1, :Lb]), [0], spec(shape))
        okc[b:b + 1], ovc[b:b + 1] = okb, ovb
    torch.cuda.synchronize()
    return kc, vc, okc, ovc, k


def _pair_magnitude(k, shape):
    """|x_d| + |x_partner(d)| of each raw key element (partner = the other
    element of its RoPE pair; itself for dims that do not rotate)."""
    a = np.abs(f64(k))
    r = int(round(shape.rotary_fraction * shape.head_dim)) if shape.rope_theta else 0
    sw = a.copy()
    if r:
        h = r // 2
        sw[..., :h], sw[..., h:r] = a[..., h:r], a[..., :h]
    return a + sw


def check_cache(kc, vc, okc, ovc, shape, dtype, k_raw=None, start=None):
    """V bit-exact; K bit-exact without rotation. A rotated K element may
    differ from the exactly rotated, rounded value by one ulp of its rounding
    plus the fp32 rotation error, at most 2^-20 (|x_d| + |x_partner|)."""
    got_v = f64(vc)
    np.testing.assert_array_equal(got_v, ovc)
    got_k = f64(kc)
    if shape.rope_theta == 0:
        want = okc if dtype == hgqa.FP32 else oracle.round_bf16(okc)
        np.testing.assert_array_equal(got_k, want)
        return
    zero = np.zeros(okc.shape)
    flat = oracle.LayerSpec(spec(shape).layer_type, spec(shape).window, shape.num_q_heads,
                            shape.num_kv_heads, shape.head_dim, 0.0)
    # the same slot map applied to the magnitudes (base 0: nothing rotates)
    mag, _ = oracle.kv_append(zero, zero, _pair_magnitude(k_raw, shape),
                              np.zeros(tuple(k_raw.shape)), start, flat)
    fp32_err = np.ldexp(mag, -20)
    if dtype == hgqa.FP32:
        diff = np.abs(got_k - okc)
        assert np.all(diff <= fp32_err + 1e-30), float((diff - fp32_err).max())
        return
    want = oracle.round_bf16(okc)
    ulp = np.ldexp(1.0, np.frexp(np.abs(want))[1] - 8)
    diff = np.abs(got_k - want)
    assert np.all(diff <= ulp + fp32_err), float((diff / ulp).max())
    print(f"rotated K: {(diff > 0).sum()} of {diff.size} values differ from the rounded exact "
          f"rotation, max {float((diff / ulp).max()):.2f} ulp", flush=True)


def check_cache_per_sequence(kc, vc, okc, ovc, shape, dtype, k_raw, lens):
    for b, Lb in enumerate(lens):
        check_cache(kc[b:b + 1], vc[b:b + 1], okc[b:b + 1], ovc[b:b + 1], shape, dtype,
                    k_raw[b:b + 1, :Lb], [0])


SMALL = [
    # shape, dtype, lengths
    (LayerShape(FULL, 0, 8, 1, 128, 5e6, 0.5), hgqa.BF16, [1, 37, 300, 513]),
    (LayerShape(SLIDING, 64, 16, 2, 128, 1e4, 1.0), hgqa.BF16, [1, 63, 64, 65, 200]),
    (LayerShape(SLIDING, 512, 64, 8, 128, 1e4, 1.0), hgqa.BF16, [100, 511, 512, 1300]),
    (LayerShape(FULL, 0, 12, 1, 128, 0.0, 1.0), hgqa.BF16, [5, 1000]),
    (LayerShape(FULL, 0, 32, 2, 128, 5e5, 1.0), hgqa.BF16, [2048, 3000]),
    (LayerShape(SLIDING, 7, 4, 4, 64, 1e4, 1.0), hgqa.BF16, [3, 7, 30]),
    (LayerShape(FULL, 0, 8, 2, 64, 1e4, 0.25), hgqa.BF16, [1, 129, 4000]),
    (LayerShape(SLIDING, 64, 4, 1, 64, 1e4, 1.0), hgqa.FP32, [10, 64, 100]),
    (LayerShape(FULL, 0, 6, 2, 128, 5e6, 0.5), hgqa.FP32, [1, 77, 300]),
    # the pages' other layers: Step's 96-head sliding layers (G = 12, W = 512) and
    # Muse's sliding (G = 16, W = 2048, base 5e5) and full (base 0) layers
    (LayerShape(SLIDING, 512, 96, 8, 128, 1e4, 1.0), hgqa.BF16, [100, 512, 2000]),
    (LayerShape(SLIDING, 2048, 32, 2, 128, 5e5, 1.0), hgqa.BF16, [700, 2048, 5000]),
    (LayerShape(FULL, 0, 32, 2, 128, 0.0, 1.0), hgqa.BF16, [3000, 9000]),
    # llama3 frequency scaling (full layers), short original context
    (LayerShape(FULL, 0, 8, 2, 128, 1e4, 1.0, 0.0, (2.0, 1.0, 4.0, 256)), hgqa.BF16, [300, 700]),
]


def test_decode_far_position_with_default_scaling():
    """The Step full layer with its long-context scaling (factor 2.0, other
    parameters at the library's defaults): keys appended at positions up to
    199999, past the original 131072-position context, then a decode there."""
    require_gpu()
    shape = LayerShape(FULL, 0, 8, 1, 128, 5e6, 0.5, 0.0, (2.0,))
    dtype = hgqa.BF16
    Lq = 200000
    key = (0, 290, 0)
    k, v = _kv(shape, 1, Lq, dtype, key)
    L = hgqa.layer_from_shape(shape, dtype)
    kc = torch.zeros(1, 1, Lq, 128, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    hgqa.kv_append(L, torch.zeros(1, dtype=torch.int32, device=DEV), Lq, k.to(DEV), v.to(DEV),
                   kc, vc)
    # the oracle's cache: slot p holds rope(k_p, p) with the scaled frequencies
    sp = spec(shape)
    pos = np.arange(Lq, dtype=np.float64)
    okc = oracle.rope(f64(k)[0, :, 0], pos, 5e6, 64, sp.frequency_scaling)[None, None]
    ovc = f64(v)[0, :, 0][None, None]
    check_cache_per_sequence(kc, vc, okc, ovc, shape, dtype, k, [Lq])
    unscaled = oracle.rope(f64(k)[0, -1000:, 0], pos[-1000:], 5e6, 64)
    assert np.abs(unscaled - okc[0, 0, -1000:]).max() > 0.5     # the scaling matters here
    q = synth.host_normal((1, shape.num_q_heads, shape.head_dim), key + (synth.Q,), torch.bfloat16)
    g = synth.host_normal((1, shape.num_q_heads), key + (synth.GATE,), torch.bfloat16)
    seq = torch.tensor([Lq], dtype=torch.int32)
    out = hgqa.attn_decode(L, q.to(DEV), g.to(DEV), kc, vc, seq.to(DEV), Lq)
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(g), okc, ovc, [Lq], sp)
    assert_close(out, ref, dtype, "decode at 199999 with llama3 scaling")


@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_append_then_decode(idx):
    require_gpu()
    shape, dtype, lens = SMALL[idx]
    key = (0, 200 + idx, 0)
    kc, vc, okc, ovc, k_raw = build_caches(shape, dtype, lens, key)
    check_cache_per_sequence(kc, vc, okc, ovc, shape, dtype, k_raw, lens)
    B = len(lens)
    dt = tdtype(dtype)
    q = synth.host_normal((B, shape.num_q_heads, shape.head_dim), key + (synth.Q,), dt)
    g = synth.host_normal((B, shape.num_q_heads), key + (synth.GATE,), dt)
    L = hgqa.layer_from_shape(shape, dtype)
    seq = torch.tensor(lens, dtype=torch.int32)
    out = hgqa.attn_decode(L, q.to(DEV), g.to(DEV), kc, vc, seq.to(DEV), max(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(g), okc, ovc, lens, spec(shape))
    assert_close(out, ref, dtype, f"decode[{idx}] {shape} lens {lens}")


def test_ring_append_keeps_last_W_positions_bitexact():
    """Position-tagged V rows: one call appends 3W+5 tokens from position 11;
    every slot must hold the highest position mapping to it."""
    require_gpu()
    W, Hkv, D = 16, 2, 64
    shape = LayerShape(SLIDING, W, 4, Hkv, D, 0.0, 1.0)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    start, n = 11, 3 * W + 5
    pos = torch.arange(start, start + n)
    tag = ((pos[:, None, None] * 61 + torch.arange(Hkv)[None, :, None] * 7
            + torch.arange(D)[None, None, :]) % 0x3f00).to(torch.int16)
    v_new = tag.view(torch.bfloat16)[None].contiguous()
    k_new = synth.host_normal((1, n, Hkv, D), (0, 300, 0, synth.NEW_K))
    kc = torch.zeros(1, Hkv, W, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    hgqa.kv_append(L, torch.tensor([start], dtype=torch.int32, device=DEV), start + n,
                   k_new.to(DEV), v_new.to(DEV), kc, vc)
    torch.cuda.synchronize()
    got = vc.cpu().view(torch.int16)[0]
    for slot in range(W):
        p = max(p for p in range(start, start + n) if p % W == slot)
        assert torch.equal(got[:, slot], tag[p - start]), slot
        # theta = 0: K is copied bit for bit
        assert torch.equal(kc.cpu()[0, :, slot].view(torch.int16),
                           k_new[0, p - start].view(torch.int16))


def test_full_append_slot_is_position_and_leaves_other_slots():
    require_gpu()
    shape = LayerShape(FULL, 0, 8, 2, 128, 5e6, 0.5)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    B, n, cap = 3, 5, 64
    k_new, v_new = _kv(shape, B, n, hgqa.BF16, (0, 301, 0))
    start = torch.tensor([0, 17, 59], dtype=torch.int32)
    sentinel = torch.full((B, 2, cap, 128), -3.0, dtype=torch.bfloat16)
    kc, vc = sentinel.clone().to(DEV), sentinel.clone().to(DEV)
    hgqa.kv_append(L, start.to(DEV), 64, k_new.to(DEV), v_new.to(DEV), kc, vc)
    torch.cuda.synchronize()
    okc, ovc = oracle.kv_append(f64(sentinel), f64(sentinel), f64(k_new), f64(v_new),
                                start.tolist(), spec(shape))
    check_cache(kc, vc, okc, ovc, shape, hgqa.BF16, k_new, start.tolist())


def test_out_of_range_device_lengths_and_starts_are_clamped():
    """Device-side integers the host cannot check: decode clamps each
    seq_lens[b] to [1, max_seq_len], and kv_append stores only the tokens
    whose position falls in [0, cap). So a decode with lengths 0, 10^9 and -7
    equals, bit for bit, one with 1, max_seq_len and 1; and an append that
    starts at -5 writes tokens 5.. at slots 0.. and nothing else, as an
    append of those tokens at 0 does."""
    require_gpu()
    shape = LayerShape(FULL, 0, 8, 2, 128, 5e6, 0.5)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    lens = [1, 50, 300]
    kc, vc, _, _, _ = build_caches(shape, hgqa.BF16, lens, (0, 304, 0))
    q = synth.host_normal((3, 8, 128), (0, 304, 0, synth.Q)).to(DEV)
    g = synth.host_normal((3, 8), (0, 304, 0, synth.GATE)).to(DEV)
    bad = torch.tensor([0, 10 ** 9, -7], dtype=torch.int32, device=DEV)
    good = torch.tensor([1, 300, 1], dtype=torch.int32, device=DEV)
    a = hgqa.attn_decode(L, q, g, kc, vc, bad, 300)
    b = hgqa.attn_decode(L, q, g, kc, vc, good, 300)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))

    n, cap = 10, 64
    k_new, v_new = _kv(shape, 1, n, hgqa.BF16, (0, 305, 0))
    sentinel = torch.full((1, 2, cap, 128), -3.0, dtype=torch.bfloat16, device=DEV)
    kc1, vc1 = sentinel.clone(), sentinel.clone()
    kc2, vc2 = sentinel.clone(), sentinel.clone()
    hgqa.kv_append(L, torch.tensor([-5], dtype=torch.int32, device=DEV), n, k_new.to(DEV),
                   v_new.to(DEV), kc1, vc1)
    hgqa.kv_append(L, torch.zeros(1, dtype=torch.int32, device=DEV), n - 5,
                   k_new[:, 5:].contiguous().to(DEV), v_new[:, 5:].contiguous().to(DEV), kc2, vc2)
    torch.cuda.synchronize()
    assert torch.equal(kc1.view(torch.int16), kc2.view(torch.int16))
    assert torch.equal(vc1.view(torch.int16), vc2.view(torch.int16))
    assert torch.equal(kc1[:, :, n - 5:].view(torch.int16), sentinel[:, :, n - 5:].view(torch.int16))


def test_decode_is_deterministic():
    require_gpu()
    shape = LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5)
    lens = [5000, 20000, 1]
    kc, vc, _, _, _ = build_caches(shape, hgqa.BF16, lens, (0, 302, 0))
    q = synth.host_normal((3, 64, 128), (0, 302, 0, synth.Q)).to(DEV)
    g = synth.host_normal((3, 64), (0, 302, 0, synth.GATE)).to(DEV)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    a = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
    b = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("shape,split_keys", [
    (LayerShape(FULL, 0, 16, 2, 128, 5e6, 0.5), sk) for sk in (None, 32, 128, 1024, 1 << 20)] + [
    # head_dim 64: two merge blocks of 32 dims per head
    (LayerShape(FULL, 0, 8, 2, 64, 1e4, 0.25), sk) for sk in (None, 32)])
def test_split_counts_agree(shape, split_keys, tuning):
    """The same decode with the keys cut into different split counts (the
    tuning override fixes the keys per split; 1 << 20 gives one split). Every
    plan matches the oracle. Against the one-split output the difference is
    bounded by the one rounding that depends on the plan: each probability is
    rounded to bf16 (relative error <= 2^-9) relative to its own split's
    running maximum, so two plans differ by at most 2 * 2^-9 * sigmoid(gate) *
    max |v| over the sequence's keys, plus one bf16 step of the output."""
    require_gpu()
    lens = [1, 100, 4000, 20000]
    kc, vc, okc, ovc, _ = build_caches(shape, hgqa.BF16, lens, (0, 303, 0))
    Hq, D = shape.num_q_heads, shape.head_dim
    q = synth.host_normal((4, Hq, D), (0, 303, 0, synth.Q)).to(DEV)
    g = synth.host_normal((4, Hq), (0, 303, 0, synth.GATE)).to(DEV)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    tuning(hgqa.TUNE_DECODE_SPLIT_KEYS, 1 << 20)
    one = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
    tuning(hgqa.TUNE_DECODE_SPLIT_KEYS, 0 if split_keys is None else split_keys)
    out = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
    torch.cuda.synchronize()
    ref = oracle.decode(f64(q), f64(g), okc, ovc, lens, spec(shape))
    assert_close(out, ref, hgqa.BF16, f"D {D} split_keys {split_keys}")
    a, b = f64(out), f64(one)
    G = shape.num_q_heads // shape.num_kv_heads
    sig = 1.0 / (1.0 + np.exp(-f64(g)))                                   # [B, Hq]
    vmax = np.stack([np.abs(ovc[i, :, :n]).max(axis=(1, 2)) for i, n in enumerate(lens)])
    bound = 2.0 ** -8 * sig * np.repeat(vmax, G, axis=1)                  # [B, Hq]
    tol = bound[:, :, None] + 2.0 ** -7 * np.abs(b) + 1e-6
    assert np.all(np.abs(a - b) <= tol), \
        f"split_keys {split_keys}: max diff {np.abs(a - b).max():.3e} from the one-split output"


# ------------------------------------------------------------ full size

@pytest.mark.parametrize("layer_index,split_keys", [(3, None), (3, 32), (0, None)])
def test_single_sequence_after_muse_prompt(layer_index, split_keys, tuning):
    """The decode step of the Muse block: one sequence, the token after a
    65536-token prompt, 32 Q / 2 KV heads. The full layer (base 0) runs in
    129 splits by default and in 2049 with 32-key splits (far more splits
    than merge threads); the W = 2048 ring layer (base 5e5) in 4. The append
    writes only slot L - 1 (or (L - 1) mod W), so the oracle's cache is the
    GPU cache's other slots plus the oracle's own append of the new token."""
    require_gpu()
    wl = workloads.MUSE_BLOCK
    shape = wl.layers[layer_index]
    Lb = wl.seq_len + 1
    Hkv, D = shape.num_kv_heads, shape.head_dim
    cap = shape.window if shape.layer_type == SLIDING else Lb
    key = (0, 960 + layer_index, 0)
    kc = torch.empty(1, Hkv, cap, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    synth.device_normal_(kc, key + (synth.CACHE_K,))
    synth.device_normal_(vc, key + (synth.CACHE_V,))
    k_new = synth.host_normal((1, 1, Hkv, D), key + (synth.NEW_K,))
    v_new = synth.host_normal((1, 1, Hkv, D), key + (synth.NEW_V,))
    q = synth.host_normal((1, shape.num_q_heads, D), key + (synth.Q,))
    g = synth.host_normal((1, shape.num_q_heads), key + (synth.GATE,))
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    if split_keys is not None:
        tuning(hgqa.TUNE_DECODE_SPLIT_KEYS, split_keys)
    hgqa.kv_append(L, torch.full((1,), Lb - 1, dtype=torch.int32, device=DEV), Lb,
                   k_new.to(DEV), v_new.to(DEV), kc, vc)
    seq = torch.full((1,), Lb, dtype=torch.int32, device=DEV)
    out = hgqa.attn_decode(L, q.to(DEV), g.to(DEV), kc, vc, seq, Lb)
    torch.cuda.synchronize()
    slot = (Lb - 1) % cap
    okc, ovc = f64(kc), f64(vc)
    okc[:, :, slot] = 0.0   # the oracle writes the new token itself
    ovc[:, :, slot] = 0.0
    okc, ovc = oracle.kv_append(okc, ovc, f64(k_new), f64(v_new), [Lb - 1], spec(shape))
    ref = oracle.decode(f64(q), f64(g), okc, ovc, [Lb], spec(shape))
    assert_close(out, ref, hgqa.BF16, f"Muse layer {layer_index} decode at {Lb}, split {split_keys}")


def _c5_state(layer_index):
    """Caches, lengths and new-token inputs of the batched decode workload."""
    wl = workloads.BATCHED_DECODE
    shape = wl.layers[layer_index]
    B, Hkv, D = wl.batch, shape.num_kv_heads, shape.head_dim
    lens = synth.host_uniform_int(wl.min_seq_len, wl.seq_len, B, (0, wl.wid, 0, synth.SEQ_LENS))
    cap = shape.window if shape.layer_type == SLIDING else wl.seq_len
    kc = torch.empty(B, Hkv, cap, D, dtype=torch.bfloat16, device=DEV)
    vc = torch.empty_like(kc)
    for b in range(B):
        synth.device_normal_(kc[b], (0, wl.wid, layer_index, synth.CACHE_K, b))
        synth.device_normal_(vc[b], (0, wl.wid, layer_index, synth.CACHE_V, b))
    key = (0, wl.wid, layer_index)
    k_new = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_K,))
    v_new = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_V,))
    q = synth.host_normal((B, shape.num_q_heads, D), key + (synth.Q,))
    g = synth.host_normal((B, shape.num_q_heads), key + (synth.GATE,))
    return shape, lens, kc, vc, k_new, v_new, q, g


@pytest.mark.parametrize("layer_index", [0, 1])
def test_batched_decode_full_size(layer_index):
    """The batched decode workload after its one-token append: every sequence
    of the ring layer, and 16 sequences of the full layer (the shortest, the
    longest and 14 seeded others). The append writes only slot L - 1 (or
    (L - 1) mod W), so the oracle's cache is the GPU cache's other slots plus
    the oracle's own append of the new token; one sequence at a time, so host
    memory stays bounded."""
    require_gpu()
    shape, lens, kc, vc, k_new, v_new, q, g = _c5_state(layer_index)
    B = len(lens)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    start = torch.tensor(lens - 1, dtype=torch.int32, device=DEV)
    hgqa.kv_append(L, start, int(lens.max()), k_new.to(DEV), v_new.to(DEV), kc, vc)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    out = hgqa.attn_decode(L, q.to(DEV), g.to(DEV), kc, vc, seq, int(lens.max()))
    torch.cuda.synchronize()
    if shape.layer_type == SLIDING:
        picks = list(range(B))
    else:
        order = np.argsort(lens)
        rng = np.random.default_rng(5)
        others = [int(b) for b in rng.permutation(order[1:-1])[:14]]
        picks = sorted({int(order[0]), int(order[-1])} | set(others))
    assert len(picks) >= 16
    got, ref = [], []
    for b in picks:
        Lb = int(lens[b])
        n = Lb if shape.layer_type == FULL else shape.window
        slot = (Lb - 1) % n if shape.layer_type == SLIDING else Lb - 1
        okc = f64(kc[b:b + 1, :, :n])
        ovc = f64(vc[b:b + 1, :, :n])
        okc[:, :, slot] = 0.0   # the oracle writes the new token itself
        ovc[:, :, slot] = 0.0
        okc, ovc = oracle.kv_append(okc, ovc, f64(k_new[b:b + 1]), f64(v_new[b:b + 1]),
                                    [Lb - 1], spec(shape))
        ref.append(oracle.decode(f64(q[b:b + 1]), f64(g[b:b + 1]), okc, ovc, [Lb],
                                 spec(shape))[0])
        got.append(f64(out[b]))
        del okc, ovc
    assert_close(np.stack(got), np.stack(ref), hgqa.BF16,
                 f"batched decode layer {layer_index}: {len(picks)} sequences incl. lengths "
                 f"{int(lens.min())} and {int(lens.max())}")
