"""Plain fp64 CPU oracle for one hybrid sliding/full grouped-query attention layer.

TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this module. The GPU library never
calls it, and it imports nothing from the GPU library.

What it computes is exact attention written out from its definition: no
tiling, no online softmax, no split over keys. Every stored bf16/fp32 input is
upcast exactly to float64 and all arithmetic stays in float64. Queries are
processed in row blocks only to bound memory; rows are independent, so this
does not change any value.

Sources (pages as published; sections as headed on each page):
  [P1] "Step-3.7-Flash-oQ3e" walkthrough (m.lqnn.cn), section 2 "sliding /
       full attention": 2.1 layer types, 2.2 how the source reads the setting
       and builds the two masks, 2.3 RoPE base per layer, partial rotary on
       full layers, head-wise sigmoid gate.
  [P2] "Step-3.7-Flash" model card (LLM Atlas), table "config.json: all 49
       fields": num_attention_heads 64, num_attention_groups 8, head_dim 128,
       sliding_window 512, rope_theta per layer, partial_rotary_factors,
       use_head_wise_attn_gate, sink false.
  [P1] 2.3 also: long-context frequency scaling ("rope_type llama3", factor
       2.0) is mounted on full layers only; sliding layers keep the default
       RoPE.
  [P4] "Muse-Glimmer-30B-6bit" architecture walkthrough (discosf.com),
       sections "each layer: double LayerNorm + gated attention" (gate_proj is
       a sigmoid gate on the attention output), "GQA 16:1", "sliding window
       attention: 39 + 13", "the RoPE zero value" (base 0 = no rotation).

Readings taken where the pages are silent (each is a choice, not a page fact):
  * window W counts keys including the query itself: key j is visible from
    query i iff i - W < j <= i ([P1] 2.2-2.3: a sliding layer "sees at most"
    W tokens and its cache keeps W tokens);
  * RoPE pairs dim i with dim i + r/2 inside the first r = round(f*D) dims,
    with frequency theta^(-2i/r); dims >= r pass through; theta == 0 or r == 0
    is the identity ([P1] 2.3, [P4] "the RoPE zero value");
  * positions are 0-based absolute token indices; a decode query sits at
    position L-1 where L counts cached tokens including the new one;
  * Q head h reads KV head floor(h / G) ([P2] 64 heads in 8 groups);
  * one gate logit per (token, head); out = sigmoid(gate) * attention
    ([P1] 2.3, [P4] gated attention);
  * softmax scale defaults to 1/sqrt(D); plain softmax with no sink ([P2]);
  * the "llama3" frequency scaling of [P1] 2.3 is the published Llama 3.1
    rule (see llama3_frequencies); the pages give only its factor, so the
    other three parameters are readings: low_freq_factor 1, high_freq_factor
    4 and an original context of 131072 positions (262144 / factor).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

FULL = "full_attention"
SLIDING = "sliding_attention"

# Rows per block in prefill: bounds the score block at ROW_BLOCK x keys.
ROW_BLOCK = 512


@dataclass(frozen=True)
class LayerSpec:
    """One attention layer as the config fields of [P2]/[P4] describe it.

    layer_type      FULL or SLIDING ([P1] 2.1 layer_types)
    window          W, keys visible to a query including itself (SLIDING only)
    num_q_heads     Hq ([P2] num_attention_heads; [P1] 2.2: 96 on sliding layers)
    num_kv_heads    Hkv ([P2] num_attention_groups; [P4] 2 KV heads)
    head_dim        D
    rope_theta      base; 0 means no rotation ([P4] "the RoPE zero value")
    rotary_fraction f; r = round(f*D) leading dims rotate ([P1] 2.3)
    softmax_scale   None means 1/sqrt(D)
    rope_scaling    None, or (factor, low_freq_factor, high_freq_factor,
                    original_max_positions) of the "llama3" frequency scaling;
                    applied on full layers only ([P1] 2.3)
    """

    layer_type: str
    window: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    rotary_fraction: float = 1.0
    softmax_scale: float | None = None
    rope_scaling: tuple | None = None

    @property
    def gqa_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rotary_dims(self) -> int:
        return int(round(self.rotary_fraction * self.head_dim))

    @property
    def scale(self) -> float:
        if self.softmax_scale is None:
            return 1.0 / math.sqrt(self.head_dim)
        return float(self.softmax_scale)

    @property
    def frequency_scaling(self):
        """The scaling this layer's RoPE uses: none on sliding layers ([P1] 2.3)."""
        if self.layer_type != FULL or self.rope_scaling is None:
            return None
        return self.rope_scaling


def sigmoid(x):
    """Logistic function 1/(1+e^-x): the per-head gate of [P1] 2.3 and [P4]."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def llama3_frequencies(omega, factor: float, low_freq_factor: float,
                       high_freq_factor: float, original_max_positions: float):
    """The "llama3" rescaling of RoPE frequencies ([P1] 2.3 names it, with
    factor 2.0, as the full layers' long-context extension).

    Per frequency w, with wavelength 2*pi/w and an original context length
    N: a wavelength shorter than N / high_freq_factor keeps w; one longer
    than N / low_freq_factor gets w / factor; in between, w is blended
    linearly, s = (N / wavelength - low_freq_factor) /
    (high_freq_factor - low_freq_factor), giving (1 - s) * w / factor + s * w.
    """
    w = np.asarray(omega, dtype=np.float64)
    if factor <= 1.0:
        return w.copy()
    wavelength = 2.0 * math.pi / w
    s = (original_max_positions / wavelength - low_freq_factor) / (high_freq_factor - low_freq_factor)
    blended = (1.0 - s) * w / factor + s * w
    out = np.where(wavelength > original_max_positions / low_freq_factor, w / factor, blended)
    return np.where(wavelength < original_max_positions / high_freq_factor, w, out)


def rope(x, positions, theta: float, rotary_dims: int, scaling=None):
    """Rotary position embedding of x at the given absolute positions.

    x has shape [..., D]; positions broadcasts against x[..., 0]. For
    i < r/2 the pair (x_i, x_{i+r/2}) is rotated by the angle p * w_i with
    w_i = theta^(-2i/r), rescaled by llama3_frequencies when scaling is given;
    dims r..D-1 are copied. theta == 0 or r == 0 returns x unchanged
    ([P1] 2.3 per-layer base, partial rotary and the full layers' scaling;
    [P4] "the RoPE zero value").
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    if theta == 0 or rotary_dims == 0:
        return out
    if rotary_dims % 2 or rotary_dims > x.shape[-1]:
        raise ValueError("rotary_dims must be even and at most head_dim")
    half = rotary_dims // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / rotary_dims)
    if scaling is not None:
        omega = llama3_frequencies(omega, *scaling)
    angle = np.asarray(positions, dtype=np.float64)[..., None] * omega
    c = np.cos(angle)
    s = np.sin(angle)
    x1 = x[..., :half]
    x2 = x[..., half:rotary_dims]
    out[..., :half] = x1 * c - x2 * s
    out[..., half:rotary_dims] = x2 * c + x1 * s
    return out


def visible(i, j, layer: LayerSpec):
    """Mask of [P1] 2.2: causal (j <= i), and for a sliding layer also i - j < W."""
    i = np.asarray(i)
    j = np.asarray(j)
    ok = j <= i
    if layer.layer_type == SLIDING:
        ok = ok & (i - j < layer.window)
    return ok


def _check_layer(layer: LayerSpec):
    if layer.layer_type not in (FULL, SLIDING):
        raise ValueError("layer_type must be FULL or SLIDING")
    if layer.layer_type == SLIDING and layer.window < 1:
        raise ValueError("a sliding layer needs window >= 1")
    if layer.num_q_heads % layer.num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")


def _softmax_attend(scores, values):
    """Row softmax of a masked score block (-inf = hidden) times values."""
    m = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - m)
    p /= p.sum(axis=-1, keepdims=True)
    return p @ values, p


def prefill(q, k, v, gate, layer: LayerSpec, return_probs: bool = False):
    """Gated causal GQA over a whole prompt starting at position 0.

    q [B,T,Hq,D], k and v [B,T,Hkv,D] (K not yet rotated), gate [B,T,Hq].
    Returns y [B,T,Hq,D] in float64 with
        y[b,i,h] = sigmoid(gate[b,i,h]) * sum_j P[i,j] v[b,j,h//G]
        P[i,:]   = softmax_j over visible j of scale * <rope(q_i,i), rope(k_j,j)>.
    With return_probs the full probability tensor [B,Hq,T,T] is also returned
    (small T only).
    """
    _check_layer(layer)
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    gate = np.asarray(gate, dtype=np.float64)
    B, T, Hq, D = q.shape
    G = layer.gqa_ratio
    pos = np.arange(T, dtype=np.float64)
    qr = rope(q, pos[None, :, None], layer.rope_theta, layer.rotary_dims, layer.frequency_scaling)
    kr = rope(k, pos[None, :, None], layer.rope_theta, layer.rotary_dims, layer.frequency_scaling)
    y = np.zeros((B, T, Hq, D), dtype=np.float64)
    probs = np.zeros((B, Hq, T, T), dtype=np.float64) if return_probs else None
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i0 in range(0, T, ROW_BLOCK):
                i1 = min(T, i0 + ROW_BLOCK)
                lo = 0
                if layer.layer_type == SLIDING:
                    lo = max(0, i0 - layer.window + 1)
                rows = np.arange(i0, i1)
                cols = np.arange(lo, i1)
                s = layer.scale * (qr[b, i0:i1, h] @ kr[b, lo:i1, kv].T)
                s = np.where(visible(rows[:, None], cols[None, :], layer), s, -np.inf)
                a, p = _softmax_attend(s, v[b, lo:i1, kv])
                y[b, i0:i1, h] = sigmoid(gate[b, i0:i1, h])[:, None] * a
                if probs is not None:
                    probs[b, h, i0:i1, lo:i1] = p
    if return_probs:
        return y, probs
    return y


def prefill_rows(q, k, v, gate, layer: LayerSpec, rows):
    """The prefill definition evaluated only at the listed (b, t, h) rows.

    Used where the whole output is too large for the CPU. Returns an array
    [len(rows), D] equal to prefill(...)[b, t, h] for each row.
    """
    _check_layer(layer)
    B, T, Hq, D = q.shape
    G = layer.gqa_ratio
    r = layer.rotary_dims
    rotated = {}
    out = np.zeros((len(rows), D), dtype=np.float64)
    for n, (b, t, h) in enumerate(rows):
        kv = h // G
        lo = 0
        if layer.layer_type == SLIDING:
            lo = max(0, t - layer.window + 1)
        key = (b, kv)
        if key not in rotated:
            kk = np.asarray(k[b, :, kv], dtype=np.float64)
            rotated[key] = rope(kk, np.arange(T, dtype=np.float64),
                                layer.rope_theta, r, layer.frequency_scaling)
        qi = rope(np.asarray(q[b, t, h], dtype=np.float64), float(t),
                  layer.rope_theta, r, layer.frequency_scaling)
        s = layer.scale * (rotated[key][lo:t + 1] @ qi)
        a, _ = _softmax_attend(s[None, :], np.asarray(v[b, lo:t + 1, kv], dtype=np.float64))
        out[n] = sigmoid(float(gate[b, t, h])) * a[0]
    return out


def kv_append(k_cache, v_cache, k_new, v_new, start_pos, layer: LayerSpec):
    """Append new tokens to a per-layer KV cache, one token at a time in order.

    k_cache, v_cache [B,Hkv,cap,D]; k_new, v_new [B,n,Hkv,D] (K not rotated);
    start_pos [B] is the absolute position of k_new[b,0]. Token n of sequence b
    sits at p = start_pos[b] + n; its rotated K and its V go to slot p of a
    full layer's cache, or to slot p mod W of a sliding layer's ring, whose
    capacity is W ([P1] 2.2: a sliding layer's cache keeps only W tokens).
    Later tokens overwrite earlier ones in a ring slot. Returns new float64
    caches; the inputs are not modified.
    """
    _check_layer(layer)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    B, n_new = k_new.shape[:2]
    cap = kc.shape[2]
    if layer.layer_type == SLIDING and cap != layer.window:
        raise ValueError("a sliding layer's ring holds exactly W slots")
    for b in range(B):
        for n in range(n_new):
            p = int(start_pos[b]) + n
            if layer.layer_type == SLIDING:
                slot = p % layer.window
            else:
                if p >= cap:
                    raise ValueError("position beyond the full cache")
                slot = p
            kc[b, :, slot] = rope(np.asarray(k_new[b, n], dtype=np.float64), float(p),
                                  layer.rope_theta, layer.rotary_dims, layer.frequency_scaling)
            vc[b, :, slot] = np.asarray(v_new[b, n], dtype=np.float64)
    return kc, vc


def cached_positions(seq_len: int, layer: LayerSpec, capacity: int):
    """Absolute positions a decode query at position seq_len-1 may attend to,
    and the cache slot each of them occupies ([P1] 2.2 masks and ring cache)."""
    if layer.layer_type == SLIDING:
        positions = np.arange(max(0, seq_len - layer.window), seq_len)
        return positions, positions % capacity
    positions = np.arange(seq_len)
    return positions, positions


def decode(q, gate, k_cache, v_cache, seq_lens, layer: LayerSpec):
    """One new query token per sequence against its cache.

    q [B,Hq,D] (not rotated), gate [B,Hq], caches [B,Hkv,cap,D] holding rotated
    K, seq_lens [B] tokens in the cache including the new one. The query sits
    at p = L-1 and sees every cached position the mask of its layer type keeps.
    Returns y [B,Hq,D] float64 = row p of prefill over the same history.
    """
    _check_layer(layer)
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = layer.gqa_ratio
    cap = k_cache.shape[2]
    y = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_lens[b])
        _, slots = cached_positions(L, layer, cap)
        qr = rope(q[b], float(L - 1), layer.rope_theta, layer.rotary_dims, layer.frequency_scaling)
        for h in range(Hq):
            kv = h // G
            kk = np.asarray(k_cache[b, kv, slots], dtype=np.float64)
            vv = np.asarray(v_cache[b, kv, slots], dtype=np.float64)
            s = layer.scale * (kk @ qr[h])
            a, _ = _softmax_attend(s[None, :], vv)
            y[b, h] = sigmoid(float(gate[b, h])) * a[0]
    return y


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits; frexp gives x = m * 2^e with
    0.5 <= |m| < 1, so m is rounded to a multiple of 2^-8 (np.rint rounds
    halves to even). Normal range only, which covers every value used here.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)
