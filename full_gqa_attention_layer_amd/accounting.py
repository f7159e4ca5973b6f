"""Algorithmic work of the attention layer: the counts a roofline is priced on.

Only work the method itself must do is counted. Keys that the mask hides are
not counted, so a kernel that computes masked tiles pays for them out of its
efficiency. Exponentials, RoPE and the gate are not counted as FLOPs.
"""
from __future__ import annotations

FULL = 0
SLIDING = 1

# MI355X published peaks.
PEAK_BF16_TFLOPS = 2516.6      # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP32_TFLOPS = 157.3       # fp32 vector
PEAK_HBM_GBPS = 8000.0         # HBM3E


def visible_pairs(seq_len: int, layer_type: int, window: int) -> int:
    """Number of (query i, key j) pairs with j <= i, and i - j < W when sliding."""
    T = int(seq_len)
    if layer_type == SLIDING and window < T:
        W = int(window)
        return W * T - W * (W - 1) // 2
    return T * (T + 1) // 2


def prefill_flops(batch, seq_len, num_q_heads, head_dim, layer_type, window) -> int:
    """4*D FLOPs per visible pair and Q head: 2*D for q.k, 2*D for p*v."""
    return 4 * head_dim * num_q_heads * batch * visible_pairs(seq_len, layer_type, window)


def prefill_min_bytes(batch, seq_len, num_q_heads, num_kv_heads, head_dim, elem_bytes) -> int:
    """Each input read once and the output written once: Q, K, V, gate, out."""
    t = batch * seq_len
    return elem_bytes * t * (2 * num_q_heads * head_dim + 2 * num_kv_heads * head_dim
                             + num_q_heads)


def decode_visible(seq_len: int, layer_type: int, window: int) -> int:
    """Cached positions a decode query at position seq_len-1 attends to."""
    if layer_type == SLIDING:
        return min(int(seq_len), int(window))
    return int(seq_len)


def decode_bytes(seq_lens, num_q_heads, num_kv_heads, head_dim, layer_type, window,
                 elem_bytes=2) -> int:
    """Visible K and V rows of every sequence, plus q, gate and the output."""
    kv = sum(decode_visible(L, layer_type, window) for L in seq_lens)
    kv_bytes = kv * num_kv_heads * head_dim * 2 * elem_bytes
    b = len(seq_lens)
    io = b * num_q_heads * (2 * head_dim + 1) * elem_bytes
    return kv_bytes + io


def decode_flops(seq_lens, num_q_heads, head_dim, layer_type, window) -> int:
    kv = sum(decode_visible(L, layer_type, window) for L in seq_lens)
    return 4 * head_dim * num_q_heads * kv


def kv_cache_bytes(num_layers, context, num_kv_heads, head_dim, elem_bytes=2) -> int:
    """K and V for every layer kept at full context length (no ring)."""
    return num_layers * context * num_kv_heads * head_dim * 2 * elem_bytes


def hybrid_schedule(num_layers: int, period: int = 4, first_full: int = 0):
    """Layer types of a hybrid stack with one full layer every `period` layers,
    the first at 0-based index first_full; all others sliding."""
    return [FULL if (i % period) == first_full else SLIDING for i in range(num_layers)]
