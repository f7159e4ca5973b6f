"""The layer shapes this library is measured and checked on.

Each workload copies the shape of a layer the model pages describe:
  * Step-3.7-Flash ("Step-3.7-Flash-oQ3e" walkthrough, section 2; model card
    "config.json: all 49 fields"): 64 Q heads in 8 KV groups on full layers,
    96 Q heads on sliding layers, head_dim 128, window 512, RoPE base 5e6 on
    full layers (half of head_dim rotated) and 1e4 on sliding layers.
  * Muse-Glimmer-30B-6bit (architecture walkthrough, sections "GQA 16:1",
    "sliding window attention: 39 + 13", "the RoPE zero value"): 32 Q heads,
    2 KV heads, head_dim 128, window 2048, base 5e5 on sliding layers and 0
    (no rotation) on the full layer closing each group of four.
Inputs are standard normals; the pages' own evaluation data is not used.
"""
from __future__ import annotations

from dataclasses import dataclass, field

FULL = 0
SLIDING = 1


@dataclass(frozen=True)
class LayerShape:
    layer_type: int          # FULL or SLIDING
    window: int              # W for SLIDING, 0 for FULL
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    rope_theta: float
    rotary_fraction: float = 1.0
    softmax_scale: float = 0.0   # <= 0 means 1/sqrt(head_dim)
    # () or (factor, low_freq_factor, high_freq_factor, original_max_positions):
    # llama3 RoPE frequency scaling, full layers only
    rope_scaling: tuple = ()

    @property
    def gqa_ratio(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass(frozen=True)
class Workload:
    wid: int                 # workload id used in the input seeds
    name: str
    kind: str                # "prefill" or "decode"
    dtype: str               # "f32" or "bf16"
    batch: int
    seq_len: int             # prefill: tokens; decode: maximum context
    layers: tuple = field(default_factory=tuple)
    min_seq_len: int = 0     # decode only: lengths are uniform in [min, seq_len]


TINY_F32 = Workload(
    1, "tiny hybrid pair, fp32: T256, 4 Q / 1 KV head, D64, sliding W64 + full",
    "prefill", "f32", 1, 256,
    (LayerShape(SLIDING, 64, 4, 1, 64, 1e4, 1.0),
     LayerShape(FULL, 0, 4, 1, 64, 1e4, 1.0)))

STEP_SLIDING = Workload(
    2, "Step-3.7-Flash sliding layer prefill: T8192, 96 Q / 8 KV, D128, W512, base 1e4",
    "prefill", "bf16", 1, 8192,
    (LayerShape(SLIDING, 512, 96, 8, 128, 1e4, 1.0),))

STEP_FULL = Workload(
    3, "Step-3.7-Flash full layer prefill: T32768, 64 Q / 8 KV, D128, base 5e6, rotary 0.5",
    "prefill", "bf16", 1, 32768,
    (LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5),))

MUSE_BLOCK = Workload(
    4, "Muse-Glimmer 4-layer block prefill: T65536, 32 Q / 2 KV, D128, "
       "3 x sliding W2048 base 5e5 + full base 0",
    "prefill", "bf16", 1, 65536,
    (LayerShape(SLIDING, 2048, 32, 2, 128, 5e5, 1.0),
     LayerShape(SLIDING, 2048, 32, 2, 128, 5e5, 1.0),
     LayerShape(SLIDING, 2048, 32, 2, 128, 5e5, 1.0),
     LayerShape(FULL, 0, 32, 2, 128, 0.0, 1.0)))

BATCHED_DECODE = Workload(
    5, "batched decode: 64 sequences, 64 Q / 8 KV, D128; full layer over a contiguous "
       "cache with lengths U[65536,131072] (base 5e6, rotary 0.5) and sliding layer over "
       "a 512-slot ring (base 1e4)",
    "decode", "bf16", 64, 131072,
    (LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5),
     LayerShape(SLIDING, 512, 64, 8, 128, 1e4, 1.0)),
    min_seq_len=65536)

ALL = (TINY_F32, STEP_SLIDING, STEP_FULL, MUSE_BLOCK, BATCHED_DECODE)
