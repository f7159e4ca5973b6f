"""Host accounting and workload shapes against the pages' printed numbers."""
import os

import numpy as np
import pytest

import oracle
from full_gqa_attention_layer_amd import accounting as acc
from full_gqa_attention_layer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_values():
    vals = {}
    with open(os.path.join(GOLDEN, "page_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split("=", 1)
            vals[key.strip()] = float(rest.split("|")[0])
    return vals


@pytest.mark.parametrize("T,lt,W", [(1, acc.FULL, 0), (17, acc.FULL, 0), (17, acc.SLIDING, 1),
                                    (17, acc.SLIDING, 5), (17, acc.SLIDING, 17),
                                    (17, acc.SLIDING, 40), (300, acc.SLIDING, 64)])
def test_visible_pairs_by_counting(T, lt, W):
    spec = oracle.LayerSpec(oracle.SLIDING if lt == acc.SLIDING else oracle.FULL,
                            max(W, 1), 1, 1, 8, 0.0)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    assert acc.visible_pairs(T, lt, W) == int(oracle.visible(i, j, spec).sum())


def test_visible_pairs_of_the_workloads():
    assert acc.visible_pairs(8192, acc.SLIDING, 512) == 4063488
    assert acc.visible_pairs(32768, acc.FULL, 0) == 536887296
    assert acc.visible_pairs(65536, acc.SLIDING, 2048) == 132121600
    assert acc.visible_pairs(65536, acc.FULL, 0) == 2147516416


def test_kv_cache_size_matches_page():
    with open(os.path.join(GOLDEN, "kv_cache_gib.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    for layers, ctx, kvh, d, eb, gib in rows:
        b = acc.kv_cache_bytes(int(layers), int(ctx), int(kvh), int(d), int(eb))
        assert b / 2 ** 30 == float(gib)


def test_hybrid_schedules_match_pages():
    pv = _page_values()
    step = acc.hybrid_schedule(int(pv["step.layers"]), int(pv["step.full_period"]), 0)
    assert step.count(acc.FULL) == pv["step.full_layers"]
    assert step.count(acc.SLIDING) == pv["step.sliding_layers"]
    # no other phase of a period-4 schedule gives 12 full layers among 45
    for phase in (1, 2, 3):
        assert acc.hybrid_schedule(45, 4, phase).count(acc.FULL) != 12
    first = int(pv["muse.first_full_layer_1based"]) - 1
    muse = acc.hybrid_schedule(int(pv["muse.layers"]), 4, first)
    assert muse.count(acc.FULL) == pv["muse.full_layers"]
    assert [i + 1 for i, t in enumerate(muse) if t == acc.FULL] == list(range(4, 53, 4))


def test_workload_shapes_follow_pages():
    pv = _page_values()
    (s,) = wl.STEP_SLIDING.layers
    assert (s.num_q_heads, s.num_kv_heads, s.head_dim, s.window, s.rope_theta,
            s.rotary_fraction) == (pv["step.sliding_q_heads"], pv["step.kv_groups"],
                                   pv["step.head_dim"], pv["step.sliding_window"],
                                   pv["step.theta_sliding"], pv["step.rotary_fraction_sliding"])
    (f,) = wl.STEP_FULL.layers
    assert (f.num_q_heads, f.num_kv_heads, f.rope_theta, f.rotary_fraction) == (
        pv["step.full_q_heads"], pv["step.kv_groups"], pv["step.theta_full"],
        pv["step.rotary_fraction_full"])
    m = wl.MUSE_BLOCK.layers
    assert [x.layer_type for x in m] == [wl.SLIDING] * 3 + [wl.FULL]
    assert all(x.num_q_heads == pv["muse.q_heads"] and x.num_kv_heads == pv["muse.kv_heads"]
               for x in m)
    assert all(x.window == pv["muse.sliding_window"] and x.rope_theta == pv["muse.theta_sliding"]
               for x in m[:3])
    assert m[3].rope_theta == pv["muse.theta_full"]


def test_flop_and_byte_counts():
    assert acc.prefill_flops(1, 8192, 96, 128, acc.SLIDING, 512) == 4 * 128 * 96 * 4063488
    assert acc.decode_bytes([512] * 64, 64, 8, 128, acc.SLIDING, 512) == \
        134217728 + 64 * 64 * 257 * 2
