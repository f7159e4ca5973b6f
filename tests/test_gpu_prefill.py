"""Prefill parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes are compared on every output element (several 64-key tiles,
ragged tails, every supported GQA ratio, both head dims, partial rotary,
base 0, window 1 and window >= T). At full size, the Step sliding layer is
compared on every element and each Muse sliding layer on every row of one KV
head; the full layers, whose oracle costs tens of TFLOP, on sampled rows the
oracle computes one by one: every head over the opening positions, around
the window edge and at the end, and seeded random rows.
"""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth, workloads
from full_gqa_attention_layer_amd.workloads import FULL, SLIDING, LayerShape
from tests.gpu_helpers import DEV, assert_close, f64, prefill_inputs, require_gpu, spec

pytestmark = pytest.mark.gpu


def run_prefill(shape, dtype, q, k, v, g):
    L = hgqa.layer_from_shape(shape, dtype)
    out = hgqa.attn_prefill(L, q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV))
    torch.cuda.synchronize()
    return out


def test_tiny_fp32_pair():
    """Two fp32 layers (sliding W=64 and full), T=256, 4 Q heads on 1 KV head."""
    require_gpu()
    wl = workloads.TINY_F32
    for li, shape in enumerate(wl.layers):
        q, k, v, g = prefill_inputs(shape, wl.batch, wl.seq_len, hgqa.FP32, (0, wl.wid, li))
        out = run_prefill(shape, hgqa.FP32, q, k, v, g)
        ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
        assert_close(out, ref, hgqa.FP32, f"tiny fp32 layer {li}")


SMALL = [
    # shape, batch, T, dtype
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), 1, 300, hgqa.BF16),
    (LayerShape(FULL, 0, 12, 1, 128, 5e6, 0.5), 2, 517, hgqa.BF16),
    (LayerShape(SLIDING, 100, 32, 2, 128, 5e5, 1.0), 1, 1000, hgqa.BF16),
    (LayerShape(FULL, 0, 32, 2, 128, 0.0, 1.0), 1, 777, hgqa.BF16),
    (LayerShape(SLIDING, 1, 4, 4, 128, 1e4, 1.0), 1, 130, hgqa.BF16),
    (LayerShape(SLIDING, 3, 8, 2, 64, 1e4, 1.0), 2, 200, hgqa.BF16),
    (LayerShape(SLIDING, 512, 16, 2, 128, 1e4, 1.0), 1, 300, hgqa.BF16),
    (LayerShape(FULL, 0, 16, 2, 64, 1e4, 0.25), 1, 129, hgqa.BF16),
    (LayerShape(FULL, 0, 24, 2, 128, 1e4, 1.0), 1, 1, hgqa.BF16),
    (LayerShape(SLIDING, 65, 96, 8, 128, 1e4, 1.0), 1, 260, hgqa.BF16),
    (LayerShape(SLIDING, 7, 6, 2, 128, 1e4, 0.5), 1, 150, hgqa.FP32),
    (LayerShape(FULL, 0, 4, 1, 64, 1e4, 6.0 / 64), 2, 90, hgqa.FP32),
    (LayerShape(FULL, 0, 2, 2, 128, 0.0, 1.0, 0.3), 1, 70, hgqa.FP32),
    # llama3 frequency scaling on a full layer, with a short original context so
    # that all three frequency regimes matter within a few hundred positions
    (LayerShape(FULL, 0, 8, 1, 128, 1e4, 1.0, 0.0, (2.0, 1.0, 4.0, 256)), 1, 600, hgqa.BF16),
    (LayerShape(FULL, 0, 4, 2, 128, 5e6, 0.5, 0.0, (3.0, 1.0, 8.0, 64)), 1, 300, hgqa.FP32),
    # ignored on a sliding layer
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0, 0.0, (2.0, 1.0, 4.0, 256)), 1, 300, hgqa.BF16),
]


@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_prefill_small_shapes_all_rows(idx):
    require_gpu()
    shape, B, T, dtype = SMALL[idx]
    q, k, v, g = prefill_inputs(shape, B, T, dtype, (0, 100 + idx, 0))
    out = run_prefill(shape, dtype, q, k, v, g)
    ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
    assert_close(out, ref, dtype, f"small[{idx}] {shape} B{B} T{T}")


# Both workgroup shapes of the bf16 kernel (4 waves / 128 rows and 8 waves /
# 256 rows) on each kind of layer, whatever the launcher would pick.
WAVE_CASES = [
    (LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0), 1, 300),
    (LayerShape(FULL, 0, 12, 1, 128, 5e6, 0.5), 2, 517),
    (LayerShape(SLIDING, 1024, 8, 1, 128, 5e5, 1.0), 1, 1200),
    (LayerShape(FULL, 0, 24, 2, 128, 1e4, 1.0), 1, 1),
    (LayerShape(FULL, 0, 16, 1, 128, 0.0, 1.0), 1, 333),
]


@pytest.mark.parametrize("waves", [4, 8])
@pytest.mark.parametrize("idx", range(len(WAVE_CASES)))
def test_prefill_both_workgroup_shapes(idx, waves, tuning):
    require_gpu()
    tuning(hgqa.TUNE_PREFILL_WAVES, waves)
    shape, B, T = WAVE_CASES[idx]
    q, k, v, g = prefill_inputs(shape, B, T, hgqa.BF16, (0, 170 + idx, 0))
    out = run_prefill(shape, hgqa.BF16, q, k, v, g)
    ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
    assert_close(out, ref, hgqa.BF16, f"waves {waves} case {idx} {shape} B{B} T{T}")


def test_peaky_scores():
    """Queries scaled by 8 make the softmax nearly one-hot and the scores 8x
    larger, so the bf16 rounding of the rotated q and k (the MFMA inputs)
    moves the scores 8x further than at unit scale. Two checks:
      * against the oracle fed the kernel's own MFMA inputs (base 0 on
        pre-rotated inputs): k rotated and rounded to bf16, and q rotated,
        multiplied by c = scale * log2(e) (the kernel takes scores in log2
        units), rounded to bf16 and divided by c again; the usual bf16 bar,
        which isolates everything else the kernel does;
      * against the plain oracle: max-abs within 8 x the usual bar (the score
        error, and with it the output error, grows linearly with q's scale),
        mean-abs within the usual bar."""
    require_gpu()
    s = 8
    shape = LayerShape(SLIDING, 64, 16, 2, 128, 1e4, 1.0)
    q, k, v, g = prefill_inputs(shape, 1, 400, hgqa.BF16, (0, 150, 0))
    q = (q.float() * s).to(torch.bfloat16)
    out = run_prefill(shape, hgqa.BF16, q, k, v, g)
    pos = np.arange(400, dtype=np.float64)[None, :, None]
    c = np.log2(np.e) / np.sqrt(128.0)
    qr = oracle.round_bf16(oracle.rope(f64(q), pos, 1e4, 128) * c) / c
    kr = oracle.round_bf16(oracle.rope(f64(k), pos, 1e4, 128))
    unrotated = LayerShape(SLIDING, 64, 16, 2, 128, 0.0, 1.0)
    ref_r = oracle.prefill(qr, kr, f64(v), f64(g), spec(unrotated))
    assert_close(out, ref_r, hgqa.BF16, "peaky vs rounded rotated inputs")
    ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
    err = np.abs(f64(out) - ref)
    print(f"peaky vs exact: max-abs {err.max():.3e} mean-abs {err.mean():.3e}", flush=True)
    assert err.max() <= s * 2e-2 and err.mean() <= 2e-3


class Rows:
    """fp64 NumPy view of a CPU tensor, converted one indexed piece at a time."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, idx):
        return f64(self.t[idx])


def sample_rows(B, T, Hq, W, n_random, seed, band=0, heads=None):
    """Rows (b, t, h) for a sampled comparison: every head at the first
    `band` positions, at the window edge and at the end, plus seeded random
    rows; heads restricts the heads."""
    rng = np.random.default_rng(seed)
    hs = list(range(Hq)) if heads is None else list(heads)
    edge = set(range(min(band, T))) | {0, 1, 2, T - 2, T - 1}
    if W:
        edge |= {W - 2, W - 1, W, W + 1, 2 * W + 3}
    edge = sorted(t for t in edge if 0 <= t < T)
    rows = [(b, t, h) for b in range(B) for t in edge for h in hs]
    for _ in range(n_random):
        rows.append((int(rng.integers(B)), int(rng.integers(T)), hs[int(rng.integers(len(hs)))]))
    return rows


def check_rows(out, inputs, shape, rows, what):
    q, k, v, g = inputs
    ref = oracle.prefill_rows(Rows(q), Rows(k), Rows(v), Rows(g), spec(shape), rows)
    idx = torch.tensor(rows)
    got = out[idx[:, 0], idx[:, 1], idx[:, 2]]
    return assert_close(got, ref, hgqa.BF16, f"{what}: {len(rows)} sampled rows")


def full_size_run(wl, li):
    shape = wl.layers[li]
    inputs = prefill_inputs(shape, wl.batch, wl.seq_len, hgqa.BF16, (0, wl.wid, li))
    return shape, inputs, run_prefill(shape, hgqa.BF16, *inputs)


def test_step_sliding_layer_full_size():
    """Every element of the Step sliding layer (T 8192, 96 Q / 8 KV heads,
    window 512) against the oracle."""
    require_gpu()
    wl = workloads.STEP_SLIDING
    shape, (q, k, v, g), out = full_size_run(wl, 0)
    ref = oracle.prefill(f64(q), f64(k), f64(v), f64(g), spec(shape))
    assert_close(out, ref, hgqa.BF16, f"{wl.name}: every element")


def test_step_full_layer_full_size():
    """The Step full layer (T 32768): every head at the first 64 positions,
    at the end, and 1500 seeded random rows."""
    require_gpu()
    wl = workloads.STEP_FULL
    shape, inputs, out = full_size_run(wl, 0)
    rows = sample_rows(wl.batch, wl.seq_len, shape.num_q_heads, 0, 1500, 0, band=64)
    check_rows(out, inputs, shape, rows, wl.name)


@pytest.mark.parametrize("li", [0, 1, 2])
def test_muse_sliding_layer_full_size(li):
    """A sliding layer of the Muse block (T 65536, window 2048, 16 Q heads per
    KV head): every row of one KV head's 16 query heads against the oracle's
    prefill of that head group, and sampled rows of the other KV head (the
    first 2048 positions of every head among them)."""
    require_gpu()
    wl = workloads.MUSE_BLOCK
    shape, (q, k, v, g), out = full_size_run(wl, li)
    G = shape.gqa_ratio
    kv = li % 2
    hs = slice(kv * G, (kv + 1) * G)
    one = oracle.LayerSpec(oracle.SLIDING, shape.window, G, 1, shape.head_dim, shape.rope_theta,
                           shape.rotary_fraction)
    ref = oracle.prefill(f64(q[:, :, hs]), f64(k[:, :, kv:kv + 1]), f64(v[:, :, kv:kv + 1]),
                         f64(g[:, :, hs]), one)
    assert_close(out[:, :, hs], ref, hgqa.BF16,
                 f"{wl.name} layer {li}: every row of KV head {kv}")
    del ref
    other = range((1 - kv) * G, (2 - kv) * G)
    rows = sample_rows(wl.batch, wl.seq_len, shape.num_q_heads, shape.window, 400, li,
                       band=shape.window, heads=[(1 - kv) * G])
    rows += sample_rows(wl.batch, wl.seq_len, shape.num_q_heads, shape.window, 400, 10 + li,
                        heads=other)
    check_rows(out, (q, k, v, g), shape, rows, f"{wl.name} layer {li}, KV head {1 - kv}")


def test_muse_full_layer_full_size():
    """The Muse block's full layer (T 65536, base 0): every head at the first
    128 positions, at the end, and 1000 seeded random rows."""
    require_gpu()
    wl = workloads.MUSE_BLOCK
    shape, inputs, out = full_size_run(wl, 3)
    rows = sample_rows(wl.batch, wl.seq_len, shape.num_q_heads, 0, 1000, 3, band=128)
    check_rows(out, inputs, shape, rows, f"{wl.name} layer 3")


def test_prefill_is_deterministic():
    require_gpu()
    shape = LayerShape(SLIDING, 512, 96, 8, 128, 1e4, 1.0)
    q, k, v, g = prefill_inputs(shape, 1, 2048, hgqa.BF16, (0, 160, 0))
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    args = [x.to(DEV) for x in (q, k, v, g)]
    a = hgqa.attn_prefill(L, *args)
    b = hgqa.attn_prefill(L, *args)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_prefill_is_a_no_op():
    require_gpu()
    shape = LayerShape(SLIDING, 64, 8, 2, 128, 1e4, 1.0)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    q = torch.empty(1, 0, 8, 128, dtype=torch.bfloat16, device=DEV)
    kv = torch.empty(1, 0, 2, 128, dtype=torch.bfloat16, device=DEV)
    g = torch.empty(1, 0, 8, dtype=torch.bfloat16, device=DEV)
    out = hgqa.attn_prefill(L, q, kv, kv.clone(), g)
    torch.cuda.synchronize()
    assert out.numel() == 0
