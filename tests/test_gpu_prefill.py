"""Prefill parity: the HIP path through the C ABI against the fp64 oracle.

Small shapes are compared on every output element (several 64-key tiles,
ragged tails, every supported GQA ratio, both head dims, partial rotary,
base 0, window 1 and window >= T). Full-size workloads are compared on
sampled rows the oracle computes one by one: rows at the start, around the
window edge, at the end, and seeded random rows.
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


def sample_rows(B, T, Hq, W, n_random, seed):
    rng = np.random.default_rng(seed)
    edge = {0, 1, 2, T - 2, T - 1}
    if W:
        edge |= {W - 2, W - 1, W, W + 1, 2 * W + 3}
    edge = sorted(t for t in edge if 0 <= t < T)
    rows = [(b, t, h) for b in range(B) for t in edge for h in range(Hq)]
    for _ in range(n_random):
        rows.append((int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(Hq))))
    return rows


def check_sampled(shape, wl, li, n_random=600):
    q, k, v, g = prefill_inputs(shape, wl.batch, wl.seq_len, hgqa.BF16, (0, wl.wid, li))
    out = run_prefill(shape, hgqa.BF16, q, k, v, g)
    rows = sample_rows(wl.batch, wl.seq_len, shape.num_q_heads, shape.window, n_random, li)
    ref = oracle.prefill_rows(Rows(q), Rows(k), Rows(v), Rows(g), spec(shape), rows)
    idx = torch.tensor(rows)
    got = out[idx[:, 0], idx[:, 1], idx[:, 2]]
    return assert_close(got, ref, hgqa.BF16, f"{wl.name} layer {li}: {len(rows)} sampled rows")


def test_step_sliding_layer_full_size():
    require_gpu()
    wl = workloads.STEP_SLIDING
    check_sampled(wl.layers[0], wl, 0)


def test_step_full_layer_full_size():
    require_gpu()
    wl = workloads.STEP_FULL
    check_sampled(wl.layers[0], wl, 0, n_random=300)


def test_muse_block_full_size():
    require_gpu()
    wl = workloads.MUSE_BLOCK
    for li, shape in enumerate(wl.layers):
        check_sampled(shape, wl, li, n_random=200)


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
