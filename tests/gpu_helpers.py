"""Shared pieces of the GPU parity tests: layer conversion, seeded inputs,
and the comparison bar (max-abs <= 2e-2 and mean-abs <= 2e-3 for bf16,
max-abs <= 1e-4 for fp32)."""
import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth
from full_gqa_attention_layer_amd.workloads import SLIDING

BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
F32_MAX_ABS = 1e-4

DEV = "cuda:0"


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    hgqa.load_library()


def spec(shape):
    lt = oracle.SLIDING if shape.layer_type == SLIDING else oracle.FULL
    sc = tuple(shape.rope_scaling)
    if sc:   # the library's defaults for parameters left at 0
        sc = tuple(x if x > 0 else d for x, d in zip(sc + (0.0, 0.0, 0.0)[len(sc) - 1:],
                                                    (sc[0], 1.0, 4.0, 131072.0)))
    return oracle.LayerSpec(lt, max(shape.window, 1), shape.num_q_heads, shape.num_kv_heads,
                            shape.head_dim, shape.rope_theta, shape.rotary_fraction,
                            shape.softmax_scale if shape.softmax_scale > 0 else None,
                            sc if sc and sc[0] > 1.0 else None)


def tdtype(dtype):
    return torch.bfloat16 if dtype == hgqa.BF16 else torch.float32


def prefill_inputs(shape, B, T, dtype, key):
    dt = tdtype(dtype)
    q = synth.host_normal((B, T, shape.num_q_heads, shape.head_dim), key + (synth.Q,), dt)
    k = synth.host_normal((B, T, shape.num_kv_heads, shape.head_dim), key + (synth.K,), dt)
    v = synth.host_normal((B, T, shape.num_kv_heads, shape.head_dim), key + (synth.V,), dt)
    g = synth.host_normal((B, T, shape.num_q_heads), key + (synth.GATE,), dt)
    return q, k, v, g


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(gpu, ref, dtype, what=""):
    got = f64(gpu) if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    mx, mean = float(err.max()), float(err.mean())
    print(f"{what}: max-abs {mx:.3e} mean-abs {mean:.3e} over {err.size} values", flush=True)
    if dtype == hgqa.BF16:
        assert mx <= BF16_MAX_ABS and mean <= BF16_MEAN_ABS, (what, mx, mean)
    else:
        assert mx <= F32_MAX_ABS, (what, mx)
    return mx, mean
