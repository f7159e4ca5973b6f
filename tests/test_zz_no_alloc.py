"""attn_decode_noalloc: decode that allocates nothing, its split partials in
the library's static per-GPU scratch. Checked through the C ABI against
attn_decode with a caller workspace (the same split plan and kernels, so the
outputs must agree bit for bit) and against the fp64 oracle, on two calls in
a row, the second smaller; and its refusal of a plan larger than the scratch
(host side, before any launch)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from full_gqa_attention_layer_amd import hgqa, synth
from full_gqa_attention_layer_amd.workloads import FULL, SLIDING, LayerShape
from tests.gpu_helpers import DEV, assert_close, f64, require_gpu, spec
from tests.test_gpu_decode import build_caches

SCRATCH_BYTES = 16 << 20


def _noalloc():
    lib = hgqa.load_library()
    fn = lib.attn_decode_noalloc
    P, I = ctypes.c_void_p, ctypes.c_int32
    fn.argtypes = [ctypes.POINTER(hgqa.HgqaLayer), I, P, P, P, P, I, P, I, P, P]
    fn.restype = ctypes.c_int
    return fn


def _call_noalloc(L, q, g, kc, vc, seq, max_len, out):
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return _noalloc()(ctypes.byref(L), q.shape[0], p(q), p(g), p(kc), p(vc), kc.shape[2], p(seq),
                      int(max_len), p(out), stream)


def test_plan_larger_than_the_scratch_is_refused():
    """B = 8, 128 Q heads on 8 KV heads, 100000 keys: the plan's 32 splits need
    8 * 128 * 32 * 130 * 4 bytes, above the 16 MiB scratch. Refused on the
    host with HGQA_ENOSPACE (fake pointers: nothing is launched)."""
    L = hgqa.layer(0, 0, 128, 16, 128, 5e6, 0.5)
    need = hgqa.load_library().attn_decode_workspace_bytes(ctypes.byref(L), 8, 100000)
    assert need == 8 * 128 * 32 * 130 * 4 > SCRATCH_BYTES
    p = ctypes.c_void_p(4096)
    o = ctypes.c_void_p(1 << 20)
    rc = _noalloc()(ctypes.byref(L), 8, p, p, p, p, 100000, p, 100000, o, None)
    assert rc == hgqa.ENOSPACE
    assert "scratch" in hgqa.hgqa_last_error()


CALLS = [
    # shape, lengths: the first call splits every sequence (40 splits of 512
    # keys, 5.3 MB of partials); the second is smaller (6 splits of 512 keys)
    (LayerShape(FULL, 0, 64, 8, 128, 5e6, 0.5), [5000, 20000, 1, 12000]),
    (LayerShape(FULL, 0, 16, 2, 128, 5e6, 0.5), [900, 3000]),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_decode_twice():
    require_gpu()
    for i, (shape, lens) in enumerate(CALLS):
        what = f"noalloc call {i}: {shape} lens {lens}"
        print(what, flush=True)
        key = (0, 950 + i, 0)
        kc, vc, okc, ovc, _ = build_caches(shape, hgqa.BF16, lens, key)
        B = len(lens)
        q = synth.host_normal((B, shape.num_q_heads, shape.head_dim), key + (synth.Q,)).to(DEV)
        g = synth.host_normal((B, shape.num_q_heads), key + (synth.GATE,)).to(DEV)
        L = hgqa.layer_from_shape(shape, hgqa.BF16)
        seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
        need = hgqa.attn_decode_workspace_bytes(L, B, max(lens))
        assert 0 < need <= SCRATCH_BYTES
        out = torch.full_like(q, float("nan"))
        assert _call_noalloc(L, q, g, kc, vc, seq, max(lens), out) == hgqa.OK, \
            hgqa.hgqa_last_error()
        ref = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), what
        exact = oracle.decode(f64(q), f64(g), okc, ovc, lens, spec(shape))
        assert_close(out, exact, hgqa.BF16, what)


@pytest.mark.gpu
def test_noalloc_without_splits():
    """A 512-slot ring of 64 sequences needs no partials: the scratch is not
    touched and the output equals attn_decode's."""
    require_gpu()
    shape = LayerShape(SLIDING, 512, 64, 8, 128, 1e4, 1.0)
    lens = [int(x) for x in np.random.default_rng(3).integers(1, 2000, size=64)]
    key = (0, 960, 0)
    kc, vc, okc, ovc, _ = build_caches(shape, hgqa.BF16, lens, key)
    q = synth.host_normal((64, 64, 128), key + (synth.Q,)).to(DEV)
    g = synth.host_normal((64, 64), key + (synth.GATE,)).to(DEV)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    assert hgqa.attn_decode_workspace_bytes(L, 64, max(lens)) == 0
    out = torch.empty_like(q)
    assert _call_noalloc(L, q, g, kc, vc, seq, max(lens), out) == hgqa.OK
    ref = hgqa.attn_decode(L, q, g, kc, vc, seq, max(lens))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert_close(out, oracle.decode(f64(q), f64(g), okc, ovc, lens, spec(shape)), hgqa.BF16,
                 "noalloc ring")
