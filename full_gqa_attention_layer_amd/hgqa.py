"""Python binding of libhgqa.so: the C ABI of include/hgqa.h under the same names.

This module only marshals arguments: it checks every tensor's shape against
the layer descriptor (Hq, Hkv = Hq / G and D come from the descriptor, never
from the tensors), its dtype and device, allocates outputs and workspaces with
torch, and passes raw device pointers and the current HIP stream. Every step
of the computation runs in the library's HIP kernels. If the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhgqa.so")

FULL, SLIDING = 0, 1
BF16, FP32 = 0, 1
OK, EINVAL, EUNSUPPORTED, ENOSPACE, EHIP = 0, -1, -2, -3, -4
TUNE_PREFILL_WAVES, TUNE_DECODE_SPLIT_KEYS, TUNE_CHUNK_SPLIT_TILES = 1, 2, 3

EXPORTED = ("attn_prefill_workspace_bytes", "attn_prefill", "attn_prefill_chunk_workspace_bytes",
            "attn_prefill_chunk", "kv_append", "attn_decode_workspace_bytes", "attn_decode",
            "attn_decode_noalloc", "hgqa_set_tuning", "hgqa_last_error")


class HgqaLayer(ctypes.Structure):
    """Mirror of the C struct hgqa_layer."""
    _fields_ = [("layer_type", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("gqa_ratio", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("rotary_fraction", ctypes.c_float), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("rope_scaling_factor", ctypes.c_float),
                ("rope_low_freq_factor", ctypes.c_float), ("rope_high_freq_factor", ctypes.c_float),
                ("rope_original_max_positions", ctypes.c_int32)]


class HgqaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"hgqa error {code}: {message}")
        self.code = code


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhgqa.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() or "
                           "python -m full_gqa_attention_layer_amd.build")
    lib = ctypes.CDLL(path)
    P, I, S = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    LP = ctypes.POINTER(HgqaLayer)
    lib.attn_prefill_workspace_bytes.argtypes = [LP, I, I]
    lib.attn_prefill_workspace_bytes.restype = S
    lib.attn_prefill.argtypes = [LP, I, I, P, P, P, P, P, P, S, P]
    lib.attn_prefill.restype = ctypes.c_int
    lib.attn_prefill_chunk_workspace_bytes.argtypes = [LP, I, I, I]
    lib.attn_prefill_chunk_workspace_bytes.restype = S
    lib.attn_prefill_chunk.argtypes = [LP, I, I, P, I, P, P, P, P, P, P, I, P, P, S, P]
    lib.attn_prefill_chunk.restype = ctypes.c_int
    lib.kv_append.argtypes = [LP, I, I, P, I, P, P, P, P, I, P]
    lib.kv_append.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [LP, I, I]
    lib.attn_decode_workspace_bytes.restype = S
    lib.attn_decode.argtypes = [LP, I, P, P, P, P, I, P, I, P, S, P, P]
    lib.attn_decode.restype = ctypes.c_int
    lib.attn_decode_noalloc.argtypes = [LP, I, P, P, P, P, I, P, I, P, P]
    lib.attn_decode_noalloc.restype = ctypes.c_int
    lib.hgqa_set_tuning.argtypes = [I, I]
    lib.hgqa_set_tuning.restype = ctypes.c_int
    lib.hgqa_last_error.argtypes = []
    lib.hgqa_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def hgqa_last_error() -> str:
    return load_library().hgqa_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise HgqaError(rc, hgqa_last_error())


def layer(layer_type: int, window: int, num_q_heads: int, gqa_ratio: int, head_dim: int,
          rope_theta: float, rotary_fraction: float = 1.0, softmax_scale: float = 0.0,
          dtype: int = BF16, rope_scaling=()) -> HgqaLayer:
    """rope_scaling: () for none, or (factor[, low_freq_factor, high_freq_factor,
    original_max_positions]) of the llama3 frequency scaling (full layers)."""
    sc = tuple(rope_scaling) + (0.0, 0.0, 0.0, 0)[len(tuple(rope_scaling)):]
    return HgqaLayer(layer_type, window, num_q_heads, gqa_ratio, head_dim, rope_theta,
                     rotary_fraction, softmax_scale, dtype, sc[0], sc[1], sc[2], int(sc[3]))


def layer_from_shape(shape, dtype: int = BF16) -> HgqaLayer:
    """Descriptor of a workloads.LayerShape."""
    return layer(shape.layer_type, shape.window, shape.num_q_heads, shape.gqa_ratio,
                 shape.head_dim, shape.rope_theta, shape.rotary_fraction,
                 shape.softmax_scale, dtype, shape.rope_scaling)


def _torch_dtype(L: HgqaLayer):
    return torch.bfloat16 if L.dtype == BF16 else torch.float32


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def _need(t, name, shape, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    """After every shape is checked: each tensor must live on the GPU. A
    workspace (any dtype; the library sees its bytes) must also be one
    contiguous block, since the library fills workspace_bytes from its start."""
    ws = tensors.get("workspace")
    if ws is not None:
        if not isinstance(ws, torch.Tensor):
            raise TypeError("workspace must be a tensor")
        if not ws.is_contiguous():
            raise ValueError("workspace must be contiguous")
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def attn_prefill_workspace_bytes(L: HgqaLayer, batch: int, seq_len: int) -> int:
    return int(load_library().attn_prefill_workspace_bytes(ctypes.byref(L), batch, seq_len))


def _heads(L: HgqaLayer):
    """(Hq, Hkv, D) as the descriptor gives them; the library indexes with these."""
    if L.gqa_ratio < 1 or L.num_q_heads < 1 or L.num_q_heads % L.gqa_ratio:
        raise ValueError(f"num_q_heads {L.num_q_heads} is not a positive multiple of "
                         f"gqa_ratio {L.gqa_ratio}")
    return L.num_q_heads, L.num_q_heads // L.gqa_ratio, L.head_dim


def set_tuning(knob: int, value: int):
    """Tuning override for tests and measurements (hgqa_set_tuning); 0 = automatic."""
    _check(load_library().hgqa_set_tuning(int(knob), int(value)))


def attn_prefill(L: HgqaLayer, q, k, v, gate, out=None, workspace=None):
    """Gated causal/sliding GQA of a prompt at positions 0..T-1 (see hgqa.h)."""
    lib = load_library()
    Hq, Hkv, D = _heads(L)
    B, T = q.shape[:2]
    dt = _torch_dtype(L)
    _need(q, "q", (B, T, Hq, D), dt)
    _need(k, "k", (B, T, Hkv, D), dt)
    _need(v, "v", (B, T, Hkv, D), dt)
    _need(gate, "gate", (B, T, Hq), dt)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, T, Hq, D), dt)
    _on_gpu(q=q, k=k, v=v, gate=gate, out=out, workspace=workspace)
    need = attn_prefill_workspace_bytes(L, B, T)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_prefill(ctypes.byref(L), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                            _ptr(out), _ptr(workspace), _nbytes(workspace), _stream()))
    return out


def attn_prefill_chunk_workspace_bytes(L: HgqaLayer, batch: int, n_new: int,
                                       max_end_pos: int) -> int:
    return int(load_library().attn_prefill_chunk_workspace_bytes(ctypes.byref(L), batch, n_new,
                                                                 max_end_pos))


def attn_prefill_chunk(L: HgqaLayer, start_pos, q, k, v, gate, k_cache, v_cache,
                       max_end_pos=None, out=None, workspace=None):
    """New tokens of sequence b at start_pos[b].. over the cache and themselves, then
    appended (see hgqa.h). start_pos: an int (every sequence) or an int32 tensor [B] on
    the GPU, which then needs max_end_pos (>= start_pos[b] + n for every b)."""
    lib = load_library()
    Hq, Hkv, D = _heads(L)
    B, n = q.shape[:2]
    cap = k_cache.shape[2]
    dt = _torch_dtype(L)
    if isinstance(start_pos, int):
        if max_end_pos is None:
            max_end_pos = start_pos + n
        start_pos = torch.full((B,), start_pos, dtype=torch.int32, device=q.device)
    elif max_end_pos is None:
        raise ValueError("a start_pos tensor needs max_end_pos")
    _need(q, "q", (B, n, Hq, D), dt)
    _need(k, "k", (B, n, Hkv, D), dt)
    _need(v, "v", (B, n, Hkv, D), dt)
    _need(gate, "gate", (B, n, Hq), dt)
    _need(k_cache, "k_cache", (B, Hkv, cap, D), dt)
    _need(v_cache, "v_cache", (B, Hkv, cap, D), dt)
    _need(start_pos, "start_pos", (B,), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, n, Hq, D), dt)
    _on_gpu(start_pos=start_pos, q=q, k=k, v=v, gate=gate, k_cache=k_cache, v_cache=v_cache,
            out=out, workspace=workspace)
    need = attn_prefill_chunk_workspace_bytes(L, B, n, int(max_end_pos))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.attn_prefill_chunk(ctypes.byref(L), B, n, _ptr(start_pos), int(max_end_pos),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(k_cache),
                                  _ptr(v_cache), cap, _ptr(out), _ptr(workspace),
                                  _nbytes(workspace), _stream()))
    return out


def kv_append(L: HgqaLayer, start_pos, max_end_pos: int, k_new, v_new, k_cache, v_cache):
    """Rotate and scatter new K/V into the layer's cache (see hgqa.h)."""
    lib = load_library()
    _, Hkv, D = _heads(L)
    B, n = k_new.shape[:2]
    cap = k_cache.shape[2]
    dt = _torch_dtype(L)
    _need(start_pos, "start_pos", (B,), torch.int32)
    _need(k_new, "k_new", (B, n, Hkv, D), dt)
    _need(v_new, "v_new", (B, n, Hkv, D), dt)
    _need(k_cache, "k_cache", (B, Hkv, cap, D), dt)
    _need(v_cache, "v_cache", (B, Hkv, cap, D), dt)
    _on_gpu(start_pos=start_pos, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache)
    _check(lib.kv_append(ctypes.byref(L), B, n, _ptr(start_pos), int(max_end_pos), _ptr(k_new),
                         _ptr(v_new), _ptr(k_cache), _ptr(v_cache), cap, _stream()))


def attn_decode_workspace_bytes(L: HgqaLayer, batch: int, max_seq_len: int) -> int:
    return int(load_library().attn_decode_workspace_bytes(ctypes.byref(L), batch, max_seq_len))


def attn_decode(L: HgqaLayer, q, gate, k_cache, v_cache, seq_lens, max_seq_len: int,
                out=None, workspace=None):
    """One query token per sequence against its cache (see hgqa.h)."""
    lib = load_library()
    Hq, Hkv, D = _heads(L)
    B = q.shape[0]
    cap = k_cache.shape[2]
    dt = _torch_dtype(L)
    _need(q, "q", (B, Hq, D), dt)
    _need(gate, "gate", (B, Hq), dt)
    _need(k_cache, "k_cache", (B, Hkv, cap, D), dt)
    _need(v_cache, "v_cache", (B, Hkv, cap, D), dt)
    _need(seq_lens, "seq_lens", (B,), torch.int32)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", (B, Hq, D), dt)
    _on_gpu(q=q, gate=gate, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, out=out,
            workspace=workspace)
    need = attn_decode_workspace_bytes(L, B, max_seq_len)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(lib.attn_decode(ctypes.byref(L), B, _ptr(q), _ptr(gate), _ptr(k_cache),
                           _ptr(v_cache), cap, _ptr(seq_lens), int(max_seq_len),
                           _ptr(workspace), _nbytes(workspace), _ptr(out), _stream()))
    return out


def attn_decode_noalloc(L: HgqaLayer, q, gate, k_cache, v_cache, seq_lens, max_seq_len: int, out):
    """attn_decode with the split partials in the library's static scratch: the
    library allocates nothing and neither does this wrapper (out is the caller's)."""
    lib = load_library()
    Hq, Hkv, D = _heads(L)
    B = q.shape[0]
    cap = k_cache.shape[2]
    dt = _torch_dtype(L)
    _need(q, "q", (B, Hq, D), dt)
    _need(gate, "gate", (B, Hq), dt)
    _need(k_cache, "k_cache", (B, Hkv, cap, D), dt)
    _need(v_cache, "v_cache", (B, Hkv, cap, D), dt)
    _need(seq_lens, "seq_lens", (B,), torch.int32)
    _need(out, "out", (B, Hq, D), dt)
    _on_gpu(q=q, gate=gate, k_cache=k_cache, v_cache=v_cache, seq_lens=seq_lens, out=out)
    _check(lib.attn_decode_noalloc(ctypes.byref(L), B, _ptr(q), _ptr(gate), _ptr(k_cache),
                                   _ptr(v_cache), cap, _ptr(seq_lens), int(max_seq_len), _ptr(out),
                                   _stream()))
    return out
