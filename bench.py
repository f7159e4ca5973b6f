"""Throughput of the hybrid GQA attention hot path on one MI355X.

One step is one pass of the whole path over the Step-3.7-Flash sliding layer
(T = 8192, 96 Q / 8 KV heads, head_dim 128, window 512, RoPE base 1e4, bf16):
  attn_prefill over the prompt, kv_append of the prompt into the layer's
  512-slot ring, kv_append of one new token at position T, attn_decode of
  that token.
`value` is the algorithmic FLOPs of the step (4*D*Hq per visible query-key
pair) per second of step time. Decode bandwidth is measured beside it on
the batched-decode workload (64 sequences, contexts U[65536, 131072], full
layer over a contiguous cache and sliding layer over 512-slot rings) and
reported under "decode", together with a multi-token step (one token plus
three drafts per sequence, through attn_prefill_chunk) on the full layer's
caches. Chunked prefill (2048 new tokens over a 30720-token cache on the Step
full layer) is reported under "chunked_prefill". The CPU oracle is timed on a
bounded sample of the same prefill (whole KV groups of the layer) and
reported under "cpu_baseline".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode]
                    [--no-cpu-baseline] [--only prefill|decode|chunk|copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn prefill TFLOP/s + decode KV GB/s, % of MI355X roofline (1 GPU)"
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["prefill", "decode", "chunk", "copy"], default=None,
                   help="copy: a plain 1 GiB device copy, the reference kernel for "
                        "scaling HBM byte counters")
    p.add_argument("--cpu-groups", type=int, default=8,
                   help="KV groups of the layer in the CPU-oracle sample")
    return p.parse_args()


def source_hash(names):
    """Hash of the kernel sources' code: comments and layout are dropped, so
    a comment edit keeps a counter summary valid and any code edit does not."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "full_gqa_attention_layer_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def load_traffic(name, sources, per_launch_units):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; None otherwise."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(sources):
        return None
    return rec["hbm_bytes_per_launch"] * per_launch_units / rec.get("units_per_launch", 1)


class EventTimer:
    """HIP events on the current stream bracketing each call of one kind."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.e0 = self.torch.cuda.Event(enable_timing=True)
        self.e1 = self.torch.cuda.Event(enable_timing=True)
        self.e0.record()
        return self

    def __exit__(self, *exc):
        self.e1.record()
        self.pairs.append((self.e0, self.e1))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(len(self.pairs), 1)


def bench_step(args, torch, hgqa, synth, workloads, acc):
    wl = workloads.STEP_SLIDING
    shape = wl.layers[0]
    dev = torch.device("cuda:0")
    B, T, Hq, Hkv, D, W = wl.batch, wl.seq_len, shape.num_q_heads, shape.num_kv_heads, \
        shape.head_dim, shape.window
    key = (0, wl.wid, 0)
    q = synth.host_normal((B, T, Hq, D), key + (synth.Q,)).to(dev)
    k = synth.host_normal((B, T, Hkv, D), key + (synth.K,)).to(dev)
    v = synth.host_normal((B, T, Hkv, D), key + (synth.V,)).to(dev)
    g = synth.host_normal((B, T, Hq), key + (synth.GATE,)).to(dev)
    q1 = synth.host_normal((B, Hq, D), key + (synth.Q, 1)).to(dev)
    g1 = synth.host_normal((B, Hq), key + (synth.GATE, 1)).to(dev)
    k1 = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_K,)).to(dev)
    v1 = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_V,)).to(dev)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    out = torch.empty_like(q)
    ws = torch.empty(hgqa.attn_prefill_workspace_bytes(L, B, T), dtype=torch.uint8, device=dev)
    kc = torch.zeros(B, Hkv, W, D, dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    zero = torch.zeros(B, dtype=torch.int32, device=dev)
    pos = torch.full((B,), T, dtype=torch.int32, device=dev)
    lens = torch.full((B,), T + 1, dtype=torch.int32, device=dev)
    dws_n = hgqa.attn_decode_workspace_bytes(L, B, T + 1, W)
    dws = torch.empty(max(dws_n, 1), dtype=torch.uint8, device=dev)
    od = torch.empty_like(q1)
    timer = EventTimer(torch)

    def step(timed):
        if timed:
            with timer:
                hgqa.attn_prefill(L, q, k, v, g, out=out, workspace=ws)
        else:
            hgqa.attn_prefill(L, q, k, v, g, out=out, workspace=ws)
        hgqa.kv_append(L, zero, T, k, v, kc, vc)
        hgqa.kv_append(L, pos, T + 1, k1, v1, kc, vc)
        hgqa.attn_decode(L, q1, g1, kc, vc, lens, T + 1, out=od, workspace=dws)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    pf_flops = acc.prefill_flops(B, T, Hq, D, shape.layer_type, W)
    dec_flops = acc.decode_flops([T + 1], Hq, D, shape.layer_type, W)
    step_flops = pf_flops + dec_flops
    pf_ms = timer.mean_ms()
    achieved = pf_flops / (pf_ms * 1e-3) / 1e12
    traffic = load_traffic("attn_prefill_step_sliding_traffic.json",
                           ["prefill.hip", "rope_kernels.hip"], 1)
    return {
        "ms_per_step": ms,
        "value": step_flops / (ms * 1e-3) / 1e12,
        "prefill_ms": pf_ms,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": acc.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / acc.PEAK_BF16_TFLOPS,
                     "traffic": traffic,
                     "kernel": "attn_prefill (rope pre-pass + prefill_bf16_kernel<128, false, 4>)",
                     "algorithmic_flops_per_launch": pf_flops},
        "config": {"workload": wl.name, "batch": B, "seq_len": T, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": D, "window": W, "rope_theta": shape.rope_theta,
                   "step": "attn_prefill + kv_append(prompt) + kv_append(1) + attn_decode(1)"},
    }


def bench_decode(args, torch, hgqa, synth, workloads, acc):
    wl = workloads.BATCHED_DECODE
    dev = torch.device("cuda:0")
    B = wl.batch
    lens_np = synth.host_uniform_int(wl.min_seq_len, wl.seq_len, B, (0, wl.wid, 0, synth.SEQ_LENS))
    lens = torch.tensor(lens_np, dtype=torch.int32, device=dev)
    res = {}
    for li, shape in enumerate(wl.layers):
        Hq, Hkv, D = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
        sliding = shape.layer_type == workloads.SLIDING
        cap = shape.window if sliding else wl.seq_len
        # rings are small: cycle through enough sets to stay out of the 256 MB MALL
        nsets = 4 if sliding else 1
        caches = []
        for s in range(nsets):
            kc = torch.empty(B, Hkv, cap, D, dtype=torch.bfloat16, device=dev)
            vc = torch.empty_like(kc)
            for b in range(B):
                synth.device_normal_(kc[b], (0, wl.wid, li, synth.CACHE_K, b, s))
                synth.device_normal_(vc[b], (0, wl.wid, li, synth.CACHE_V, b, s))
            caches.append((kc, vc))
        print(f"[bench] decode layer {li}: {nsets} cache set(s) filled", file=sys.stderr,
              flush=True)
        key = (0, wl.wid, li)
        q = synth.host_normal((B, Hq, D), key + (synth.Q,)).to(dev)
        g = synth.host_normal((B, Hq), key + (synth.GATE,)).to(dev)
        kn = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_K,)).to(dev)
        vn = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_V,)).to(dev)
        L = hgqa.layer_from_shape(shape, hgqa.BF16)
        mx = int(lens_np.max())
        ws = torch.empty(max(hgqa.attn_decode_workspace_bytes(L, B, mx, cap), 1),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)
        start = lens - 1
        for kc, vc in caches:
            hgqa.kv_append(L, start, mx, kn, vn, kc, vc)
        timer, atimer = EventTimer(torch), EventTimer(torch)
        for i in range(args.warmup + args.steps):
            kc, vc = caches[i % nsets]
            if i >= args.warmup:
                with atimer:
                    hgqa.kv_append(L, start, mx, kn, vn, kc, vc)
                with timer:
                    hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out, workspace=ws)
            else:
                hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out, workspace=ws)
        torch.cuda.synchronize()
        ms = timer.mean_ms()
        nbytes = acc.decode_bytes(lens_np.tolist(), Hq, Hkv, D, shape.layer_type, shape.window)
        gbps = nbytes / (ms * 1e-3) / 1e9
        name = "full" if not sliding else "sliding"
        srcs = ["decode.hip"]
        res[name] = {
            "ms": ms, "GB/s": gbps, "kv_append_ms": atimer.mean_ms(),
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": acc.PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": gbps / acc.PEAK_HBM_GBPS,
                         "traffic": load_traffic(f"attn_decode_{name}_traffic.json", srcs, 1),
                         "kernel": "attn_decode (decode_bf16_kernel<128> + merge)",
                         "algorithmic_bytes_per_launch": nbytes},
            "workload": f"{B} sequences, {Hq} Q / {Hkv} KV heads, D{D}, "
                        + (f"{shape.window}-slot ring x {nsets} sets" if sliding
                           else f"contiguous cache, lengths U[{wl.min_seq_len},{wl.seq_len}]"),
        }
        if sliding:
            # labelled side figure: one ring set read again and again, so after
            # the first call it sits in the 256 MB MALL instead of HBM
            ctimer = EventTimer(torch)
            kc, vc = caches[0]
            for i in range(args.warmup + args.steps):
                if i >= args.warmup:
                    with ctimer:
                        hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out, workspace=ws)
                else:
                    hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out, workspace=ws)
            torch.cuda.synchronize()
            cms = ctimer.mean_ms()
            res[name]["in_cache"] = {"ms": cms, "GB/s": nbytes / (cms * 1e-3) / 1e9,
                                     "note": "one ring set, resident in the 256 MB MALL; "
                                             "not an HBM figure"}
        else:
            res["multi_token_full"] = bench_multi_token(args, torch, hgqa, synth, acc, L, caches[0],
                                                        key)
        del caches
        torch.cuda.empty_cache()
    return res


def bench_multi_token(args, torch, hgqa, synth, acc, L, cache, key):
    """A multi-token decode step (one token plus three drafts, causal among
    themselves) through attn_prefill_chunk, on the full layer's caches: every
    sequence at position 98300, the mean context of the batched workload."""
    kc, vc = cache
    B, Hkv, cap, D = kc.shape
    Hq, n, p0 = L.num_q_heads, 4, 98300
    dev = kc.device
    q = synth.host_normal((B, n, Hq, D), key + (synth.Q, 1)).to(dev)
    g = synth.host_normal((B, n, Hq), key + (synth.GATE, 1)).to(dev)
    kn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_K, 1)).to(dev)
    vn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_V, 1)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(hgqa.attn_prefill_chunk_workspace_bytes(L, B, n), dtype=torch.uint8, device=dev)
    timer = EventTimer(torch)
    for i in range(args.warmup + args.steps):
        if i >= args.warmup:
            with timer:
                hgqa.attn_prefill_chunk(L, p0, q, kn, vn, g, kc, vc, out=out, workspace=ws)
        else:
            hgqa.attn_prefill_chunk(L, p0, q, kn, vn, g, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    ms = timer.mean_ms()
    nbytes = B * (p0 + n) * Hkv * D * 2 * 2 + 2 * q.numel() * 2 + g.numel() * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"ms": ms, "GB/s": gbps, "frac_hbm": gbps / acc.PEAK_HBM_GBPS,
            "workload": f"{B} sequences at position {p0}, {n} new tokens each (1 + 3 drafts), "
                        f"{Hq} Q / {Hkv} KV heads, D{D}, full layer; attn_prefill_chunk incl. "
                        "the append of the 4 tokens"}


def bench_chunk(args, torch, hgqa, synth, workloads, acc):
    """Chunked prefill: the last 2048 tokens of the Step full layer's
    T = 32768 prompt, after the first 30720 are in the cache."""
    shape = workloads.STEP_FULL.layers[0]
    Hq, Hkv, D = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
    p0, n = 30720, 2048
    dev = torch.device("cuda:0")
    key = (0, workloads.STEP_FULL.wid, 0, 9)
    L = hgqa.layer_from_shape(shape, hgqa.BF16)
    kc = torch.empty(1, Hkv, p0 + n, D, dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    synth.device_normal_(kc, key + (synth.CACHE_K,))
    synth.device_normal_(vc, key + (synth.CACHE_V,))
    q = synth.host_normal((1, n, Hq, D), key + (synth.Q,)).to(dev)
    k = synth.host_normal((1, n, Hkv, D), key + (synth.K,)).to(dev)
    v = synth.host_normal((1, n, Hkv, D), key + (synth.V,)).to(dev)
    g = synth.host_normal((1, n, Hq), key + (synth.GATE,)).to(dev)
    out = torch.empty_like(q)
    ws = torch.empty(hgqa.attn_prefill_chunk_workspace_bytes(L, 1, n), dtype=torch.uint8, device=dev)
    timer = EventTimer(torch)
    for i in range(args.warmup + min(args.steps, 10)):
        if i >= args.warmup:
            with timer:
                hgqa.attn_prefill_chunk(L, p0, q, k, v, g, kc, vc, out=out, workspace=ws)
        else:
            hgqa.attn_prefill_chunk(L, p0, q, k, v, g, kc, vc, out=out, workspace=ws)
    torch.cuda.synchronize()
    ms = timer.mean_ms()
    pairs = n * p0 + n * (n + 1) // 2
    tflops = 4 * D * Hq * pairs / (ms * 1e-3) / 1e12
    return {"ms": ms, "TFLOP/s": tflops, "frac_mfma": tflops / acc.PEAK_BF16_TFLOPS,
            "workload": f"Step full layer (64 Q / 8 KV, D128, base 5e6, rotary 0.5): {n} new "
                        f"tokens at positions {p0}..{p0 + n - 1} over a {p0}-token cache; "
                        "attn_prefill_chunk incl. the append"}


def cpu_baseline(args, torch, synth, workloads, acc):
    """The fp64 oracle on the first KV groups of the same sliding layer."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    wl = workloads.STEP_SLIDING
    shape = wl.layers[0]
    ng = args.cpu_groups
    G = shape.gqa_ratio
    B, T, D = wl.batch, wl.seq_len, shape.head_dim
    key = (0, wl.wid, 0)
    q = synth.host_normal((B, T, shape.num_q_heads, D), key + (synth.Q,))[:, :, :ng * G]
    k = synth.host_normal((B, T, shape.num_kv_heads, D), key + (synth.K,))[:, :, :ng]
    v = synth.host_normal((B, T, shape.num_kv_heads, D), key + (synth.V,))[:, :, :ng]
    g = synth.host_normal((B, T, shape.num_q_heads), key + (synth.GATE,))[:, :, :ng * G]
    f = lambda t: t.to(torch.float64).numpy()
    spec = oracle.LayerSpec(oracle.SLIDING, shape.window, ng * G, ng, D, shape.rope_theta,
                            shape.rotary_fraction)
    qa, ka, va, ga = f(q), f(k), f(v), f(g)
    t0 = time.perf_counter()
    oracle.prefill(qa, ka, va, ga, spec)
    dt = time.perf_counter() - t0
    flops = acc.prefill_flops(B, T, ng * G, D, shape.layer_type, shape.window)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": dt,
            "sample": f"prefill of {ng} of {shape.num_kv_heads} KV groups ({ng * G} Q heads) of "
                      f"the T={T} sliding layer, all positions, fp64 NumPy"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path has no multi-GPU mode here).", file=sys.stderr)
        sys.exit(2)
    import torch

    from full_gqa_attention_layer_amd import accounting as acc
    from full_gqa_attention_layer_amd import hgqa, synth, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    hgqa.load_library()
    rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) inputs at the layer shapes; no weights)"}
    if args.only in (None, "prefill"):
        r = bench_step(args, torch, hgqa, synth, workloads, acc)
        rec.update({"value": r["value"], "unit": "TFLOP/s", "ms_per_step": r["ms_per_step"],
                    "config": r["config"], "roofline": r["roofline"],
                    "prefill_ms": r["prefill_ms"]})
        print(f"[bench] step {r['ms_per_step']:.4f} ms, prefill {r['prefill_ms']:.4f} ms, "
              f"{r['roofline']['achieved']:.1f} TFLOP/s", file=sys.stderr, flush=True)
    if not args.no_decode and args.only in (None, "decode"):
        rec["decode"] = bench_decode(args, torch, hgqa, synth, workloads, acc)
        print(f"[bench] decode {json.dumps(rec['decode'])}", file=sys.stderr, flush=True)
    if args.only is None or args.only == "chunk":
        rec["chunked_prefill"] = bench_chunk(args, torch, hgqa, synth, workloads, acc)
        print(f"[bench] chunked prefill {json.dumps(rec['chunked_prefill'])}", file=sys.stderr,
              flush=True)
    if not args.no_cpu_baseline and args.only is None:
        rec["cpu_baseline"] = cpu_baseline(args, torch, synth, workloads, acc)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
