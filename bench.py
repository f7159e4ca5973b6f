"""Throughput of the hybrid GQA attention hot path on one MI355X.

Headline step: the Muse-Glimmer-shaped 4-layer block ("Muse-Glimmer-30B-6bit"
walkthrough: 32 Q / 2 KV heads, head_dim 128, three sliding layers with
window 2048 and RoPE base 5e5, then a full layer with base 0), T = 65536,
bf16. One step runs, for each of the four layers: attn_prefill over the
prompt, kv_append of the prompt into the layer's cache (a 2048-slot ring or a
contiguous cache), kv_append of one new token at position T and attn_decode of
that token. `value` is the step's algorithmic FLOPs (4*D*Hq per visible
query-key pair) per second of step time.

`roofline` is priced on the block's dominant launch, the full layer's
attn_prefill (84% of the block's FLOPs): its mean duration comes from one HIP
event pair around back-to-back calls on the launch stream, so the window holds
the kernels and no host time. Beside it:
  prefill      the Step full layer (T 32768, 64 Q / 8 KV, base 5e6, rotary 0.5)
               and the Step sliding layer (T 8192, 96 Q / 8 KV, window 512);
  decode       64 sequences, contexts U[65536, 131072]: the full layer over a
               contiguous cache and the sliding layer over 512-slot rings, and a
               1 + 3 token verify step at every sequence's own position;
  chunked      2048 new tokens over a 30720-token cache on the Step full layer;
  cpu_baseline the fp64 oracle on a seeded row sample of the same block, timed
               on the host's cores before the GPU is touched, extrapolated;
  clocks       GFX clock samples taken during the block's timed steps.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only block|prefill|decode|chunk|copy]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import threading
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["block", "prefill", "decode", "chunk", "copy"], default=None,
                   help="copy: a plain 1 GiB device copy, the reference kernel for "
                        "scaling HBM byte counters")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="target wall time of the CPU-oracle sample")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


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


PREFILL_SOURCES = ["prefill.hip", "rope_kernels.hip", "device_util.h", "hgqa_internal.h"]
DECODE_SOURCES = ["decode.hip", "device_util.h", "hgqa_internal.h"]


def load_traffic(name, sources):
    """HBM bytes per launch from a committed counter summary (rocprofv3
    FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading), if it was
    taken on the current kernel source; None otherwise."""
    path = os.path.join(PROFILES, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(sources):
        return None
    return rec["hbm_bytes_per_launch"]


def window_ms(torch, fn, n):
    """Mean GPU time of fn() over n back-to-back calls: one HIP event pair on
    the current stream (the library launches on it). One call runs ahead of
    the first event, so the host has queued the timed calls before the GPU
    reaches them and no host time falls inside the window."""
    fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


class ClockSampler:
    """GFX clock samples (MHz) from amdsmi's GPU metrics in a side thread while
    a timed region runs: the SMU's average GFX clock and the mean of the
    per-XCD current clocks, with the socket power (W) and hotspot temperature
    (C) beside them. Only readings of a refreshed metrics table count. Empty
    when amdsmi is not usable."""

    def __init__(self, period=0.01):
        self.period, self.avg, self.cur, self.error = period, [], [], None
        self.power, self.temp, self.power_cap = [], [], None
        self._stop = threading.Event()
        self._thread = None

    def __enter__(self):
        try:
            import amdsmi
            import torch
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            # amdsmi lists every GPU of the node: take the one whose PCI address
            # is this process's device 0
            p = torch.cuda.get_device_properties(0)
            want = (int(p.pci_domain_id), int(p.pci_bus_id), int(p.pci_device_id))
            self._h = None
            for h in amdsmi.amdsmi_get_processor_handles():
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, bus, rest = bdf.split(":")
                if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                    self._h, self.bdf = h, bdf
            if self._h is None:
                raise RuntimeError(f"no amdsmi device at PCI {want}")
            try:
                self.power_cap = amdsmi.amdsmi_get_power_cap_info(self._h)
            except Exception:  # noqa: BLE001 - optional
                self.power_cap = None
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        except Exception as e:  # noqa: BLE001 - the clock record is optional
            self.error = repr(e)
        return self

    def _run(self):
        def num(x):
            return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None
        # the SMU refreshes its metrics table on its own schedule: a reading
        # counts only when the table's own timestamp has moved since the last
        # one (and since the region started)
        last = None
        try:
            last = self._smi.amdsmi_get_gpu_metrics_info(self._h).get("system_clock_counter")
        except Exception:  # noqa: BLE001
            pass
        while not self._stop.is_set():
            try:
                m = self._smi.amdsmi_get_gpu_metrics_info(self._h)
                stamp = m.get("system_clock_counter")
                if stamp is not None and stamp == last:
                    time.sleep(self.period)
                    continue
                last = stamp
                a = num(m.get("average_gfxclk_frequency"))
                if a is not None:
                    self.avg.append(a)
                xcd = [num(x) for x in (m.get("current_gfxclks") or []) if num(x) is not None]
                if xcd:
                    self.cur.append(sum(xcd) / len(xcd))
                w = num(m.get("current_socket_power")) or num(m.get("average_socket_power"))
                if w is not None:
                    self.power.append(w)
                t = num(m.get("temperature_hotspot"))
                if t is not None:
                    self.temp.append(t)
            except Exception as e:  # noqa: BLE001
                self.error = repr(e)
                return
            time.sleep(self.period)

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()
            try:
                self._smi.amdsmi_shut_down()
            except Exception:  # noqa: BLE001
                pass

    def summary(self):
        def stats(v):
            if not v:
                return None
            v = sorted(v)
            return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "samples": len(v),
                    "distinct": len(set(v))}
        return {"average_gfxclk_mhz": stats(self.avg), "current_gfxclk_mhz_xcd_mean": stats(self.cur),
                "socket_power_w": stats(self.power), "hotspot_temp_c": stats(self.temp),
                "power_cap_info": self.power_cap,
                "error": self.error, "pci": getattr(self, "bdf", None),
                "source": "amdsmi GPU metrics, sampled every 10 ms during the timed region"}


# ----------------------------------------------------------------- inputs

def block_inputs(torch, synth, workloads):
    """Host bf16 inputs of the Muse block: per layer q, k, v, gate over the
    prompt, and one new token (q, gate, k, v) at position T."""
    wl = workloads.MUSE_BLOCK
    B, T = wl.batch, wl.seq_len
    layers = []
    for li, shape in enumerate(wl.layers):
        Hq, Hkv, D = shape.num_q_heads, shape.num_kv_heads, shape.head_dim
        key = (0, wl.wid, li)
        layers.append({
            "q": synth.host_normal((B, T, Hq, D), key + (synth.Q,)),
            "k": synth.host_normal((B, T, Hkv, D), key + (synth.K,)),
            "v": synth.host_normal((B, T, Hkv, D), key + (synth.V,)),
            "g": synth.host_normal((B, T, Hq), key + (synth.GATE,)),
            "q1": synth.host_normal((B, Hq, D), key + (synth.Q, 1)),
            "g1": synth.host_normal((B, Hq), key + (synth.GATE, 1)),
            "k1": synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_K,)),
            "v1": synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_V,)),
        })
    return layers


# ----------------------------------------------------------------- CPU oracle

_POOL_DATA = {}  # set before the worker pool forks; read by the workers


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)  # one BLAS thread per worker process
    except Exception:  # noqa: BLE001
        pass


def _oracle_task(task):
    """oracle.prefill on one head of one layer over the first positions.
    Returns seconds."""
    import oracle
    q, k, v, g, spec = _POOL_DATA["prefill"][task]
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, g, spec)
    return time.perf_counter() - t0


def _oracle_decode_task(task):
    import oracle
    q, g, kc, vc, lens, spec = _POOL_DATA["decode"][task]
    t0 = time.perf_counter()
    oracle.decode(q, g, kc, vc, lens, spec)
    return time.perf_counter() - t0


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(args, torch, synth, workloads, acc, block):
    """The fp64 oracle as it stands (oracle.prefill_rows, oracle.decode) on a
    seeded sample of the block's rows and of the batched decode's sequences,
    in a process pool: one worker per usable core (the affinity mask, capped
    by OMP_NUM_THREADS where that is set), one BLAS thread each. The pool forks
    before the GPU is touched. The block's time is extrapolated from the
    sample by visible query-key pairs."""
    import multiprocessing as mp

    import numpy as np

    import oracle

    affinity = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS", affinity) or affinity)
    workers = max(1, min(affinity, cap))
    wl = workloads.MUSE_BLOCK
    T = wl.seq_len
    rng = np.random.default_rng([0, wl.wid, 99])
    # one task = oracle.prefill of one seeded head of one layer over the first
    # Tp positions; per layer two tasks per worker, so the pool runs two
    # rounds of equal tasks per layer
    Tp = max(512, min(T, int(16384 * max(args.cpu_seconds, 1.0) / 20.0) // 512 * 512))
    tasks, sampled_flops = [], 0
    for li, shape in enumerate(wl.layers):
        lt = oracle.SLIDING if shape.layer_type == workloads.SLIDING else oracle.FULL
        G = shape.gqa_ratio
        spec = oracle.LayerSpec(lt, max(shape.window, 1), 1, 1, shape.head_dim, shape.rope_theta,
                                shape.rotary_fraction)
        L = block[li]
        # bf16 values are exact in fp32 and fp64; slices copied out before the fork
        np64 = lambda t: t.double().numpy().copy()
        for h in rng.choice(shape.num_q_heads, size=2 * workers,
                            replace=2 * workers > shape.num_q_heads):
            h = int(h)
            kv = h // G
            _POOL_DATA.setdefault("prefill", []).append(
                (np64(L["q"][:, :Tp, h:h + 1]), np64(L["k"][:, :Tp, kv:kv + 1]),
                 np64(L["v"][:, :Tp, kv:kv + 1]), np64(L["g"][:, :Tp, h:h + 1]), spec))
            tasks.append(len(_POOL_DATA["prefill"]) - 1)
            sampled_flops += acc.prefill_flops(1, Tp, 1, shape.head_dim, shape.layer_type,
                                               shape.window)
    # decode: 2 sequences of each layer of the batched workload, host caches of
    # the same shape and distribution (the values do not change the work)
    dwl = workloads.BATCHED_DECODE
    lens = synth.host_uniform_int(dwl.min_seq_len, dwl.seq_len, dwl.batch,
                                  (0, dwl.wid, 0, synth.SEQ_LENS))
    dec_tasks, dec_bytes = [], 0
    for li, shape in enumerate(dwl.layers):
        lt = oracle.SLIDING if shape.layer_type == workloads.SLIDING else oracle.FULL
        spec = oracle.LayerSpec(lt, max(shape.window, 1), shape.num_q_heads, shape.num_kv_heads,
                                shape.head_dim, shape.rope_theta, shape.rotary_fraction)
        for j, b in enumerate((0, 1)):
            Lb = int(lens[b])
            cap = shape.window if lt == oracle.SLIDING else Lb
            key = (0, dwl.wid, li, 50 + j)
            kc = synth.host_normal((1, shape.num_kv_heads, cap, shape.head_dim),
                                   key + (synth.CACHE_K,)).float().numpy()
            vc = synth.host_normal((1, shape.num_kv_heads, cap, shape.head_dim),
                                   key + (synth.CACHE_V,)).float().numpy()
            q = synth.host_normal((1, shape.num_q_heads, shape.head_dim), key + (synth.Q,))
            g = synth.host_normal((1, shape.num_q_heads), key + (synth.GATE,))
            _POOL_DATA.setdefault("decode", []).append(
                (q.double().numpy(), g.double().numpy(), kc, vc, [Lb], spec))
            dec_tasks.append(len(_POOL_DATA["decode"]) - 1)
            dec_bytes += acc.decode_bytes([Lb], shape.num_q_heads, shape.num_kv_heads,
                                          shape.head_dim, shape.layer_type, shape.window)
    log(f"cpu oracle: {len(tasks)} prefill tasks (T' = {Tp}), {len(dec_tasks)} decode tasks, "
        f"{workers} workers")
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_pool_init) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_task, tasks, chunksize=1)
        pf_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        pool.map(_oracle_decode_task, dec_tasks, chunksize=1)
        dec_s = time.perf_counter() - t0
    _POOL_DATA.clear()
    rate = sampled_flops / pf_s
    block_flops = sum(acc.prefill_flops(wl.batch, T, s.num_q_heads, s.head_dim, s.layer_type,
                                        s.window) for s in wl.layers)
    return {
        "value": rate / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
        "sample": (f"fp64 oracle.prefill of {len(tasks)} seeded single heads ({2 * workers} per layer) "
                   f"of the T={T} Muse block over their first {Tp} positions "
                   f"({sampled_flops / 1e9:.1f} GFLOP in {pf_s:.1f} s); the whole block's time "
                   "extrapolated from that rate (FLOPs of visible pairs)"),
        "affinity_cores": affinity, "cpu_model": cpu_model(),
        "blas_threads_per_worker": 1,
        "block_seconds_extrapolated": block_flops / rate,
        "decode": {"GB/s": dec_bytes / dec_s / 1e9, "seconds": dec_s,
                   "sample": "fp64 oracle.decode of 2 sequences of each batched-decode layer "
                             "(full cache and 512-slot ring) at the workload's first lengths",
                   "batch_seconds_extrapolated_full_layer":
                       dec_s * float(lens.sum()) / float(lens[:2].sum()) / 2},
    }


# ----------------------------------------------------------------- GPU legs

def bench_block(args, torch, hgqa, workloads, acc, block):
    """The headline step over the Muse 4-layer block."""
    wl = workloads.MUSE_BLOCK
    dev = torch.device("cuda:0")
    B, T = wl.batch, wl.seq_len
    st = []
    for li, shape in enumerate(wl.layers):
        h = {k: t.to(dev) for k, t in block[li].items()}
        L = hgqa.layer_from_shape(shape, hgqa.BF16)
        Hkv, D = shape.num_kv_heads, shape.head_dim
        sliding = shape.layer_type == workloads.SLIDING
        cap = shape.window if sliding else T + 1
        h["out"] = torch.empty_like(h["q"])
        h["ws"] = torch.empty(hgqa.attn_prefill_workspace_bytes(L, B, T), dtype=torch.uint8,
                              device=dev)
        h["kc"] = torch.zeros(B, Hkv, cap, D, dtype=torch.bfloat16, device=dev)
        h["vc"] = torch.zeros_like(h["kc"])
        h["od"] = torch.empty_like(h["q1"])
        dws = hgqa.attn_decode_workspace_bytes(L, B, T + 1)
        h["dws"] = torch.empty(max(dws, 1), dtype=torch.uint8, device=dev)
        h["zero"] = torch.zeros(B, dtype=torch.int32, device=dev)
        h["pos"] = torch.full((B,), T, dtype=torch.int32, device=dev)
        h["lens"] = torch.full((B,), T + 1, dtype=torch.int32, device=dev)
        st.append((L, shape, h))

    def prefill(L, h):
        hgqa.attn_prefill(L, h["q"], h["k"], h["v"], h["g"], out=h["out"], workspace=h["ws"])

    def step():
        for L, shape, h in st:
            prefill(L, h)
            hgqa.kv_append(L, h["zero"], T, h["k"], h["v"], h["kc"], h["vc"])
            hgqa.kv_append(L, h["pos"], T + 1, h["k1"], h["v1"], h["kc"], h["vc"])
            hgqa.attn_decode(L, h["q1"], h["g1"], h["kc"], h["vc"], h["lens"], T + 1,
                             out=h["od"], workspace=h["dws"])

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps
    flops = 0
    layers = []
    n_win = max(3, min(args.steps, 10))
    for li, (L, shape, h) in enumerate(st):
        pf = acc.prefill_flops(B, T, shape.num_q_heads, shape.head_dim, shape.layer_type,
                               shape.window)
        dec = acc.decode_flops([T + 1], shape.num_q_heads, shape.head_dim, shape.layer_type,
                               shape.window)
        flops += pf + dec
        wms = window_ms(torch, lambda: prefill(L, h), n_win)
        kind = "sliding W2048 base 5e5" if shape.layer_type == workloads.SLIDING else "full base 0"
        layers.append({"layer": li, "kind": kind, "prefill_ms": wms, "prefill_flops": pf,
                       "TFLOP/s": pf / (wms * 1e-3) / 1e12,
                       "frac_mfma": pf / (wms * 1e-3) / 1e12 / acc.PEAK_BF16_TFLOPS})
        log(f"block layer {li} ({kind}): {wms:.3f} ms, {layers[-1]['TFLOP/s']:.0f} TFLOP/s")
    full = layers[-1]
    kernel = "prefill_bf16_kernel<128, 0, 8, false> (+ its pre-pass: rotated K, cos/sin rows, V^T)"
    return {
        "ms_per_step": ms,
        "value": flops / (ms * 1e-3) / 1e12,
        "roofline": {"bound": "mfma", "achieved": full["TFLOP/s"], "peak": acc.PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": full["frac_mfma"],
                     "traffic": load_traffic("attn_prefill_muse_full_traffic.json",
                                             PREFILL_SOURCES),
                     "kernel": f"attn_prefill of the block's full layer: {kernel}",
                     "algorithmic_flops_per_launch": full["prefill_flops"],
                     "launch_ms": full["prefill_ms"],
                     "timing": f"one HIP event pair around {n_win} back-to-back calls"},
        "layers": layers,
        "prefill_block_ms": sum(x["prefill_ms"] for x in layers),
        "prefill_block_TFLOP/s": sum(x["prefill_flops"] for x in layers)
                                 / (sum(x["prefill_ms"] for x in layers) * 1e-3) / 1e12,
        "clocks": clk.summary(),
        "config": {"workload": wl.name, "batch": B, "seq_len": T, "q_heads": 32, "kv_heads": 2,
                   "head_dim": 128, "layers": "3 x sliding (W2048, base 5e5) + full (base 0)",
                   "step": "per layer: attn_prefill + kv_append(prompt) + kv_append(1) + "
                           "attn_decode(1)"},
    }


def bench_prefill(args, torch, hgqa, synth, workloads, acc):
    """Step full layer (T 32768) and Step sliding layer (T 8192)."""
    dev = torch.device("cuda:0")
    res = {}
    for name, wl, n in (("step_full", workloads.STEP_FULL, 5),
                        ("step_sliding", workloads.STEP_SLIDING, 20)):
        shape = wl.layers[0]
        B, T = wl.batch, wl.seq_len
        key = (0, wl.wid, 0)
        q = synth.host_normal((B, T, shape.num_q_heads, shape.head_dim), key + (synth.Q,)).to(dev)
        k = synth.host_normal((B, T, shape.num_kv_heads, shape.head_dim), key + (synth.K,)).to(dev)
        v = synth.host_normal((B, T, shape.num_kv_heads, shape.head_dim), key + (synth.V,)).to(dev)
        g = synth.host_normal((B, T, shape.num_q_heads), key + (synth.GATE,)).to(dev)
        L = hgqa.layer_from_shape(shape, hgqa.BF16)
        out = torch.empty_like(q)
        ws = torch.empty(hgqa.attn_prefill_workspace_bytes(L, B, T), dtype=torch.uint8, device=dev)
        fn = lambda: hgqa.attn_prefill(L, q, k, v, g, out=out, workspace=ws)
        for _ in range(args.warmup):
            fn()
        with ClockSampler() as clk:
            ms = window_ms(torch, fn, n)
        pf = acc.prefill_flops(B, T, shape.num_q_heads, shape.head_dim, shape.layer_type,
                               shape.window)
        tf = pf / (ms * 1e-3) / 1e12
        res[name] = {"ms": ms, "TFLOP/s": tf, "frac_mfma": tf / acc.PEAK_BF16_TFLOPS,
                     "flops": pf, "workload": wl.name, "clocks": clk.summary(),
                     "timing": f"one HIP event pair around {n} back-to-back attn_prefill calls "
                               "(pre-pass + attention kernel)"}
        log(f"prefill {name}: {ms:.3f} ms, {tf:.0f} TFLOP/s")
        del q, k, v, g, out, ws
        torch.cuda.empty_cache()
    return res


def bench_decode(args, torch, hgqa, synth, workloads, acc):
    wl = workloads.BATCHED_DECODE
    dev = torch.device("cuda:0")
    B = wl.batch
    lens_np = synth.host_uniform_int(wl.min_seq_len, wl.seq_len, B, (0, wl.wid, 0, synth.SEQ_LENS))
    lens = torch.tensor(lens_np, dtype=torch.int32, device=dev)
    mx = int(lens_np.max())
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
        log(f"decode layer {li}: {nsets} cache set(s) filled")
        key = (0, wl.wid, li)
        q = synth.host_normal((B, Hq, D), key + (synth.Q,)).to(dev)
        g = synth.host_normal((B, Hq), key + (synth.GATE,)).to(dev)
        kn = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_K,)).to(dev)
        vn = synth.host_normal((B, 1, Hkv, D), key + (synth.NEW_V,)).to(dev)
        L = hgqa.layer_from_shape(shape, hgqa.BF16)
        ws = torch.empty(max(hgqa.attn_decode_workspace_bytes(L, B, mx), 1), dtype=torch.uint8,
                         device=dev)
        out = torch.empty_like(q)
        start = lens - 1
        for kc, vc in caches:
            hgqa.kv_append(L, start, mx, kn, vn, kc, vc)
        it = [0]

        def dec():
            kc, vc = caches[it[0] % nsets]
            it[0] += 1
            hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out, workspace=ws)

        def app():
            kc, vc = caches[it[0] % nsets]
            it[0] += 1
            hgqa.kv_append(L, start, mx, kn, vn, kc, vc)

        for _ in range(args.warmup):
            dec()
        n = max(args.steps, 4 * nsets)
        ms = window_ms(torch, dec, n)
        ams = window_ms(torch, app, n)
        nbytes = acc.decode_bytes(lens_np.tolist(), Hq, Hkv, D, shape.layer_type, shape.window)
        gbps = nbytes / (ms * 1e-3) / 1e9
        name = "full" if not sliding else "sliding"
        res[name] = {
            "ms": ms, "GB/s": gbps, "kv_append_ms": ams,
            "roofline": {"bound": "hbm", "achieved": gbps, "peak": acc.PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": gbps / acc.PEAK_HBM_GBPS,
                         "traffic": load_traffic(f"attn_decode_{name}_traffic.json",
                                                 DECODE_SOURCES),
                         "kernel": "attn_decode (decode_bf16_kernel<128> + merge)",
                         "algorithmic_bytes_per_launch": nbytes},
            "workload": f"{B} sequences, {Hq} Q / {Hkv} KV heads, D{D}, "
                        + (f"{shape.window}-slot ring x {nsets} sets" if sliding
                           else f"contiguous cache, lengths U[{wl.min_seq_len},{wl.seq_len}]"),
        }
        log(f"decode {name}: {ms:.4f} ms, {gbps:.0f} GB/s")
        if sliding:
            # labelled side figure: one ring set read again and again, so after
            # the first call it sits in the 256 MB MALL instead of HBM
            kc, vc = caches[0]
            cms = window_ms(torch, lambda: hgqa.attn_decode(L, q, g, kc, vc, lens, mx, out=out,
                                                            workspace=ws), args.steps)
            res[name]["in_cache"] = {"ms": cms, "GB/s": nbytes / (cms * 1e-3) / 1e9,
                                     "note": "one ring set, resident in the 256 MB MALL; "
                                             "not an HBM figure"}
        else:
            res["multi_token_full"] = bench_verify(args, torch, hgqa, synth, acc, L, caches[0],
                                                   key, lens_np)
        del caches
        torch.cuda.empty_cache()
    return res


def bench_verify(args, torch, hgqa, synth, acc, L, cache, key, lens_np):
    """A 1 + 3 token verify step (causal among the four new tokens) through
    attn_prefill_chunk on the full layer's caches, every sequence at its own
    position: its last new token sits where the batched decode's query sits
    (position L_b - 1), so it sees the same L_b keys."""
    kc, vc = cache
    B, Hkv, cap, D = kc.shape
    Hq, n = L.num_q_heads, 4
    dev = kc.device
    q = synth.host_normal((B, n, Hq, D), key + (synth.Q, 1)).to(dev)
    g = synth.host_normal((B, n, Hq), key + (synth.GATE, 1)).to(dev)
    kn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_K, 1)).to(dev)
    vn = synth.host_normal((B, n, Hkv, D), key + (synth.NEW_V, 1)).to(dev)
    starts = lens_np - n
    sp = torch.tensor(starts, dtype=torch.int32, device=dev)
    end = int(lens_np.max())
    out = torch.empty_like(q)
    ws = torch.empty(hgqa.attn_prefill_chunk_workspace_bytes(L, B, n, end), dtype=torch.uint8,
                     device=dev)
    fn = lambda: hgqa.attn_prefill_chunk(L, sp, q, kn, vn, g, kc, vc, max_end_pos=end, out=out,
                                         workspace=ws)
    for _ in range(args.warmup):
        fn()
    ms = window_ms(torch, fn, args.steps)
    nbytes = int(lens_np.sum()) * Hkv * D * 2 * 2 + 2 * q.numel() * 2 + g.numel() * 2
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"verify step: {ms:.3f} ms, {gbps:.0f} GB/s")
    return {"ms": ms, "GB/s": gbps, "frac_hbm": gbps / acc.PEAK_HBM_GBPS,
            "workload": f"{B} sequences at their own positions (the batched decode's lengths "
                        f"L_b ~ U[65536, 131072]), {n} new tokens each (1 + 3 drafts) ending at "
                        f"L_b - 1, {Hq} Q / {Hkv} KV heads, D{D}, full layer; "
                        "attn_prefill_chunk incl. the append of the 4 tokens"}


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
    ws = torch.empty(hgqa.attn_prefill_chunk_workspace_bytes(L, 1, n, p0 + n), dtype=torch.uint8,
                     device=dev)
    fn = lambda: hgqa.attn_prefill_chunk(L, p0, q, k, v, g, kc, vc, out=out, workspace=ws)
    for _ in range(args.warmup):
        fn()
    ms = window_ms(torch, fn, min(args.steps, 10))
    pairs = n * p0 + n * (n + 1) // 2
    tflops = 4 * D * Hq * pairs / (ms * 1e-3) / 1e12
    log(f"chunked prefill: {ms:.3f} ms, {tflops:.0f} TFLOP/s")
    return {"ms": ms, "TFLOP/s": tflops, "frac_mfma": tflops / acc.PEAK_BF16_TFLOPS,
            "workload": f"Step full layer (64 Q / 8 KV, D128, base 5e6, rotary 0.5): {n} new "
                        f"tokens at positions {p0}..{p0 + n - 1} over a {p0}-token cache; "
                        "attn_prefill_chunk incl. the append"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path has no multi-GPU mode here).", file=sys.stderr)
        sys.exit(2)
    import torch

    from full_gqa_attention_layer_amd import accounting as acc
    from full_gqa_attention_layer_amd import hgqa, synth, workloads

    rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded N(0,1) inputs at the layer shapes; no weights)"}
    block = None
    if args.only in (None, "block"):
        block = block_inputs(torch, synth, workloads)
        log("block inputs drawn")
    # the CPU oracle forks its worker pool before anything touches the GPU
    cpu = None
    if not args.no_cpu_baseline and args.only is None:
        cpu = cpu_baseline(args, torch, synth, workloads, acc, block)
        log(f"cpu oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} cores")

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
    if block is not None:
        r = bench_block(args, torch, hgqa, workloads, acc, block)
        rec.update({"value": r["value"], "unit": "TFLOP/s", "ms_per_step": r["ms_per_step"],
                    "config": r["config"], "roofline": r["roofline"]})
        rec["block"] = {k: r[k] for k in ("layers", "prefill_block_ms", "prefill_block_TFLOP/s",
                                          "clocks")}
        log(f"block step {r['ms_per_step']:.3f} ms, {r['value']:.0f} TFLOP/s; full layer "
            f"{r['roofline']['achieved']:.0f} TFLOP/s ({r['roofline']['frac']:.3f})")
        del block
    if args.only in (None, "prefill"):
        rec["prefill"] = bench_prefill(args, torch, hgqa, synth, workloads, acc)
    if args.only in (None, "decode"):
        rec["decode"] = bench_decode(args, torch, hgqa, synth, workloads, acc)
    if args.only in (None, "chunk"):
        rec["chunked_prefill"] = bench_chunk(args, torch, hgqa, synth, workloads, acc)
    if cpu is not None:
        rec["cpu_baseline"] = cpu
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
