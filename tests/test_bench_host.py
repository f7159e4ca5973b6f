"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
committed counter summaries it prices traffic from."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_source_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    csrc = tmp_path / "full_gqa_attention_layer_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("int f(int x) {\n  return x + 1;  // one\n}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.source_hash(["a.hip"])
    (csrc / "a.hip").write_text("/* note */ int f(int x) { return x + 1; }\n")
    assert bench.source_hash(["a.hip"]) == h0
    (csrc / "a.hip").write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash(["a.hip"]) != h0


def test_committed_traffic_summaries_match_the_kernels():
    """Each committed HBM-byte summary was taken on the kernel sources as they
    are now, so the bench line reports its traffic instead of null."""
    cases = [("attn_prefill_muse_full_traffic.json", bench.PREFILL_SOURCES),
             ("attn_decode_full_traffic.json", bench.DECODE_SOURCES),
             ("attn_decode_sliding_traffic.json", bench.DECODE_SOURCES)]
    for name, sources in cases:
        with open(os.path.join(bench.PROFILES, name)) as f:
            rec = json.load(f)
        assert rec["source_hash"] == bench.source_hash(sources), name
        assert bench.load_traffic(name, sources) == rec["hbm_bytes_per_launch"] > 0
