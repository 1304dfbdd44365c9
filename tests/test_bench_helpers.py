"""The measurement code's own arithmetic, on the CPU: algorithmic work counts against
brute force over the tokens, the percentile summary, and the rule that a recorded HBM
traffic figure is used only while the kernel sources it was measured on are unchanged."""
import os

import numpy as np
import pytest

import bench
from workloads import make_batch


def _prefill_batch():
    return make_batch(B=5, Hq=8, Hkv=2, D=64, BS=16, dtype="bf16", scale=0.125, seed=3,
                      n_new=37, ctx_range=(0, 90), NB=256)


def test_prefill_flops_counts_each_visible_key_once():
    b = _prefill_batch()
    visible = 0
    for L, n in zip(b.context_lens.astype(int), b.n_new.astype(int)):
        c = L - n
        for t in range(n):            # query t of the chunk sees keys 0 .. c + t
            visible += c + t + 1
    assert bench.prefill_flops(b) == 4 * b.D * b.Hq * visible


def test_decode_byte_counts():
    b = make_batch(B=6, Hq=8, Hkv=4, D=128, BS=16, dtype="bf16", scale=0.088, seed=4,
                   lens_range=(1, 300), NB=512)
    rows = int(b.context_lens.sum())
    assert b.kv_bytes() == rows * b.Hkv * b.D * 2 * 2
    assert bench.int8_kv_bytes(b) == rows * b.Hkv * (b.D + 4) * 2   # codes + one fp32 scale per row
    T = len(b.slot_mapping)
    assert bench.rope_bytes(b) == T * (2 * b.Hq * b.D * 2 + 4 * b.Hkv * b.D * 2 + 2 * (b.D // 2) * 4)


def test_stats_summary():
    ms = np.linspace(0.1, 0.2, 11)          # 100 .. 200 us
    s = bench._stats_us(ms)
    assert s == {"n": 11, "mean": 150.0, "p10": 110.0, "p50": 150.0, "p90": 190.0}


def test_recorded_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// one version of a kernel\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sha = bench.kernel_source_sha(["kernel.hip"])
    (tmp_path / "s.md").write_text(f"text\n\nkernel_source_sha: {sha}\ntraffic_bytes_per_launch: 1234.5\n")
    assert bench.traffic_from("s.md", ["kernel.hip"]) == pytest.approx(1234.5)
    src.write_text("// the kernel changed\n")
    assert bench.traffic_from("s.md", ["kernel.hip"]) is None
    assert bench.traffic_from("missing.md", ["kernel.hip"]) is None


def test_committed_summaries_name_their_sources():
    """Every committed counter summary carries a hash and a traffic figure bench.py can read."""
    names = [n for n in os.listdir(bench.PROFILES) if n.endswith("_counters.md")]
    assert names
    for n in names:
        text = open(os.path.join(bench.PROFILES, n)).read()
        assert "kernel_source_sha: " in text and "traffic_bytes_per_launch: " in text, n
