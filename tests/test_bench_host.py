"""Host-side logic of bench.py: the roofline arithmetic, the source-hash gate on the
committed counter traffic, and the single-GPU refusal.  No GPU work runs here."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_block_arithmetic():
    peaks = {"mfma_bf16_tflops": 2000.0, "mfma_fp8_tflops": 4000.0, "stream_read_gbs": 7000.0}
    # 1e15 flops in 1000 ms = 1000 TFLOP/s; 7e12 bytes in 1 s = 7000 GB/s
    b = bench.roofline_block("k", 1e15, 1000.0, "bf16", peaks, traffic=7e12)
    assert b["achieved"] == pytest.approx(1000.0)
    assert b["frac"] == pytest.approx(1000.0 / bench.PEAK_BF16_TFLOPS)
    assert b["frac_measured"] == pytest.approx(0.5)
    assert b["traffic_gbs"] == pytest.approx(7000.0)
    assert b["traffic_frac_hbm_peak"] == pytest.approx(7000.0 / bench.PEAK_HBM_GBS)
    assert b["traffic_frac_stream_measured"] == pytest.approx(1.0)
    f = bench.roofline_block("k", 1e15, 1000.0, "fp8", {}, traffic=None)
    assert f["frac"] == pytest.approx(1000.0 / bench.PEAK_FP8_TFLOPS)
    assert f["peak_measured"] is None and f["traffic"] is None and "traffic_gbs" not in f


def test_counter_traffic_follows_the_attention_source():
    src = os.path.join(ROOT, "block_sparse_long_pooled_amd", "csrc", "attn.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for name in ("attn_128k_bf16_counters.txt", "attn_256k_fp8_counters.txt"):
        text = open(os.path.join(ROOT, "profiles", name)).read()
        fields = dict(line.split(":", 1) for line in text.splitlines() if ":" in line and not line.startswith("#"))
        expected = float(fields["attn_traffic_bytes"])
        got = bench.counter_traffic(name)
        if fields["attn_kernel_source_sha256"].strip() == sha:
            assert got == expected
        else:  # counters taken on another kernel source are never reported
            assert got is None
    assert bench.counter_traffic("no_such_profile.txt") is None


def test_counter_traffic_rejects_a_stale_profile(tmp_path, monkeypatch):
    # a copy of the repository layout whose profile names another source hash
    (tmp_path / "profiles").mkdir()
    (tmp_path / "block_sparse_long_pooled_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "block_sparse_long_pooled_amd" / "csrc" / "attn.hip").write_text("// kernel\n")
    sha = hashlib.sha256(b"// kernel\n").hexdigest()
    (tmp_path / "profiles" / "fresh.txt").write_text(f"# x\nattn_kernel_source_sha256: {sha}\nattn_traffic_bytes: 123\n")
    (tmp_path / "profiles" / "stale.txt").write_text(f"attn_kernel_source_sha256: {'0' * 64}\nattn_traffic_bytes: 123\n")
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.counter_traffic("fresh.txt") == 123.0
    assert bench.counter_traffic("stale.txt") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "single-GPU" in line["error"]
