"""Host logic of bench.py, no GPU: the algorithmic byte and flop counts the
rooflines divide by, the refusal of more than one GPU, and the lookup of
recorded HBM traffic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_algorithmic_counts_decode_shape():
    # 1 token, hidden 5120, intermediate 17408: 3 * 5120 * 17408 NVFP4
    # weights at 0.5625 B each, and 2 * (2 I H + H I) flops per token.
    a = bench.algorithmic(1, 5120, 17408, "w4a4", 2)
    weights = 3 * 5120 * 17408 * 9 // 16
    assert weights == 150_405_120
    assert a["flops"] == 534_773_760
    assert a["flops_fused"] == 2 * 2 * 17408 * 5120
    acts = a["total"] - weights
    # x bf16 read, x NVFP4 written + read, h NVFP4 written + read, out bf16
    assert acts == pytest.approx(5120 * 2 + 2 * 5120 * 0.5625 + 2 * 17408 * 0.5625 + 5120 * 2)
    assert a["fused"] == pytest.approx(2 * 17408 * 5120 * 0.5625 + (5120 + 17408) * 0.5625)


def test_algorithmic_counts_prefill_and_w4a16():
    a = bench.algorithmic(8192, 7168, 18432, "w4a4", 2)
    assert a["flops"] == 6_493_990_551_552
    b = bench.algorithmic(4096, 5120, 17408, "w4a16", 2)
    assert b["quant"] == 0
    assert b["flops"] == 4096 * 534_773_760
    # bf16 x and h, each written and read once across the two GEMMs
    assert b["total"] == pytest.approx(150_405_120 + 4096 * (5120 * 2 + 2 * 17408 * 2 + 5120 * 2))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout


def test_recorded_traffic_needs_matching_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    src = bench.kernel_source_hash()
    (prof / "k.md").write_text(
        "# summary\n"
        f"bench-traffic: workload=decode_w4a4 M=1 bytes_per_launch=123456 src={src}\n"
        "bench-traffic: workload=decode_w4a4 M=2 bytes_per_launch=777 src=0000000000000000\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # The kernel hash reads ROOT too: point it back at the real sources.
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: src)
    assert bench.recorded_traffic("decode_w4a4", 1) == 123456.0
    assert bench.recorded_traffic("decode_w4a4", 2) is None       # taken on other sources
    assert bench.recorded_traffic("prefill_w4a4", 8192) is None   # no line for it
