"""Host logic of bench.py, on the CPU: the multi-GPU refusal, the algorithmic
flop count it divides by, and the rule that it reports the counter-measured HBM
traffic only while the kernel sources are the ones the counters were taken on."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_flops_of_the_workloads():
    # 4 D Hq B s(s+1)/2: every causal (query head, key) pair scored once and multiplied into V once
    assert bench.prefill_flops(1, 131072, 32) == 140738562097152.0
    assert bench.prefill_flops(1, 65536, 16) == 17592454479872.0
    assert bench.prefill_flops(1, 2048, 1) == 4 * 128 * 2048 * 2049 / 2
    # the 128K workload is the one the headline is quoted on: g = 4 at L = 32768
    wid, b, s, hq, hkv, big_l, w, base = bench.WORKLOADS["qwen3_8b_128k"]
    assert (b, s, hq, hkv, big_l, w, base) == (1, 131072, 32, 8, 32768, 4096, 1e6)


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    value = bench.measured_traffic()
    assert value is not None and value > 0, "the committed summary must match the committed sources"
    # a copy of the tree's sources and summary: matching hashes give the value ...
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    csrc = root / "zero_shot_rope_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    for name in ("jl_prefill.hip", "jl_device.h"):
        shutil.copy(os.path.join(ROOT, "zero_shot_rope_attention_amd", "csrc", name), csrc / name)
    summary = root / "profiles" / os.path.basename(bench.TRAFFIC_FILE)
    shutil.copy(bench.TRAFFIC_FILE, summary)
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(summary))
    assert bench.measured_traffic() == value
    # ... and any change to a hashed source makes it null
    with open(csrc / "jl_device.h", "a") as f:
        f.write("\n// changed\n")
    assert bench.measured_traffic() is None
    # as does a summary without hashes
    summary.write_text("traffic_bytes_per_launch: 123\n")
    assert bench.measured_traffic() is None
