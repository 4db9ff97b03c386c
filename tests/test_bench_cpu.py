"""bench.py's contract on the host (no GPU): the one-GPU rule, the byte
accounting of its roofline, and the source hash that keys the counters."""

import os
import subprocess
import sys

import pytest

import bench
from workloads import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# Algorithmic MB per step (dispatch, combine) of each workload, all ids valid:
# dispatch reads every token row once and writes it to its k rows (+ the fp32
# 1x128 scale rows of the fp8 workload) and reads T*k int32 row indices;
# combine reads the T*k expert rows, writes T output rows and reads T*k
# indices and T*k fp32 weights.  Worked out by hand from the shapes.
EXPECTED_MB = {
    "uniform_T32_H4096_E256_k8": (2.360, 2.361),
    "uniform_T4096_H7168_E256_k8_pad128": (528.61, 528.74),
    "khot8_T8192_H7168_E256_k8": (1057.23, 1057.49),
    "zipf1.2_T16384_H4096fp8_E128_k8": (623.38, 1209.01),
    "replica288_T65536_H7168_k8_f32out": (8457.81, 9399.44),
}


@pytest.mark.parametrize("name", sorted(EXPECTED_MB))
def test_algorithmic_bytes_match_hand_count(name):
    w = WORKLOADS[name]
    n = w.T * w.k
    b = bench.algorithmic_bytes(w, n, n, 8)
    disp, comb = EXPECTED_MB[name]
    assert b["dispatch"] / 1e6 == pytest.approx(disp, abs=0.01)
    assert b["combine"] / 1e6 == pytest.approx(comb, abs=0.01)


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr


def test_source_hash_ignores_comments_and_whitespace():
    a = "int f(int x) {  // add one\n    return x + 1; /* done */\n}\n"
    b = "int f(int x)\n{\n\treturn x + 1;\n}"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(b.replace("1", "2"))


def test_stats_and_gate():
    s = bench.stats([1.0, 2.0, 3.0, 4.0])
    assert s["mean"] == 2.5 and s["min"] == 1.0 and s["samples"] == 4
    assert s["p50"] == 2.5 and s["p999"] <= 4.0
    r = bench.rep_stats([[1.0, 3.0], [2.0, 2.0], [4.0, 4.0]])
    assert r["rep_means"] == [2.0, 2.0, 4.0] and r["rep_spread"] == 2.0
    assert r["mean"] == pytest.approx(8.0 / 3.0)
    # 70% of 8 TB/s: the T = 4096 workload's 1.058 GB give about 189 us
    w = WORKLOADS["uniform_T4096_H7168_E256_k8_pad128"]
    assert bench.gate_ms(w, 1_057_971_200) == pytest.approx(0.18892, abs=1e-4)
    assert bench.gate_ms(WORKLOADS["uniform_T32_H4096_E256_k8"], 10**6) is None
    assert bench.gate_ms(WORKLOADS["zipf1.2_T16384_H4096fp8_E128_k8"], 10**9) is None


def test_cpu_baseline_legs_on_the_host():
    """The oracle timed on one thread and on the host's cores, on a bounded
    sample; routing stays single-threaded, the row loops split."""
    w = WORKLOADS["uniform_T32_H4096_E256_k8"]
    r = bench.cpu_baseline(w, 0.2, "cpu")
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s"
    assert r["legs"]["single_thread"]["threads"] == 1
    assert r["cores"] == r["legs"]["all_cores"]["threads"] >= 1
    assert r["value"] > 0 and r["single_thread_value"] > 0
    assert r["nproc"] >= 1 and isinstance(r["cpu_model"], str)
