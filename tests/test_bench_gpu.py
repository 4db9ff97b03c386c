"""bench.py end to end on the GPU: one small workload through every pass,
and the JSON line the benchmark contract asks for."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line_small_workload():
    if os.environ.get("MXMOE_LIBRARY", "") not in ("", "product"):
        pytest.skip("bench.py measures the normal library only")
    print("case: bench.py uniform_T32_H4096_E256_k8", flush=True)
    proc = subprocess.run(
        [sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "1", "--steps", "3",
         "--warmup", "1", "--workload", "uniform_T32_H4096_E256_k8", "--cpu-seconds", "0.2"],
        cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stderr[-3000:]
    lines = [ln for ln in proc.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "workloads"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert abs(d["value"] - 32 / (d["ms_per_step"] * 1e-3)) / d["value"] < 1e-6
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == 8000.0 and r["unit"] == "GB/s"
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0
    assert set(c["legs"]["all_cores"]["stage_median_ms"]) == {"prepare", "dispatch", "combine"}
    head = d["headline"]
    for regime in ("cold", "warm"):
        for stage in ("e2e_ms", "dispatch_ms", "combine_ms"):
            st = head[regime][stage]
            assert st["samples"] == 5 * 3
            assert st["min"] <= st["p50"] <= st["p90"] <= st["p99"] <= st["p999"]
        assert head[regime]["e2e_reps"]["reps"] == 5
    assert d["workloads"]["uniform_T32_H4096_E256_k8"]["step_ms_cold"] == d["ms_per_step"]
    ref = d["reference_ops"]
    assert set(ref) == {"sum_over_k", "fill", "copy"}
    for name, op in ref.items():
        assert op["us"] > 0 and op["bytes"] > 0, name
        assert abs(op["frac"] - op["gbps"] / 8000.0) < 1e-9, name
    # T = 32, H = 4096, k = 8: the reduction moves the combine's bytes with bf16 output
    assert ref["sum_over_k"]["bytes"] == 32 * 8 * 4096 * 2 + 32 * 4096 * 2
    oc = d["workloads"]["uniform_T32_H4096_E256_k8"]
    assert oc["step_ms_cold_one_call_dispatch"] > 0 and oc["step_ms_warm_one_call_dispatch"] > 0
    assert oc["step_ms_warm_graph"] > 0 and oc["step_ms_warm_graph_one_call_dispatch"] > 0


def test_kernel_sweep_lines():
    if os.environ.get("MXMOE_LIBRARY", "") not in ("", "product"):
        pytest.skip("bench.py measures the normal library only")
    print("case: bench.py kernel sweep at T = 32 and 2048", flush=True)
    code = ("import bench; bench.kernel_sweep(sizes=(32, 2048), reps=2)")
    proc = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=300)
    assert proc.returncode == 0, proc.stderr[-3000:]
    rows = [json.loads(ln)["kernel_sweep"] for ln in proc.stdout.splitlines()
            if ln.startswith('{"kernel_sweep"')]
    calls = ("prepare_moe_input", "dispatch_rows", "shuffle_rows", "apply_shuffle_mul_sum")
    assert [(r["T"], r["call"]) for r in rows] == [(T, c) for T in (32, 2048) for c in calls]
    for r in rows:
        assert r["us_back_to_back"] > 0 and r["bytes"] > 0
        t = r["kernel_us"] if r["kernel_us"] is not None else r["us_back_to_back"]
        assert abs(r["gbps"] - r["bytes"] / t / 1e3) < 1e-6 * r["gbps"]
        assert (r["kernel_us"] is None) == (r["call"] == "shuffle_rows")
    # T = 2048, H = 7168, k = 8: combine reads 8 bf16 rows and writes one per token
    comb = [r for r in rows if r["T"] == 2048 and r["call"] == "apply_shuffle_mul_sum"][0]
    assert comb["bytes"] == 2048 * 8 * 7168 * 2 + 2048 * 7168 * 2 + 2048 * 8 * 8
