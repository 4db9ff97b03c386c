#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole hot path on one batch: prepare_moe_input (routing
metadata) -> dispatch_rows (token rows into expert-contiguous rows) ->
apply_shuffle_mul_sum (gather, weight, fp32 sum back to tokens).  Inputs are
seeded synthetic routing and activations, resident in HBM before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Prints one JSON line: tokens/s over the K timed steps (wall clock between
two device synchronisations); from a second pass of K steps, per-stage times
from HIP events recorded on the launch stream around each stage, and the
dispatch and combine kernels' own durations from HIP events recorded with
the kernels' begin and end timestamps; the dominant kernel's achieved
algorithmic HBM bandwidth against MI355X's 8 TB/s; and the CPU oracle timed
on a bounded sample of the same workload on the host.

--graph captures one step's launches in a HIP graph and times K replays of
it, so the headline holds no host launch cost (the per-stage event pass stays
eager).  --copy-probe BYTES times a plain device copy of BYTES bytes instead
(the reference kernel whose HBM counters calibrate the traffic figures).
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
DEFAULT_WORKLOAD = "uniform_T4096_H7168_E256_k8_pad128"
METRIC = "dispatch+combine tokens/s; achieved HBM GB/s vs MI355X peak"
KERNEL_SOURCES = ("route.hip", "rows.hip", "combine.hip", "device_common.h")


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so the
    hash changes with the code, not with its comments."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return re.sub(r"\s+", " ", text).strip()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "combine_topk_ids_expert_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=DEFAULT_WORKLOAD)
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="wall-clock budget of the CPU-oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a HIP graph of one step instead of eager launches")
    p.add_argument("--with", dest="extras", default="",
                   help="comma-separated extra stages added to each step and reported "
                        "separately: zero_padding (zero-fill the padding rows after "
                        "dispatch), output_memset (zero the output rows before combine), "
                        "moe_sort (tile-padded sort metadata over all experts, tiles of "
                        "row_align rows, after prepare), quantize_dispatch (bf16 rows "
                        "quantized to fp8 e4m3 with 1x128 scales and dispatched, after "
                        "dispatch)")
    return p.parse_args()


def algorithmic_bytes(w, n_valid: int, cap: int, id_bytes: int) -> dict:
    """Bytes each stage must move: every source row read once, every
    destination row written once, index and weight arrays once; padding
    rows are never touched."""
    T, k, E = w.T, w.k, w.E
    row = w.H * w.x_elem_bytes
    side = w.scale_width * 4
    y_b = {"bf16": 2, "f16": 2, "f32": 4}[w.y_dtype]
    o_b = {"bf16": 2, "f16": 2, "f32": 4}[w.out_dtype]
    prep = T * k * id_bytes + T * k * 4 + cap * 4 + E * 4 * 3 + E * 12 * 2
    disp = T * (row + side) + n_valid * (row + side) + T * k * 4
    comb = n_valid * w.H * y_b + T * w.H * o_b + T * k * 4 + T * k * 4
    return {"prepare": prep, "dispatch": disp, "combine": comb}


def load_traffic(workload: str, kernel: str) -> dict | None:
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3
    counter summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the same
    counter reads for a plain copy of known size), if it was taken on the
    current kernel sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel)


def cpu_baseline(w, inp, x, y, budget_s: float) -> dict:
    """The oracle, as it stands, on the same workload: whole steps (prepare,
    row gather, combine) repeated until the time budget is spent."""
    import numpy as np
    import torch
    import oracle

    ids = inp["ids"]
    x_bits = x.cpu().contiguous()
    x_bits = x_bits.view(torch.uint8).numpy()
    y_bits = y.cpu().view(torch.int16).numpy().view(np.uint16) if y.dtype != torch.float32 \
        else y.cpu().numpy()
    y_code = {"bf16": "bf16", "f16": "f16", "f32": "f32"}[w.y_dtype]
    steps, t_total = 0, 0.0
    while steps == 0 or (t_total < budget_s and steps < 50):
        t0 = time.perf_counter()
        m = oracle.prepare_moe_input(ids, w.E, row_align=w.row_align)
        oracle.shuffle_rows(x_bits, m["input_permutation"])
        oracle.apply_shuffle_mul_sum(y_bits, y_code, m["output_permutation"], inp["weights"],
                                     "f32", w.T, w.k, w.out_dtype)
        t_total += time.perf_counter() - t0
        steps += 1
    return {"value": w.T * steps / t_total, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{steps} whole step(s) of {w.name} (T={w.T}), single-threaded C oracle, "
                      f"{t_total:.1f} s"}


def copy_probe(nbytes: int, steps: int) -> None:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": nbytes, "steps": steps, "ms": dt * 1e3,
                      "gbps_read_plus_write": 2 * nbytes / dt / 1e9}), flush=True)


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return

    import combine_topk_ids_expert_amd as mx
    from workloads import get_workload, build_inputs
    from workloads.configs import expert_output

    w = get_workload(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = build_inputs(w, dev)
    T, k, E, H = w.T, w.k, w.E, w.H
    ids = torch.from_numpy(inp["ids"]).to(dev)
    weights = torch.from_numpy(inp["weights"]).to(dev)
    x, scales = inp["x"], inp["scales"]
    r = mx.empty_routing(T, k, E, dev, row_align=w.row_align, blockscale=w.blockscale)
    cap = r["input_permutation"].numel()
    xd = torch.empty((cap, H), dtype=x.dtype, device=dev)
    sd = torch.empty((cap, scales.shape[1]), dtype=torch.float32, device=dev) \
        if scales is not None else None
    y = expert_output(w, cap, dev)
    odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.out_dtype]
    out = torch.empty((T, H), dtype=odt, device=dev)
    stream = torch.cuda.current_stream(dev)

    def prepare():
        mx.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                             r["input_permutation"], r["output_permutation"], E, 2048, H,
                             r["blockscale_offsets"], row_align=w.row_align,
                             workspace=r["workspace"])

    def dispatch(kernel_events=None):
        mx.dispatch_rows(x, r["output_permutation"], k, xd, scales, sd,
                         kernel_events=kernel_events)

    def combine(kernel_events=None):
        mx.apply_shuffle_mul_sum(y, out, r["output_permutation"], weights,
                                 kernel_events=kernel_events)

    def zero_padding():
        mx.zero_padding_rows(xd, r["input_permutation"], r["expert_offsets"])

    def output_memset():
        mx.moe_output_memset(out, r["output_permutation"], k)

    sort_tile = max(w.row_align, 1)
    sort_out = {}
    sort_ws = torch.empty(max(mx.prepare_workspace_size(T, k, E), 4), dtype=torch.uint8,
                          device=dev)

    def moe_sort():
        sort_out.update(mx.moe_sort(ids, E, 0, E, sort_tile, out=sort_out or None,
                                    workspace=sort_ws))

    extras = [e for e in args.extras.split(",") if e]
    xq = sq = None
    if "quantize_dispatch" in extras:
        if x.dtype != torch.bfloat16 or H % 128:
            raise SystemExit("quantize_dispatch needs a bf16 workload with hidden % 128 == 0")
        xq = torch.empty((cap, H), dtype=torch.float8_e4m3fn, device=dev)
        sq = torch.empty((cap, H // 128), dtype=torch.float32, device=dev)

    def quantize_dispatch():
        mx.dispatch_rows_fp8(x, r["output_permutation"], k, xq, sq)

    known = {"zero_padding": zero_padding, "output_memset": output_memset, "moe_sort": moe_sort,
             "quantize_dispatch": quantize_dispatch}
    for e in extras:
        if e not in known:
            raise SystemExit(f"unknown --with stage {e!r}; known: {sorted(known)}")
    stages = [("prepare", prepare)]
    if "moe_sort" in extras:
        stages.append(("moe_sort", moe_sort))
    stages.append(("dispatch", dispatch))
    if "quantize_dispatch" in extras:
        stages.append(("quantize_dispatch", quantize_dispatch))
    if "zero_padding" in extras:
        stages.append(("zero_padding", zero_padding))
    if "output_memset" in extras:
        stages.append(("output_memset", output_memset))
    stages.append(("combine", combine))
    stages = tuple(stages)
    for _ in range(args.warmup):
        for _, fn in stages:
            fn()
    torch.cuda.synchronize()

    K = args.steps
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _, fn in stages:
                fn()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    # Headline: exactly K steps between two device synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(K):
            graph.replay()
    else:
        for _ in range(K):
            for _, fn in stages:
                fn()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Per-stage and per-kernel durations: a second pass of K steps (kept out of
    # the headline pass, since each event record adds a few microseconds
    # between kernels).  HIP events are recorded on the launch stream around
    # every stage; dispatch and combine also record a pair of events with
    # their kernels' own begin and end timestamps (the timed entry points).
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(K)]
    kev = {name: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(K)] for name in ("dispatch", "combine")}
    for pairs in kev.values():
        for a, b in pairs:                  # torch creates an event's HIP handle at its first record
            a.record(stream)
            b.record(stream)
    torch.cuda.synchronize()
    for s in range(K):
        ev[s][0].record(stream)
        for i, (name, fn) in enumerate(stages):
            if name in kev:
                fn(kernel_events=kev[name][s])
            else:
                fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    kernel_ms = {}
    for name, pairs in kev.items():
        ts = np.array([a.elapsed_time(b) for a, b in pairs])
        kernel_ms[name] = {"mean": float(ts.mean()), "p50": float(np.percentile(ts, 50)),
                           "p90": float(np.percentile(ts, 90)), "min": float(ts.min())}

    stage_ms = {}
    for i, (name, _) in enumerate(stages):
        ts = np.array([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)])
        stage_ms[name] = {"mean": float(ts.mean()), "p50": float(np.percentile(ts, 50)),
                          "p90": float(np.percentile(ts, 90)), "p99": float(np.percentile(ts, 99)),
                          "min": float(ts.min())}
    counts = r["problem_sizes1"][:, 0].cpu().numpy()
    n_valid = int(counts.sum())
    nbytes = algorithmic_bytes(w, n_valid, cap, ids.element_size())
    row_b = H * x.element_size()
    extra_report = {}
    if "zero_padding" in extras:
        padded = int(r["expert_offsets"][-1].item())
        nbytes["zero_padding"] = (padded - n_valid) * row_b + cap * 4
    if "output_memset" in extras:
        has_pick = (r["output_permutation"].view(T, k) >= 0).any(dim=1).sum().item()
        nbytes["output_memset"] = int(has_pick) * H * out.element_size() + T * k * 4
    if "quantize_dispatch" in extras:
        nbytes["quantize_dispatch"] = T * H * 2 + n_valid * (H + H // 128 * 4) + T * k * 4
    if "moe_sort" in extras:
        scap = sort_out["permuted_idx_to_expanded_idx"].numel()
        nbytes["moe_sort"] = (T * k * ids.element_size() + T * k * 4 + scap * 4
                              + 2 * 4 * sort_out["tile_idx_to_group_idx"].numel() + 4 * (E + 3))
    for e in extras:
        gbps = nbytes[e] / (stage_ms[e]["mean"] * 1e-3) / 1e9
        extra_report[e] = {"ms": stage_ms[e]["mean"], "algorithmic_bytes": nbytes[e],
                           "achieved_gbps": gbps, "frac": gbps / HBM_PEAK_GBPS}
    dom = max(("dispatch", "combine"), key=lambda n: kernel_ms[n]["mean"])
    kernel_name = {"dispatch": "dispatch_rows_kernel", "combine": "combine_vec_kernel"}[dom]
    achieved = nbytes[dom] / (kernel_ms[dom]["mean"] * 1e-3) / 1e9
    traffic = load_traffic(w.name, kernel_name)
    step_bytes = sum(nbytes.values())
    ms_per_step = elapsed / K * 1e3
    value = T * K / elapsed

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, x, y, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-e4m3 rows, bf16 combine"}.get(w.x_dtype, w.x_dtype),
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "H": H, "E": E, "topk": k, "routing": w.mode,
                   "row_align": w.row_align, "x_dtype": w.x_dtype, "out_dtype": w.out_dtype,
                   "launch": "hip_graph" if graph is not None else "eager"},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "traffic_detail": traffic, "bytes_per_launch": nbytes[dom],
                     "avg_launch_ms": kernel_ms[dom]["mean"],
                     "avg_launch_ms_source": "HIP events recorded with the kernel's own begin "
                                             "and end timestamps (hipExtLaunchKernel)",
                     "avg_stage_ms_events_between_launches": stage_ms[dom]["mean"]},
        "cpu_baseline": cpu,
        "stages_ms": stage_ms,
        "kernels_ms": kernel_ms,
        "extras": extra_report or None,
        "algorithmic_bytes": nbytes,
        "step_hbm_gbps": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "step_frac_of_peak": step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "expert_load": {"max": int(counts.max()), "min": int(counts.min()),
                        "mean": float(counts.mean()),
                        "imbalance_ratio": float(counts.max() / max(counts.mean(), 1e-9))},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
