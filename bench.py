#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole hot path on one batch: prepare_moe_input (routing
metadata) -> dispatch_rows (token rows into expert-contiguous rows) ->
apply_shuffle_mul_sum (gather, weight, fp32 sum back to tokens).  Inputs are
seeded synthetic routing and activations, resident in HBM before timing.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

Prints one JSON line.  The headline workload is the largest one that fits one
GPU (T = 65536 tokens, hidden 7168, 288 expert slots, fp32 output); with the
default ``--workload all`` the other four workloads ride along in the same
line under ``workloads``.  Each workload is timed three ways, each over 5
repetitions of exactly K steps between two device synchronisations:

  cold  -- before every step, outside the timed interval, 512 MiB are written
           and then 1 GiB is read, which evicts the 256 MB Infinity Cache and
           the L2s and leaves only clean lines behind; each step is timed by an
           event pair recorded on the stream around its three calls.
           ``value`` and ``ms_per_step`` are the cold figures.
  warm  -- K steps back to back with one event pair around the K steps (the
           figure a pipeline that keeps its data resident would see; a step's
           deferred write-backs land in the next step, so they are counted);
           per-step percentiles from a second pass with an event pair around
           each step.

Event pairs around every step add about 3 us per step to what back-to-back
steps take (T = 4096 on MI355X); the timed entry points, whose events carry
the kernels' own begin and end timestamps, add more gaps between kernels, so
they run in passes of their own and give only the kernel times: the stages
of the benchmark RFC page, dispatch = prepare_moe_input + dispatch_rows
kernels and combine = apply_shuffle_mul_sum's kernel.  Every pass runs 5
repetitions; reported are the mean over repetitions, the spread of the
repetition means, and p50 / p90 / p99 / p999 over all steps.

The roofline is the dominant row kernel's algorithmic bytes per launch over
its mean cold kernel time, against 8 TB/s.  ``cpu_baseline`` times the CPU
oracle on a bounded token sample of the headline workload, on one thread and
on the host's cores (the row loops split over threads; routing stays one
thread, as it is defined).

--graph captures one step in a HIP graph and adds a warm figure of K graph
replays.  --copy-probe BYTES times a plain device copy instead.  --calibrate
runs the two row kernels on identity maps (T tokens of 14 KiB rows, k = 8,
T = 16384 unless --calibrate-tokens: every row read once and written once, in
order), the known byte counts that scale the L2-to-fabric counters of the
traffic figures, and a sequential-write reference for the kernel times.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "dispatch+combine tokens/s; achieved HBM GB/s vs MI355X peak"
HEADLINE = "replica288_T65536_H7168_k8_f32out"
# headline first, then the other workloads carried in the same line
ORDER = (HEADLINE, "uniform_T4096_H7168_E256_k8_pad128", "khot8_T8192_H7168_E256_k8",
         "zipf1.2_T16384_H4096fp8_E128_k8", "uniform_T32_H4096_E256_k8")
REPS = 5
# Workloads of at most this many picks also time the step with routing and
# dispatch in one prepare_dispatch call (the library runs both in one launch
# up to 2048 picks when the rows allow it).
ONE_CALL_MAX_PICKS = 2048
# Steps per HIP graph in the graph-replay passes.
GRAPH_STEPS = 20
FLUSH_WRITE_BYTES = 512 << 20
FLUSH_READ_BYTES = 1 << 30
KERNEL_SOURCES = ("route.hip", "rows.hip", "combine.hip", "device_common.h")
KERNEL_NAMES = {"dispatch": "dispatch_rows_kernel", "combine": "combine_vec_kernel"}


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


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50, help="steps per repetition")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="all",
                   help="'all' (headline plus the other workloads) or one workload name")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="wall-clock budget of each leg of the CPU-oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-reference-ops", action="store_true",
                   help="skip the PyTorch reference kernels timed over the headline's bytes")
    p.add_argument("--copy-probe", type=int, default=0, metavar="BYTES")
    p.add_argument("--calibrate", action="store_true",
                   help="run dispatch_rows and apply_shuffle_mul_sum on identity maps "
                        "(known bytes, for counter calibration) and print them")
    p.add_argument("--calibrate-tokens", type=int, default=16384,
                   help="tokens of the --calibrate run (rows of 14 KiB, k = 8)")
    p.add_argument("--calibrate-out", choices=("bf16", "f32"), default="bf16",
                   help="combine output dtype of the --calibrate run")
    p.add_argument("--one-call-sweep", action="store_true",
                   help="time routing + dispatch as prepare_dispatch (one call) against "
                        "prepare_moe_input + dispatch_rows (two calls) at decode-sized batches, "
                        "eager and as HIP-graph replays, and print one JSON line per size")
    p.add_argument("--kernel-sweep", action="store_true",
                   help="each call alone at T = 32 to 65536 (H = 7168): us, GB/s, fraction of peak")
    p.add_argument("--routing-sweep", action="store_true",
                   help="time prepare_moe_input alone at T = 128 to 4096 under several routings "
                        "and print one JSON line per case")
    p.add_argument("--graph", action="store_true",
                   help="also time the step replayed from a HIP graph of 20 steps (warm) on "
                        "workloads of more than 2048 picks (smaller ones always do)")
    p.add_argument("--with", dest="extras", default="",
                   help="comma-separated extra stages added to each step of the first "
                        "workload and reported separately: zero_padding (zero-fill the "
                        "padding rows after dispatch), output_memset (zero the output rows "
                        "before combine), moe_sort (tile-padded sort metadata over all "
                        "experts, tiles of row_align rows, after prepare), quantize_dispatch "
                        "(bf16 rows quantized to fp8 e4m3 with 1x128 scales and dispatched, "
                        "after dispatch)")
    return p.parse_args(argv)


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


def gate_ms(w, step_bytes: int):
    """Step time at 70% of 8 TB/s for the gated workloads (T >= 4096 and
    hidden 7168), else None."""
    if w.T >= 4096 and w.H == 7168:
        return step_bytes / (0.7 * HBM_PEAK_GBPS * 1e9) * 1e3
    return None


def load_traffic(workload: str, kernel: str) -> dict | None:
    """L2-to-fabric bytes per launch of ``kernel`` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by the
    factors of a calibration kernel), if it was taken on the current kernel
    sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("kernels", {}).get(kernel)


def stats(values) -> dict:
    """mean, p50 / p90 / p99 / p999 and min over all samples (ms)."""
    import numpy as np
    a = np.asarray(values, dtype=np.float64)
    return {"mean": float(a.mean()), "p50": float(np.percentile(a, 50)),
            "p90": float(np.percentile(a, 90)), "p99": float(np.percentile(a, 99)),
            "p999": float(np.percentile(a, 99.9)), "min": float(a.min()),
            "samples": int(a.size)}


def rep_stats(per_rep) -> dict:
    """Mean over repetitions of the repetition means, and their spread."""
    import numpy as np
    m = np.array([float(np.mean(r)) for r in per_rep])
    return {"mean": float(m.mean()), "rep_means": [float(x) for x in m],
            "rep_spread": float(m.max() - m.min()), "reps": int(m.size)}


# ---- CPU baseline -----------------------------------------------------------

def host_description() -> dict:
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": avail, "os_cpu_count": os.cpu_count()}


def cpu_baseline(w, budget_s: float, dev) -> dict:
    """The oracle, as it stands, on a bounded sample of the workload: the
    same routing, hidden size and dtypes with fewer tokens.  One step of the
    sample = prepare_moe_input over its picks (one thread, as defined), the
    row gather into expert-contiguous rows, and the combine.  Timed on one
    thread and with the row loops split over the host's cores (threads call
    the C oracle, which releases the GIL), each leg repeated until its budget
    is spent."""
    import numpy as np
    import torch
    import oracle
    from workloads import build_inputs
    from workloads.configs import expert_output

    host = host_description()
    threads = max(1, min(host["nproc"], 16))
    legs = {}
    for name, n_threads, t_sample in (("single_thread", 1, min(w.T, 2048)),
                                      ("all_cores", threads, min(w.T, 8192))):
        inp = build_inputs(w, dev, T=t_sample)
        ids = inp["ids"]
        m = oracle.prepare_moe_input(ids, w.E, row_align=w.row_align)
        rows = len(m["input_permutation"])
        x = inp["x"]
        x_host = x.cpu().contiguous().view(torch.uint8).numpy().reshape(t_sample, -1)
        y = expert_output(w, rows, dev)
        y_host = (y.cpu().view(torch.int16).numpy().view(np.uint16) if y.dtype != torch.float32
                  else y.cpu().numpy())
        del x, y
        torch.cuda.empty_cache()
        xd = np.zeros((rows, x_host.shape[1]), np.uint8)
        out = {}

        def rows_part(r0, r1, perm):
            oracle.shuffle_rows(x_host, perm[r0:r1], dst=xd[r0:r1])

        def comb_part(t0, t1, perm):
            out[t0] = oracle.apply_shuffle_mul_sum(
                y_host, w.y_dtype, perm[t0 * w.k:t1 * w.k], inp["weights"][t0:t1], "f32",
                t1 - t0, w.k, w.out_dtype)

        def run_split(fn, n, perm):
            if n_threads == 1:
                fn(0, n, perm)
                return
            bounds = [n * i // n_threads for i in range(n_threads + 1)]
            ts = [threading.Thread(target=fn, args=(bounds[i], bounds[i + 1], perm))
                  for i in range(n_threads) if bounds[i + 1] > bounds[i]]
            for t in ts:
                t.start()
            for t in ts:
                t.join()

        steps, t_total = 0, 0.0
        stage_s = {"prepare": [], "dispatch": [], "combine": []}
        while steps == 0 or (t_total < budget_s and steps < 20):
            t0 = time.perf_counter()
            m = oracle.prepare_moe_input(ids, w.E, row_align=w.row_align)
            t1 = time.perf_counter()
            run_split(rows_part, rows, m["input_permutation"])
            t2 = time.perf_counter()
            run_split(comb_part, t_sample, m["output_permutation"])
            t3 = time.perf_counter()
            stage_s["prepare"].append(t1 - t0)
            stage_s["dispatch"].append(t2 - t1)
            stage_s["combine"].append(t3 - t2)
            t_total += t3 - t0
            steps += 1
        legs[name] = {"value": t_sample * steps / t_total, "threads": n_threads,
                      "sample_tokens": t_sample, "steps": steps, "seconds": t_total,
                      "stage_median_ms": {k: float(np.median(v)) * 1e3
                                          for k, v in stage_s.items()}}
    allc = legs["all_cores"]
    return {"value": allc["value"], "unit": "tokens/s", "cores": allc["threads"],
            "kind": "oracle",
            "sample": (f"{w.name} routing, hidden and dtypes with T = {allc['sample_tokens']} "
                       f"tokens ({legs['single_thread']['sample_tokens']} on one thread); whole "
                       f"steps: prepare (one thread), row gather and combine split over "
                       f"threads; {allc['steps']} steps on {allc['threads']} threads, "
                       f"{legs['single_thread']['steps']} on one"),
            "single_thread_value": legs["single_thread"]["value"], "legs": legs, **host}


# ---- GPU measurement ----------------------------------------------------------

class Flusher:
    """Evicts the Infinity Cache and the L2s: writes 512 MiB, then reads
    1 GiB of other memory, so the written lines are written back during the
    flush and only clean lines stay cached."""

    def __init__(self, dev):
        import torch
        self.w = torch.empty(FLUSH_WRITE_BYTES, dtype=torch.uint8, device=dev)
        self.r = torch.ones(FLUSH_READ_BYTES // 4, dtype=torch.int32, device=dev)
        self.n = 0

    def __call__(self):
        self.n += 1
        self.w.fill_(self.n & 0xff)
        self.r.max()


class Step:
    """Buffers and bound calls of one step of workload ``w``."""

    def __init__(self, w, dev, extras=()):
        import torch
        import combine_topk_ids_expert_amd as mx
        from workloads import build_inputs
        from workloads.configs import expert_output

        self.w = w
        inp = build_inputs(w, dev)
        T, k, E, H = w.T, w.k, w.E, w.H
        self.ids = torch.from_numpy(inp["ids"]).to(dev)
        self.weights = torch.from_numpy(inp["weights"]).to(dev)
        x, scales = inp["x"], inp["scales"]
        r = mx.empty_routing(T, k, E, dev, row_align=w.row_align, blockscale=w.blockscale)
        self.r = r
        self.cap = r["input_permutation"].numel()
        xd = torch.empty((self.cap, H), dtype=x.dtype, device=dev)
        sd = (torch.empty((self.cap, scales.shape[1]), dtype=torch.float32, device=dev)
              if scales is not None else None)
        y = expert_output(w, self.cap, dev)
        odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.out_dtype]
        out = torch.empty((T, H), dtype=odt, device=dev)
        self.x, self.xd, self.y, self.out = x, xd, y, out
        self.prepare = mx.bind(mx.prepare_moe_input, self.ids, r["expert_offsets"],
                               r["problem_sizes1"], r["problem_sizes2"], r["input_permutation"],
                               r["output_permutation"], E, 2048, H, r["blockscale_offsets"],
                               row_align=w.row_align, workspace=r["workspace"])
        self.dispatch = mx.bind(mx.dispatch_rows, x, r["output_permutation"], k, xd, scales, sd)
        # routing and dispatch as one call (one launch where the library fuses them)
        self.prepare_dispatch = mx.bind(
            mx.prepare_dispatch, self.ids, r["expert_offsets"], r["problem_sizes1"],
            r["problem_sizes2"], r["input_permutation"], r["output_permutation"], E, 2048, H, x,
            xd, r["blockscale_offsets"], side_input=scales, side_output=sd,
            row_align=w.row_align, workspace=r["workspace"])
        self.combine = mx.bind(mx.apply_shuffle_mul_sum, y, out, r["output_permutation"],
                               self.weights)
        self.extras = []
        self.extra_bytes = {}
        row_b = H * x.element_size()
        for e in extras:
            if e == "zero_padding":
                fn = mx.bind(mx.zero_padding_rows, xd, r["input_permutation"],
                             r["expert_offsets"])
            elif e == "output_memset":
                fn = mx.bind(mx.moe_output_memset, out, r["output_permutation"], k)
            elif e == "moe_sort":
                sort_ws = torch.empty(max(mx.prepare_workspace_size(T, k, E), 16),
                                      dtype=torch.uint8, device=dev)
                sort_out = mx.moe_sort(self.ids, E, 0, E, max(w.row_align, 1), workspace=sort_ws)
                self._sort = (sort_out, sort_ws)

                def fn(so=sort_out, ws=sort_ws):
                    mx.moe_sort(self.ids, E, 0, E, max(w.row_align, 1), out=so, workspace=ws)
            elif e == "quantize_dispatch":
                if x.dtype != torch.bfloat16 or H % 128:
                    raise SystemExit("quantize_dispatch needs a bf16 workload with hidden % 128 == 0")
                xq = torch.empty((self.cap, H), dtype=torch.float8_e4m3fn, device=dev)
                sq = torch.empty((self.cap, H // 128), dtype=torch.float32, device=dev)
                fn = mx.bind(mx.dispatch_rows_fp8, x, r["output_permutation"], k, xq, sq)
            else:
                raise SystemExit(f"unknown --with stage {e!r}; known: zero_padding, "
                                 "output_memset, moe_sort, quantize_dispatch")
            self.extras.append((e, fn))
        self.row_b = row_b

    def run(self):
        self.prepare()
        for name, fn in self.extras:
            if name == "moe_sort":
                fn()
        self.dispatch()
        for name, fn in self.extras:
            if name in ("quantize_dispatch", "zero_padding", "output_memset"):
                fn()
        self.combine()

    def run_one_call_dispatch(self):
        """The step with routing and dispatch through prepare_dispatch."""
        self.prepare_dispatch()
        self.combine()

    def run_timed(self, ev):
        """The step through the timed entry points; ev = six events (prepare,
        dispatch and combine kernel begin / end).  Extra stages run plain."""
        self.prepare(kernel_events=(ev[0], ev[1]))
        for name, fn in self.extras:
            if name == "moe_sort":
                fn()
        self.dispatch(kernel_events=(ev[2], ev[3]))
        for name, fn in self.extras:
            if name in ("quantize_dispatch", "zero_padding", "output_memset"):
                fn()
        self.combine(kernel_events=(ev[4], ev[5]))


def _events(n):
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:              # torch creates an event's HIP handle at its first record
        e.record()
    return evs


def steps_pass(run, K: int, flush) -> dict:
    """REPS repetitions of K steps with an event pair around each step; with
    ``flush`` the caches are evicted before every step, outside the pair.
    Per-rep lists of step times (ms) and the host's clock per step."""
    import torch
    evs = [_events(2) for _ in range(K)]
    out = {"e2e": [], "wall_per_step": []}
    for _ in range(REPS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(K):
            if flush is not None:
                flush()
            evs[s][0].record()
            run()
            evs[s][1].record()
        torch.cuda.synchronize()
        out["wall_per_step"].append((time.perf_counter() - t0) / K * 1e3)
        out["e2e"].append([a.elapsed_time(b) for a, b in evs])
    return out


def kernels_pass(step: Step, K: int, flush) -> dict:
    """REPS repetitions of K steps through the timed entry points (caches
    evicted before every step with ``flush``): each kernel's own duration."""
    import torch
    evs = [_events(6) for _ in range(K)]
    out = {"prepare_kernel": [], "dispatch_kernel": [], "combine_kernel": []}
    for _ in range(REPS):
        torch.cuda.synchronize()
        for s in range(K):
            if flush is not None:
                flush()
            step.run_timed(evs[s])
        torch.cuda.synchronize()
        out["prepare_kernel"].append([e[0].elapsed_time(e[1]) for e in evs])
        out["dispatch_kernel"].append([e[2].elapsed_time(e[3]) for e in evs])
        out["combine_kernel"].append([e[4].elapsed_time(e[5]) for e in evs])
    return out


def warm_pass(run, K: int) -> dict:
    """REPS repetitions of K back-to-back steps, one event pair around each
    repetition, and the host's clock between the two synchronisations."""
    import torch
    a, b = _events(2)
    per_rep, wall = [], []
    for _ in range(REPS):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record()
        for _ in range(K):
            run()
        b.record()
        torch.cuda.synchronize()
        wall.append((time.perf_counter() - t0) / K * 1e3)
        per_rep.append([a.elapsed_time(b) / K])
    return {"per_rep": per_rep, "wall": wall}


def extras_pass(step: Step, K: int) -> dict:
    """Stage events around every stage of the step (extra stages included),
    warm, for the extra stages' times."""
    import torch
    names = ["prepare"] + [n for n, _ in step.extras if n == "moe_sort"] + ["dispatch"] + \
        [n for n, _ in step.extras if n != "moe_sort"] + ["combine"]
    fns = dict(step.extras)
    fns.update(prepare=step.prepare, dispatch=step.dispatch, combine=step.combine)
    ev = [_events(len(names) + 1) for _ in range(K)]
    torch.cuda.synchronize()
    for s in range(K):
        ev[s][0].record()
        for i, n in enumerate(names):
            fns[n]()
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    return {n: [ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(K)]
            for i, n in enumerate(names)}


def measure(w, args, dev, flush, extras=()) -> dict:
    import numpy as np
    import torch

    step = Step(w, dev, extras)
    K = args.steps
    for _ in range(args.warmup):
        step.run()
    torch.cuda.synchronize()
    cold = steps_pass(step.run, K, flush)
    cold_k = kernels_pass(step, K, flush)
    warm = warm_pass(step.run, K)
    warm_s = steps_pass(step.run, K, None)
    warm_k = kernels_pass(step, K, None)
    small = w.T * w.k <= ONE_CALL_MAX_PICKS
    one_call = None
    if small:
        one_call = (steps_pass(step.run_one_call_dispatch, K, flush),
                    warm_pass(step.run_one_call_dispatch, K))

    def graph_pass(fn):
        # One graph holds GRAPH_STEPS steps, so a replay's own launch cost is
        # spread over them; per-step times divide by it.
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(GRAPH_STEPS):
                fn()
        for _ in range(max(args.warmup // GRAPH_STEPS, 1)):
            g.replay()
        reps = max(K // GRAPH_STEPS, 1)
        r = warm_pass(g.replay, reps)
        return {"per_rep": [[v / GRAPH_STEPS for v in rep] for rep in r["per_rep"]],
                "wall": [v / GRAPH_STEPS for v in r["wall"]]}

    # Small workloads are bound by host time per call; replaying steps from a
    # HIP graph shows what the GPU takes.
    graph = graph_pass(step.run) if args.graph or small else None
    graph_one = graph_pass(step.run_one_call_dispatch) if small else None

    counts = step.r["problem_sizes1"][:, 0].cpu().numpy()
    n_valid = int(counts.sum())
    nbytes = algorithmic_bytes(w, n_valid, step.cap, step.ids.element_size())
    step_bytes = sum(nbytes.values())
    T = w.T

    def flat(per_rep):
        return [v for r in per_rep for v in r]

    def kernels(kp: dict) -> dict:
        kp_ = {k: flat(v) for k, v in kp.items()}
        kd, kc = stats(kp_["dispatch_kernel"]), stats(kp_["combine_kernel"])
        dom = "dispatch" if kd["mean"] >= kc["mean"] else "combine"
        kdom = kd if dom == "dispatch" else kc
        gbps = nbytes[dom] / (kdom["mean"] * 1e-3) / 1e9
        return {
            "prepare_kernel_ms": stats(kp_["prepare_kernel"]), "dispatch_kernel_ms": kd,
            "combine_kernel_ms": kc,
            # the RFC page's stages: dispatch = routing + row dispatch, combine
            "dispatch_ms": stats([p + d for p, d in zip(kp_["prepare_kernel"],
                                                        kp_["dispatch_kernel"])]),
            "combine_ms": kc,
            "dominant_kernel": KERNEL_NAMES[dom], "dominant_stage": dom,
            "dominant_kernel_gbps": gbps, "dominant_kernel_frac": gbps / HBM_PEAK_GBPS,
            "row_kernels_frac": (nbytes["dispatch"] + nbytes["combine"])
                                / ((kd["mean"] + kc["mean"]) * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        }

    def summary(steps: dict, kp: dict, label: str, mean_ms=None) -> dict:
        e2e = stats(flat(steps["e2e"]))
        ms = e2e["mean"] if mean_ms is None else mean_ms
        return {
            "cache": label,
            "step_ms": ms, "tokens_per_s": T / (ms * 1e-3),
            "step_gbps": step_bytes / (ms * 1e-3) / 1e9,
            "step_frac": step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "e2e_ms": e2e, "e2e_reps": rep_stats(steps["e2e"]),
            "host_wall_ms_per_step": float(np.mean(steps["wall_per_step"])),
            **kernels(kp),
        }

    res = {
        "workload": w.name, "T": T, "H": w.H, "E": w.E, "topk": w.k, "routing": w.mode,
        "row_align": w.row_align, "x_dtype": w.x_dtype, "out_dtype": w.out_dtype,
        "algorithmic_bytes": nbytes, "step_bytes": step_bytes,
        "cold": summary(cold, cold_k, "cold: 512 MiB written and 1 GiB read before each "
                                      "step, outside the event pair around the step"),
        "expert_load": {"max": int(counts.max()), "min": int(counts.min()),
                        "mean": float(counts.mean()),
                        "imbalance_ratio": float(counts.max() / max(counts.mean(), 1e-9))},
    }
    wm = rep_stats(warm["per_rep"])
    res["warm"] = summary(warm_s, warm_k, "warm: K steps back to back; step_ms from one event "
                                          "pair around each repetition, e2e percentiles from "
                                          "a pass with a pair around each step",
                          mean_ms=wm["mean"])
    res["warm"]["reps"] = wm
    res["warm"]["host_wall_ms_per_step_back_to_back"] = float(np.mean(warm["wall"]))
    wm = wm["mean"]
    if one_call is not None:
        oc = stats(flat(one_call[0]["e2e"]))["mean"]
        ow = rep_stats(one_call[1]["per_rep"])["mean"]
        res["one_call_dispatch"] = {
            "what": "the same step with routing and dispatch in one prepare_dispatch call (one "
                    "launch where the library fuses them), then combine",
            "step_ms_cold": oc, "tokens_per_s_cold": T / (oc * 1e-3),
            "step_ms_warm": ow, "tokens_per_s_warm": T / (ow * 1e-3),
            "warm_reps": rep_stats(one_call[1]["per_rep"])}
    if graph is not None:
        gm = rep_stats(graph["per_rep"])["mean"]
        res["warm_graph"] = {"what": "steps replayed back to back from a HIP graph of "
                                     f"{GRAPH_STEPS} steps",
                             "step_ms": gm, "tokens_per_s": T / (gm * 1e-3),
                             "reps": rep_stats(graph["per_rep"])}
    if graph_one is not None:
        go = rep_stats(graph_one["per_rep"])["mean"]
        res["warm_graph_one_call_dispatch"] = {
            "what": f"steps replayed from a HIP graph of {GRAPH_STEPS} steps, routing and "
                    "dispatch in one prepare_dispatch call", "step_ms": go,
            "tokens_per_s": T / (go * 1e-3),
            "reps": rep_stats(graph_one["per_rep"])}
    g = gate_ms(w, step_bytes)
    if g is not None:
        res["gate_70pct"] = {"step_ms_max": g, "met_cold": res["cold"]["step_ms"] <= g,
                             "met_warm": wm <= g}
    if step.extras:
        ex = extras_pass(step, K)
        row_b = step.row_b
        extra_b = {}
        for e, _ in step.extras:
            if e == "zero_padding":
                padded = int(step.r["expert_offsets"][-1].item())
                extra_b[e] = (padded - n_valid) * row_b + step.cap * 4
            elif e == "output_memset":
                has_pick = (step.r["output_permutation"].view(T, w.k) >= 0).any(dim=1).sum().item()
                extra_b[e] = int(has_pick) * w.H * step.out.element_size() + T * w.k * 4
            elif e == "quantize_dispatch":
                extra_b[e] = T * w.H * 2 + n_valid * (w.H + w.H // 128 * 4) + T * w.k * 4
            elif e == "moe_sort":
                so = step._sort[0]
                scap = so["permuted_idx_to_expanded_idx"].numel()
                extra_b[e] = (T * w.k * step.ids.element_size() + T * w.k * 4 + scap * 4
                              + 2 * 4 * so["tile_idx_to_group_idx"].numel() + 4 * (w.E + 3))
        res["extras"] = {e: {"ms": float(np.mean(ex[e])), "algorithmic_bytes": extra_b[e],
                             "frac": extra_b[e] / (float(np.mean(ex[e])) * 1e-3) / 1e9
                             / HBM_PEAK_GBPS} for e, _ in step.extras}
    res["_cap"] = step.cap
    del step
    torch.cuda.empty_cache()
    return res


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


def reference_ops(w, dev, steps: int = 10, reps: int = 3) -> dict:
    """PyTorch's own kernels over the byte counts of workload ``w``, timed
    with events on the current stream (median of ``reps`` means over
    ``steps`` launches), as ceilings measured on the same GPU beside the
    published 8 TB/s: the combine's bytes as a reduction over k contiguous
    rows (bf16 in, the combine's output dtype out), a fill of a buffer the
    size of the dispatch output (writes only) and a device copy of half of it
    (read + write).  None of this is the library's code."""
    import torch
    T, k, H = w.T, w.k, w.H
    odt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.out_dtype]
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev).normal_()
    out = torch.empty((T, H), dtype=odt, device=dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def time_op(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            ev[0].record()
            for _ in range(steps):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            ms.append(ev[0].elapsed_time(ev[1]) / steps)
        return sorted(ms)[len(ms) // 2]

    res = {}

    def add(name, ms, nbytes, what):
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"us": ms * 1e3, "bytes": nbytes, "gbps": gbps,
                     "frac": gbps / HBM_PEAK_GBPS, "what": what}

    yv = y.view(T, k, H)
    ms = time_op(lambda: torch.sum(yv, dim=1, dtype=odt, out=out))
    add("sum_over_k", ms, y.numel() * 2 + out.numel() * out.element_size(),
        "torch.sum of [T, k, H] bf16 over k into the combine's output dtype: the combine's "
        "bytes, with a token's k rows contiguous")
    ms = time_op(lambda: y.fill_(0.5))
    add("fill", ms, y.numel() * 2, "torch fill_ of a buffer the size of the dispatch output")
    half = (T * k) // 2
    src, dst = y[:half], y[half:2 * half]
    ms = time_op(lambda: dst.copy_(src))
    add("copy", ms, 2 * src.numel() * 2, "torch device copy of half that buffer (read + write)")
    del y, out, yv, src, dst
    torch.cuda.empty_cache()
    return res


def one_call_sweep(sizes=(1, 8, 32, 64, 128, 192, 256), hiddens=(4096, 7168), E=256, k=8,
                   calls=200, reps=5) -> None:
    """prepare_dispatch against prepare_moe_input + dispatch_rows on uniform
    routing, bf16 rows: microseconds per call pair, the minimum over ``reps``
    means of ``calls`` bound calls back to back (eager, host included), and
    of graphs of 20 call pairs replayed (GPU time only)."""
    import numpy as np
    import torch
    import combine_topk_ids_expert_amd as mx
    from workloads import routing
    dev = torch.device("cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def per_call(fn, n, div=1):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            ev[0].record()
            for _ in range(n):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            best = min(best, ev[0].elapsed_time(ev[1]) * 1e3 / (n * div))
        return best

    for H in hiddens:
        for T in sizes:
            ids = torch.from_numpy(routing.uniform_topk(np.random.default_rng(T), T, E, k)).to(dev)
            x = routing.normal_rows(T, H, "bf16", seed=T, device=dev)
            r = mx.empty_routing(T, k, E, dev)
            xd = torch.empty((r["input_permutation"].numel(), H), dtype=x.dtype, device=dev)
            meta = (ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                    r["input_permutation"], r["output_permutation"], E, 2048, H)
            one = mx.bind(mx.prepare_dispatch, *meta, x, xd, workspace=r["workspace"])
            prep = mx.bind(mx.prepare_moe_input, *meta, workspace=r["workspace"])
            disp = mx.bind(mx.dispatch_rows, x, r["output_permutation"], k, xd)

            def two():
                prep()
                disp()

            graphs = []
            for fn in (one, two):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for _ in range(20):
                        fn()
                graphs.append(g)
            print(json.dumps({"one_call_sweep": {
                "T": T, "H": H, "E": E, "topk": k,
                "eager_one_call_us": per_call(one, calls), "eager_two_calls_us": per_call(two, calls),
                "graph_one_call_us": per_call(graphs[0].replay, 10, 20),
                "graph_two_calls_us": per_call(graphs[1].replay, 10, 20)}}), flush=True)


KERNEL_SWEEP = (32, 128, 512, 2048, 8192, 32768, 65536)


def kernel_sweep(sizes=KERNEL_SWEEP, H=7168, E=256, k=8, reps=5) -> None:
    """Each call of the path alone, from decode-sized batches to the largest
    workload: uniform routing over E experts, bf16 rows of H, fp32 weights,
    bf16 combine output.  Per call: microseconds back to back (bound calls on
    one stream, the minimum over ``reps`` means; data left in the caches by
    the previous call of the same kind stays there where it fits), and the
    kernels' own time from the timed entry points (median of single calls)
    where the call has one.  GB/s and the fraction of 8 TB/s use the
    algorithmic bytes of the call (shuffle_rows: those of the dispatch it
    equals)."""
    import types
    import numpy as np
    import torch
    import combine_topk_ids_expert_amd as mx
    from workloads import routing
    dev = torch.device("cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    kev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in kev:
        e.record()
    torch.cuda.synchronize()

    def back_to_back(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            ev[0].record()
            for _ in range(n):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            best = min(best, ev[0].elapsed_time(ev[1]) * 1e3 / n)
        return best

    def kernel_time(fn):
        us = []
        for _ in range(4 * reps):
            fn(kernel_events=kev)
            torch.cuda.synchronize()
            us.append(kev[0].elapsed_time(kev[1]) * 1e3)
        return float(np.median(us))

    for T in sizes:
        rng = np.random.default_rng(T)
        ids = torch.from_numpy(routing.uniform_topk(rng, T, E, k)).to(dev)
        wts = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(dev)
        x = routing.normal_rows(T, H, "bf16", seed=T, device=dev)
        r = mx.empty_routing(T, k, E, dev)
        cap = r["input_permutation"].numel()
        xd = torch.empty((cap, H), dtype=x.dtype, device=dev)
        y = routing.normal_rows(cap, H, "bf16", seed=T + 1, device=dev)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        calls = {
            "prepare_moe_input": mx.bind(mx.prepare_moe_input, ids, r["expert_offsets"],
                                         r["problem_sizes1"], r["problem_sizes2"],
                                         r["input_permutation"], r["output_permutation"], E,
                                         2048, H, workspace=r["workspace"]),
            "dispatch_rows": mx.bind(mx.dispatch_rows, x, r["output_permutation"], k, xd),
            "shuffle_rows": mx.bind(mx.shuffle_rows, x, r["input_permutation"], xd),
            "apply_shuffle_mul_sum": mx.bind(mx.apply_shuffle_mul_sum, y, out,
                                             r["output_permutation"], wts),
        }
        calls["prepare_moe_input"]()
        torch.cuda.synchronize()
        w = types.SimpleNamespace(T=T, k=k, E=E, H=H, x_elem_bytes=2, scale_width=0,
                                  y_dtype="bf16", out_dtype="bf16")
        ab = algorithmic_bytes(w, T * k, cap, 8)
        nbytes = {"prepare_moe_input": ab["prepare"], "dispatch_rows": ab["dispatch"],
                  "shuffle_rows": ab["dispatch"], "apply_shuffle_mul_sum": ab["combine"]}
        n = max(10, min(200, 20000 // T))
        for name, fn in calls.items():
            us = back_to_back(fn, n)
            kus = kernel_time(fn) if name != "shuffle_rows" else None
            t = kus if kus is not None else us
            print(json.dumps({"kernel_sweep": {
                "call": name, "T": T, "H": H, "E": E, "topk": k, "bytes": nbytes[name],
                "us_back_to_back": us, "kernel_us": kus,
                "gbps": nbytes[name] / t / 1e3, "frac": nbytes[name] / t / 1e3 / HBM_PEAK_GBPS}}),
                flush=True)
        del calls, x, xd, y, out, r
        torch.cuda.empty_cache()


ROUTING_SWEEP = [  # (T, E, k, row_align, routing)
    (128, 256, 8, 1, "uniform"), (300, 256, 8, 1, "uniform"), (512, 256, 8, 1, "uniform"),
    (1024, 256, 8, 1, "uniform"), (1024, 256, 8, 128, "uniform"), (1024, 256, 8, 1, "k_hot"),
    (1024, 128, 8, 1, "zipf"), (1024, 1024, 8, 1, "uniform"), (1000, 8, 8, 1, "dups"),
    (1000, 1, 8, 1, "dups"), (1025, 256, 8, 1, "uniform"), (2048, 256, 8, 1, "uniform"),
    (2048, 256, 8, 1, "k_hot"), (4096, 256, 8, 128, "uniform")]


def routing_sweep(calls=200, reps=5) -> None:
    """prepare_moe_input alone, bound and called back to back on one stream:
    microseconds per call, the minimum and median of ``reps`` means of
    ``calls`` calls, for the cases of ROUTING_SWEEP (seeded ids)."""
    import numpy as np
    import torch
    import combine_topk_ids_expert_amd as mx
    from workloads import routing
    dev = torch.device("cuda:0")
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for T, E, k, A, mode in ROUTING_SWEEP:
        rng = np.random.default_rng(T * 31 + E)
        if mode == "uniform":
            ids = routing.uniform_topk(rng, T, E, k)
        elif mode == "k_hot":
            ids = routing.k_hot_topk(rng, T, E, k, 8, 0.8)
        elif mode == "zipf":
            ids = routing.zipf_topk(rng, T, E, k, 1.2)
        else:
            ids = rng.integers(0, E, (T, k))
        t_ids = torch.from_numpy(ids).to(dev)
        r = mx.empty_routing(T, k, E, dev, row_align=A)
        call = mx.bind(mx.prepare_moe_input, t_ids, r["expert_offsets"], r["problem_sizes1"],
                       r["problem_sizes2"], r["input_permutation"], r["output_permutation"], E,
                       2048, 7168, row_align=A, workspace=r["workspace"])
        for _ in range(20):
            call()
        torch.cuda.synchronize()
        us = []
        for _ in range(reps):
            ev[0].record()
            for _ in range(calls):
                call()
            ev[1].record()
            torch.cuda.synchronize()
            us.append(ev[0].elapsed_time(ev[1]) * 1e3 / calls)
        us.sort()
        print(json.dumps({"routing_sweep": {"T": T, "E": E, "topk": k, "row_align": A,
                                            "routing": mode, "picks": T * k,
                                            "us_min": us[0], "us_median": us[len(us) // 2]}}),
              flush=True)


CALIBRATE_K, CALIBRATE_H = 8, 7168


def calibrate(steps: int, T: int, out_dtype: str = "bf16") -> None:
    """The row kernels on identity maps: dispatch reads T rows and writes
    token t to rows t*k .. t*k+k-1; combine reads those T*k rows once each
    (unit fp32 weights) and writes T rows.  Prints the algorithmic bytes of each
    launch, which the FETCH_SIZE / WRITE_SIZE counters of the same launches
    are divided by."""
    import torch
    import combine_topk_ids_expert_amd as mx
    from workloads import routing
    k, H = CALIBRATE_K, CALIBRATE_H
    dev = torch.device("cuda:0")
    x = routing.normal_rows(T, H, "bf16", 7, device=dev)
    perm = torch.arange(T * k, dtype=torch.int32, device=dev)
    xd = torch.empty((T * k, H), dtype=torch.bfloat16, device=dev)
    ob = 4 if out_dtype == "f32" else 2
    out = torch.empty((T, H), dtype=torch.float32 if ob == 4 else torch.bfloat16, device=dev)
    ones = torch.ones((T, k), dtype=torch.float32, device=dev)
    disp = mx.bind(mx.dispatch_rows, x, perm, k, xd)
    # fp32 unit weights: the same kernel instantiation as the benchmark's combine
    comb = mx.bind(mx.apply_shuffle_mul_sum, xd, out, perm, ones)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in evs:
        e.record()
    td, tc = [], []
    for _ in range(steps):
        disp(kernel_events=(evs[0], evs[1]))
        comb(kernel_events=(evs[2], evs[3]))
        torch.cuda.synchronize()
        td.append(evs[0].elapsed_time(evs[1]))
        tc.append(evs[2].elapsed_time(evs[3]))
    row = H * 2
    print(json.dumps({"calibrate": {
        "dispatch_rows_kernel": {"read_bytes": T * row + T * k * 4, "write_bytes": T * k * row},
        "combine_vec_kernel": {"read_bytes": T * k * row + T * k * 8, "write_bytes": T * H * ob},
        "launches": steps, "tokens": T,
        "kernel_ms": {"dispatch_rows_kernel": sorted(td)[len(td) // 2],
                      "combine_vec_kernel": sorted(tc)[len(tc) // 2]}}}), flush=True)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("MXMOE_LIBRARY", "") not in ("", "product"):
        print("bench.py measures libmxmoe.so: unset MXMOE_LIBRARY (the test builds are "
              "not the measured library)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(args.copy_probe, max(args.steps, 1))
        return
    if args.calibrate:
        calibrate(max(args.steps, 1), args.calibrate_tokens, args.calibrate_out)
        return
    if args.one_call_sweep:
        one_call_sweep()
        return
    if args.routing_sweep:
        routing_sweep()
        return
    if args.kernel_sweep:
        kernel_sweep()
        return

    from workloads import get_workload

    names = ORDER if args.workload == "all" else (args.workload,)
    ws = [get_workload(n) for n in names]
    extras = [e for e in args.extras.split(",") if e]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = Flusher(dev)
    results = []
    for i, w in enumerate(ws):
        print(f"bench: {w.name} ...", file=sys.stderr, flush=True)
        results.append(measure(w, args, dev, flush, extras if i == 0 else ()))
    head, w = results[0], ws[0]
    del flush
    torch.cuda.empty_cache()

    cold = head["cold"]
    dom = cold["dominant_stage"]
    kernel_name = KERNEL_NAMES[dom]
    kms = cold["dispatch_kernel_ms" if dom == "dispatch" else "combine_kernel_ms"]["mean"]
    achieved = head["algorithmic_bytes"][dom] / (kms * 1e-3) / 1e9
    traffic = load_traffic(w.name, kernel_name)

    ref_ops = None
    if not args.no_reference_ops:
        print("bench: reference ops ...", file=sys.stderr, flush=True)
        ref_ops = reference_ops(w, dev)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, args.cpu_seconds, dev)

    def brief(r):
        c, wm = r["cold"], r["warm"]
        b = {"step_ms_cold": c["step_ms"], "tokens_per_s_cold": c["tokens_per_s"],
             "step_frac_cold": c["step_frac"], "step_ms_warm": wm["step_ms"],
             "tokens_per_s_warm": wm["tokens_per_s"], "step_frac_warm": wm["step_frac"],
             "dominant_kernel": c["dominant_kernel"],
             "dominant_kernel_frac_cold": c["dominant_kernel_frac"],
             "dominant_kernel_frac_warm": wm["dominant_kernel_frac"],
             "row_kernels_frac_cold": c["row_kernels_frac"],
             "row_kernels_frac_warm": wm["row_kernels_frac"]}
        if "gate_70pct" in r:
            b["gate_70pct"] = r["gate_70pct"]
        if "one_call_dispatch" in r:
            b["step_ms_cold_one_call_dispatch"] = r["one_call_dispatch"]["step_ms_cold"]
            b["step_ms_warm_one_call_dispatch"] = r["one_call_dispatch"]["step_ms_warm"]
        if "warm_graph" in r:
            b["step_ms_warm_graph"] = r["warm_graph"]["step_ms"]
        if "warm_graph_one_call_dispatch" in r:
            b["step_ms_warm_graph_one_call_dispatch"] = r["warm_graph_one_call_dispatch"]["step_ms"]
        return b

    for r in results:
        r.pop("_cap", None)
    line = {
        "metric": METRIC,
        "value": cold["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": cold["step_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "fp8-e4m3 rows, bf16 combine"}.get(w.x_dtype, w.x_dtype),
        "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "H": w.H, "E": w.E, "topk": w.k,
                   "routing": w.mode, "row_align": w.row_align, "x_dtype": w.x_dtype,
                   "out_dtype": w.out_dtype, "launch": "eager",
                   "cache": "cold (value, ms_per_step); warm beside it",
                   "repetitions": REPS},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": traffic["traffic_bytes"] if traffic else None,
                     "traffic_meaning": "bytes between the L2s and the fabric (FETCH_SIZE + "
                                        "WRITE_SIZE, calibrated); Infinity Cache hits count "
                                        "too, so these are not HBM bytes",
                     "traffic_detail": traffic,
                     "bytes_per_launch": head["algorithmic_bytes"][dom],
                     "avg_launch_ms": kms,
                     "avg_launch_ms_source": "HIP events recorded with the kernel's own begin "
                                             "and end timestamps (hipExtLaunchKernel), cold steps"},
        "timing_note": "value / ms_per_step: mean over 5 repetitions of K cold steps, each "
                       "timed by an event pair around its three calls (adds about 3 us per "
                       "step); kernel times from separate passes through the timed entry "
                       "points",
        "cpu_baseline": cpu,
        "reference_ops": ref_ops,
        "warm": {"ms_per_step": head["warm"]["step_ms"],
                 "tokens_per_s": head["warm"]["tokens_per_s"],
                 "step_frac_of_peak": head["warm"]["step_frac"]},
        "step_frac_of_peak": cold["step_frac"],
        "headline": head,
        "workloads": {r["workload"]: brief(r) for r in results},
        "workload_detail": {r["workload"]: r for r in results[1:]},
        "kernel_source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
