"""The five synthetic workloads, by name.

Shapes and routing follow the workloads the pages measure on:

* ``uniform_T32_H4096_E256_k8`` -- the Mooncake EP JIT page's test and
  performance configuration (BF16, 32 tokens, hidden 4096, top-8 of 256
  experts; section "Performance Test").
* ``uniform_T4096_H7168_E256_k8_pad128`` -- the EP benchmark RFC's CLI shape
  (hidden 7168, top-8, 4096 tokens; section "CLI Interface") with uniform
  routing and expert segments padded to 128 rows for a grouped GEMM.
* ``khot8_T8192_H7168_E256_k8`` -- K-hot incast of the same RFC ("Routing
  Modes", item 2): 8 hot experts, each pick hot with probability 0.8.
* ``zipf1.2_T16384_H4096fp8_E128_k8`` -- Zipfian routing ("Routing Modes",
  item 3, alpha 1.2) over 128 experts, FP8 e4m3 activations with one fp32
  scale per 1x128 block (the FP8 blockscale offsets of the sglang
  prepare_moe_input page), bf16 expert output.
* ``replica288_T65536_H7168_k8_f32out`` -- 256 experts plus 32 redundant
  slots (288 slots, TensorRT-LLM large-EP page, load_balancer num_slots),
  uniform routing, fp32 combine output.

No public dataset or benchmark suite is involved: these seeded inputs are the
workloads themselves.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

from . import routing


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int
    H: int
    E: int
    k: int
    mode: str                      # uniform | k_hot | zipf | replica
    x_dtype: str = "bf16"          # bf16 | fp8
    y_dtype: str = "bf16"
    out_dtype: str = "bf16"
    row_align: int = 1
    blockscale: bool = False
    params: dict = field(default_factory=dict)

    @property
    def scale_width(self) -> int:
        return self.H // 128 if self.x_dtype == "fp8" else 0

    @property
    def x_elem_bytes(self) -> int:
        return 1 if self.x_dtype == "fp8" else {"bf16": 2, "f16": 2, "f32": 4}[self.x_dtype]


WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("uniform_T32_H4096_E256_k8", 1, 32, 4096, 256, 8, "uniform"),
    Workload("uniform_T4096_H7168_E256_k8_pad128", 2, 4096, 7168, 256, 8, "uniform",
             row_align=128),
    Workload("khot8_T8192_H7168_E256_k8", 3, 8192, 7168, 256, 8, "k_hot",
             params={"n_hot": 8, "p_hot": 0.8}),
    Workload("zipf1.2_T16384_H4096fp8_E128_k8", 4, 16384, 4096, 128, 8, "zipf",
             x_dtype="fp8", blockscale=True, params={"s": 1.2}),
    Workload("replica288_T65536_H7168_k8_f32out", 5, 65536, 7168, 288, 8, "replica",
             out_dtype="f32", params={"n_experts": 256, "n_replicas": 32}),
]}


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}") from None


def routing_ids(w: Workload, rng: np.random.Generator, T: int | None = None) -> np.ndarray:
    T = w.T if T is None else T
    if w.mode == "uniform":
        return routing.uniform_topk(rng, T, w.E, w.k)
    if w.mode == "k_hot":
        return routing.k_hot_topk(rng, T, w.E, w.k, w.params["n_hot"], w.params["p_hot"])
    if w.mode == "zipf":
        return routing.zipf_topk(rng, T, w.E, w.k, w.params["s"])
    if w.mode == "replica":
        ids, _ = routing.replica_topk(rng, T, w.params["n_experts"], w.params["n_replicas"], w.k)
        return ids
    raise ValueError(w.mode)


def build_inputs(w: Workload, device: str | torch.device = "cpu", T: int | None = None,
                 seed: int | None = None) -> dict:
    """Routing ids (numpy int64 [T,k]), softmax weights (numpy float32 [T,k])
    and activations on ``device``: ``x`` [T,H] (bf16, or fp8 e4m3fn bytes plus
    ``scales`` [T,H/128] float32).  ``T`` overrides the token count (smaller
    parity cases of the same routing); ``seed`` overrides the workload seed."""
    T = w.T if T is None else T
    seed = w.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    ids = routing_ids(w, rng, T)
    weights = routing.softmax_weights(rng, T, w.k)
    out = {"ids": ids, "weights": weights, "scales": None}
    if w.x_dtype == "fp8":
        out["x"], out["scales"] = routing.fp8_blockscaled_rows(T, w.H, seed * 7919 + 1,
                                                               device=device)
    else:
        out["x"] = routing.normal_rows(T, w.H, w.x_dtype, seed * 7919 + 1, device=device)
    return out


def expert_output(w: Workload, rows: int, device: str | torch.device = "cpu",
                  seed: int | None = None) -> torch.Tensor:
    """Stand-in for the expert GEMM output: ``rows`` x H values from N(0,1)
    in the workload's expert-output dtype, seeded separately from ``x``."""
    seed = w.seed if seed is None else seed
    return routing.normal_rows(rows, w.H, w.y_dtype, seed * 7919 + 2, device=device)
