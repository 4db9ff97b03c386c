"""Seeded routing generators and activation generators.

Routing modes follow the EP benchmark RFC "Comprehensive MoE / EP Kernel
Benchmark Under Incast Traffic", section "Routing Modes": uniform routing,
K-hot-expert incast (a hot set of low-numbered experts, as in its example hot
set 0..3, receiving a configurable share of picks) and Zipfian routing with an
exponent knob.  The redundant-slot mode follows the expert-slot layout of the
TensorRT-LLM page "Enable CuteDSL MoE with Large EP" (load balancer with 288
slots for 256 experts).

Every generator draws k *distinct* experts per token (a router's top-k never
repeats an expert) and returns int64 ids of shape [T, k], row-major, in the
order the picks were drawn.  Randomness comes only from the numpy Generator
passed in (ids, weights) or from a seeded torch Generator (activation values),
so a seed fixes every byte.
"""

from __future__ import annotations

import numpy as np
import torch


def _random_order_prefix(keys: np.ndarray, k: int) -> np.ndarray:
    """Columns of the k smallest keys per row, ordered by ascending key."""
    part = np.argpartition(keys, k - 1, axis=1)[:, :k] if k < keys.shape[1] else \
        np.tile(np.arange(keys.shape[1]), (keys.shape[0], 1))
    sub = np.take_along_axis(keys, part, axis=1)
    order = np.argsort(sub, axis=1, kind="stable")
    return np.take_along_axis(part, order, axis=1)


def uniform_topk(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """Each token picks k distinct experts uniformly from E, in random order.

    Uniform routing of the EP benchmark RFC (section "Routing Modes", item 1).
    """
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if T == 0:
        return np.zeros((0, k), dtype=np.int64)
    keys = rng.random((T, E))
    return _random_order_prefix(keys, k).astype(np.int64)


def k_hot_topk(rng: np.random.Generator, T: int, E: int, k: int,
               n_hot: int, p_hot: float) -> np.ndarray:
    """K-hot incast: experts 0..n_hot-1 are hot.

    For each pick in turn, with probability ``p_hot`` the pick is a hot
    expert chosen uniformly among the hot experts this token has not used
    yet, otherwise a cold expert chosen uniformly among the unused cold ones
    (EP benchmark RFC, "Routing Modes", item 2).  When a token has used every
    hot expert, further picks are cold; when it has used every cold expert,
    further picks are hot.
    """
    if not (1 <= k <= E and 0 <= n_hot <= E and 0.0 <= p_hot <= 1.0):
        raise ValueError("bad k_hot parameters")
    if T == 0:
        return np.zeros((0, k), dtype=np.int64)
    n_cold = E - n_hot
    want_hot = rng.random((T, k)) < p_hot
    hot_order = np.argsort(rng.random((T, max(n_hot, 1))), axis=1)[:, :n_hot]
    cold_order = np.argsort(rng.random((T, max(n_cold, 1))), axis=1)[:, :n_cold] + n_hot
    out = np.empty((T, k), dtype=np.int64)
    used_h = np.zeros(T, dtype=np.int64)
    used_c = np.zeros(T, dtype=np.int64)
    rows = np.arange(T)
    for j in range(k):
        take_hot = (want_hot[:, j] & (used_h < n_hot)) | (used_c >= n_cold)
        h_idx = np.minimum(used_h, max(n_hot - 1, 0))
        c_idx = np.minimum(used_c, max(n_cold - 1, 0))
        hot_pick = hot_order[rows, h_idx] if n_hot else np.zeros(T, dtype=np.int64)
        cold_pick = cold_order[rows, c_idx] if n_cold else np.zeros(T, dtype=np.int64)
        out[:, j] = np.where(take_hot, hot_pick, cold_pick)
        used_h += take_hot
        used_c += ~take_hot
    return out


def zipf_topk(rng: np.random.Generator, T: int, E: int, k: int, s: float) -> np.ndarray:
    """Zipfian routing: expert of popularity rank r has weight r**-s.

    Ranks are assigned to experts by a seeded random permutation.  The k
    distinct picks are drawn one after another, each from the weights of the
    experts not yet picked (Gumbel-top-k, which is the same distribution as
    successive renormalised draws).  EP benchmark RFC, "Routing Modes", item 3.
    """
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    rank_of_expert = rng.permutation(E) + 1
    logp = -s * np.log(rank_of_expert.astype(np.float64))
    if T == 0:
        return np.zeros((0, k), dtype=np.int64)
    gumbel = -np.log(-np.log(rng.random((T, E))))
    return _random_order_prefix(-(logp[None, :] + gumbel), k).astype(np.int64)


def replica_topk(rng: np.random.Generator, T: int, n_experts: int, n_replicas: int,
                 k: int) -> tuple[np.ndarray, np.ndarray]:
    """Uniform top-k over logical experts, mapped onto redundant expert slots.

    ``n_replicas`` logical experts (a seeded choice) get one extra slot each,
    numbered ``n_experts + i``.  A pick of a replicated expert goes to the
    original slot or to its replica with probability 1/2 each.  Returns the
    slot ids [T, k] and the logical expert of each replica slot.
    """
    if not 0 <= n_replicas <= n_experts:
        raise ValueError("bad replica count")
    logical = uniform_topk(rng, T, n_experts, k)
    replicated = np.sort(rng.choice(n_experts, size=n_replicas, replace=False))
    slot_of = np.full(n_experts, -1, dtype=np.int64)
    slot_of[replicated] = n_experts + np.arange(n_replicas)
    coin = rng.random(logical.shape) < 0.5
    rep = slot_of[logical]
    slots = np.where((rep >= 0) & coin, rep, logical)
    return slots.astype(np.int64), replicated.astype(np.int64)


def softmax_weights(rng: np.random.Generator, T: int, k: int) -> np.ndarray:
    """Router weights: softmax over the k picks of N(0,1) logits.

    Computed in float64 and stored as float32 [T, k].
    """
    logits = rng.standard_normal((T, k))
    if T == 0:
        return np.zeros((0, k), dtype=np.float32)
    z = logits - logits.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


_TORCH_DTYPES = {
    "bf16": torch.bfloat16,
    "f16": torch.float16,
    "f32": torch.float32,
}


def normal_rows(rows: int, width: int, dtype: str, seed: int,
                device: str | torch.device = "cpu") -> torch.Tensor:
    """[rows, width] values drawn from N(0,1) in float32, then converted by
    torch to ``dtype`` ("bf16", "f16" or "f32"), using a seeded generator on
    ``device``.  The same seed on a different device gives different values;
    callers that check results copy the tensor to the host instead of
    regenerating it."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(rows, width, generator=g, device=device, dtype=torch.float32)
    return t.to(_TORCH_DTYPES[dtype])


def fp8_blockscaled_rows(rows: int, width: int, seed: int, block: int = 128,
                         device: str | torch.device = "cpu") -> tuple[torch.Tensor, torch.Tensor]:
    """FP8 (OCP e4m3fn) activations with one float32 scale per 1 x ``block``
    block: values from N(0,1), ``scale = amax / 448`` per block, ``q = x /
    scale`` converted by torch to float8_e4m3fn.  Returns (q [rows, width],
    scales [rows, width // block] float32)."""
    if width % block:
        raise ValueError("width must be a multiple of the block")
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(rows, width // block, block, generator=g, device=device,
                    dtype=torch.float32)
    amax = x.abs().amax(dim=2)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (x / scale[:, :, None]).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.reshape(rows, width), scale.contiguous()
