"""Routing-distribution validation of the seeded generators (no GPU).

The EP benchmark RFC ("Validation Plan", item 2) asks that uniform, K-hot and
Zipfian modes produce the expected expert-load distributions; these tests
check that, plus distinct picks per token, determinism under a seed, and the
weight and FP8 generators.
"""

import numpy as np
import pytest
import torch

from workloads import WORKLOADS, build_inputs, routing


def _distinct_rows(ids):
    s = np.sort(ids, axis=1)
    return np.all(s[:, 1:] != s[:, :-1])


def test_uniform_distribution():
    rng = np.random.default_rng(0)
    T, E, k = 20000, 64, 8
    ids = routing.uniform_topk(rng, T, E, k)
    assert ids.shape == (T, k) and ids.dtype == np.int64
    assert ids.min() >= 0 and ids.max() < E and _distinct_rows(ids)
    c = np.bincount(ids.ravel(), minlength=E)
    expect = T * k / E
    # each count is binomial-like with sd < sqrt(expect); 6 sd is a loose bound
    assert np.all(np.abs(c - expect) < 6 * np.sqrt(expect))
    # position j within a token is also uniform (the pick order is random)
    c0 = np.bincount(ids[:, 0], minlength=E)
    assert np.all(np.abs(c0 - T / E) < 6 * np.sqrt(T / E))


def test_k_hot_distribution():
    rng = np.random.default_rng(1)
    T, E, k, n_hot, p = 20000, 256, 8, 8, 0.8
    ids = routing.k_hot_topk(rng, T, E, k, n_hot, p)
    assert ids.min() >= 0 and ids.max() < E and _distinct_rows(ids)
    hot_share = np.mean(ids < n_hot)
    assert abs(hot_share - p) < 0.01
    c = np.bincount(ids.ravel(), minlength=E)
    hot_expect = T * k * p / n_hot
    assert np.all(np.abs(c[:n_hot] - hot_expect) < 6 * np.sqrt(hot_expect))
    cold_expect = T * k * (1 - p) / (E - n_hot)
    assert np.all(np.abs(c[n_hot:] - cold_expect) < 6 * np.sqrt(cold_expect) + 3)


def test_k_hot_extremes():
    rng = np.random.default_rng(2)
    ids = routing.k_hot_topk(rng, 500, 16, 4, 4, 1.0)      # every pick hot
    assert np.all(ids < 4) and _distinct_rows(ids)
    ids = routing.k_hot_topk(rng, 500, 16, 6, 4, 1.0)      # hot set exhausted -> cold
    assert _distinct_rows(ids) and np.all(np.sum(ids < 4, axis=1) == 4)
    ids = routing.k_hot_topk(rng, 500, 16, 4, 4, 0.0)      # never hot
    assert np.all(ids >= 4)


def test_zipf_distribution():
    rng = np.random.default_rng(3)
    T, E, k, s = 20000, 128, 8, 1.2
    ids = routing.zipf_topk(rng, T, E, k, s)
    assert ids.min() >= 0 and ids.max() < E and _distinct_rows(ids)
    c = np.bincount(ids.ravel(), minlength=E)
    # first picks follow the Zipf law exactly: p(rank r) = r^-s / H_{E,s}
    rng2 = np.random.default_rng(3)
    rank_of_expert = rng2.permutation(E) + 1
    p = rank_of_expert.astype(float) ** -s
    p /= p.sum()
    first = np.bincount(ids[:, 0], minlength=E) / T
    assert np.abs(first - p).max() < 0.01
    # heavier experts get more load overall
    order = np.argsort(rank_of_expert)
    top, tail = c[order[:8]].mean(), c[order[-64:]].mean()
    assert top > 10 * tail


def test_replica_slots():
    rng = np.random.default_rng(4)
    T, n_exp, n_rep, k = 20000, 256, 32, 8
    slots, replicated = routing.replica_topk(rng, T, n_exp, n_rep, k)
    assert slots.min() >= 0 and slots.max() < n_exp + n_rep
    logical = np.where(slots >= n_exp, replicated[np.clip(slots - n_exp, 0, n_rep - 1)], slots)
    assert _distinct_rows(logical)
    c = np.bincount(slots.ravel(), minlength=n_exp + n_rep)
    per_copy = T * k / n_exp / 2
    assert np.all(np.abs(c[replicated] - per_copy) < 6 * np.sqrt(per_copy))
    assert np.all(np.abs(c[n_exp:] - per_copy) < 6 * np.sqrt(per_copy))


def test_softmax_weights():
    rng = np.random.default_rng(5)
    w = routing.softmax_weights(rng, 1000, 8)
    assert w.dtype == np.float32 and np.all(w > 0)
    assert np.abs(w.astype(np.float64).sum(1) - 1).max() < 1e-6


def test_fp8_blockscaled():
    q, sc = routing.fp8_blockscaled_rows(8, 512, seed=3)
    assert q.dtype == torch.float8_e4m3fn and sc.shape == (8, 4)
    qf = q.float()
    assert qf.abs().max() <= 448 and torch.all(sc > 0)
    g = torch.Generator().manual_seed(3)
    x = torch.randn(8, 4, 128, generator=g)
    deq = (qf.reshape(8, 4, 128) * sc[:, :, None])
    # e4m3 keeps 3 fraction bits: relative error <= 2^-4 for normal values
    assert torch.all((deq - x).abs() <= x.abs() * 2 ** -4 + sc[:, :, None] * 2 ** -9)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workloads_deterministic(name):
    w = WORKLOADS[name]
    T = min(w.T, 256)
    a = build_inputs(w, "cpu", T=T)
    b = build_inputs(w, "cpu", T=T)
    np.testing.assert_array_equal(a["ids"], b["ids"])
    np.testing.assert_array_equal(a["weights"], b["weights"])
    assert torch.equal(a["x"].view(torch.uint8), b["x"].view(torch.uint8))
    assert a["ids"].shape == (T, w.k) and _distinct_rows(a["ids"])
    assert a["ids"].max() < w.E
    c = build_inputs(w, "cpu", T=T, seed=w.seed + 100)
    assert not np.array_equal(a["ids"], c["ids"])
