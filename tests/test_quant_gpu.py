"""Dispatch with FP8 quantization on the GPU against the oracle, bit for bit:
codes and scales of every dispatched row (needs the GPU)."""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu
from workloads import WORKLOADS, routing
from workloads.configs import routing_ids

pytestmark = pytest.mark.gpu
DEV = gu.DEV


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16)


def _check(x: torch.Tensor, ids: np.ndarray, E: int, A: int):
    T, H = x.shape
    k = ids.shape[1]
    meta = gu.check_prepare(ids, E, A)
    t = meta["_t"]
    rows = t["input_permutation"].numel()
    q = torch.full((rows, H), 0x55, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows, H // 128), -3.0, dtype=torch.float32, device=DEV)
    mx.dispatch_rows_fp8(x.to(DEV), t["output_permutation"], k, q, sc)
    torch.cuda.synchronize()
    xq, xs = oracle.quantize_fp8_rows(x.view(torch.int16).cpu().numpy().view(np.uint16))
    inp = meta["input_permutation"]
    used = inp >= 0
    want_q = oracle.shuffle_rows(xq, inp)
    want_s = oracle.shuffle_rows(xs, inp)
    got_q, got_s = q.cpu().numpy(), sc.cpu().numpy()
    np.testing.assert_array_equal(got_q[used], want_q[used])
    np.testing.assert_array_equal(got_s[used], want_s[used])
    assert np.all(got_q[~used] == 0x55) and np.all(got_s[~used] == -3.0)


@pytest.mark.parametrize("T,H,E,k,A", [
    (1, 128, 4, 1, 1),
    (37, 4096, 64, 8, 128),
    (100, 7168, 256, 8, 1),
    (20, 20480, 16, 4, 1),          # 1280 threads per row: two column chunks
    (9, 384, 8, 2, 1),              # three groups: a partly live wave
    (30, 256, 40, 70, 1),           # topk > 64
])
def test_fp8_dispatch_random(T, H, E, k, A):
    print("case: fp8 dispatch", T, H, E, k, A, flush=True)
    rng = np.random.default_rng(T * H + k)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x *= 10.0 ** rng.uniform(-6, 6, (T, H // 128, 1)).repeat(128, axis=2).reshape(T, H)
    ids = routing.uniform_topk(rng, T, E, k) if k <= E else rng.integers(-1, E + 1, (T, k))
    _check(_bf16(x), ids, E, A)


def test_fp8_dispatch_edge_groups():
    """All-zero groups (scale 1), groups of bf16 subnormals only, signed
    zeros, and exact e4m3 ties: with amax 448 the scale is 1 and values such
    as 1 + 2^-4 sit halfway between neighbouring e4m3 codes."""
    print("case: fp8 dispatch edges", flush=True)
    H = 128 * 6
    x = np.zeros((3, H), np.float32)
    x[0, 128:256] = np.float32(2.0 ** -130) * np.arange(1, 129)       # bf16 subnormals
    x[0, 256:384] = -0.0
    mids = np.array([1.0625, 1.1875, 2.125, 3.25, 0.015625 * 1.5, 0.001953125 * 1.5,
                     -1.0625, -2.375, 13.0, 208.0, 0.0029296875, 448.0], np.float32)
    x[1, 384:512] = np.resize(mids, 128)
    x[1, 384] = 448.0
    x[2] = np.linspace(-5, 5, H, dtype=np.float32)
    ids = np.array([[0, 1], [1, 2], [2, 0]], np.int64)
    _check(_bf16(x), ids, 3, 1)


def test_fp8_dispatch_nan_and_inf():
    """Non-finite inputs, same reading on both sides: amax skips NaN, a NaN
    element codes to 0x7f; an infinite element makes the group's scale
    infinite, so its finite elements code to signed zero and the infinite
    ones (inf / inf) to 0x7f; a group of NaN only has amax 0 and scale 1."""
    print("case: fp8 dispatch nan/inf", flush=True)
    H = 128 * 5
    x = np.linspace(-3, 3, 2 * H, dtype=np.float32).reshape(2, H)
    x[0, 5] = np.nan                              # group 0: NaN among normals
    x[0, 130] = np.inf                            # group 1: +inf
    x[0, 260] = -np.inf                           # group 2: -inf
    x[0, 300] = np.nan
    x[1, 384:512] = np.nan                        # group 3 of row 1: NaN only
    ids = np.array([[0, 2], [1, 0]], np.int64)
    _check(_bf16(x), ids, 3, 1)


def test_fp8_dispatch_full_size_zipf_bf16():
    """The Zipf workload's shape at full size (T = 16384, H = 4096, E = 128,
    top-8) with bf16 activations quantized on the way; every dispatched row's
    codes and scales against the oracle."""
    w = WORKLOADS["zipf1.2_T16384_H4096fp8_E128_k8"]
    print("case: fp8 dispatch full", w.name, flush=True)
    ids = routing_ids(w, np.random.default_rng(w.seed))
    g = torch.Generator(device="cpu").manual_seed(99)
    x = torch.randn(w.T, w.H, generator=g).to(torch.bfloat16)
    _check(x, ids, w.E, 1)
