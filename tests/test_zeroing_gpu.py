"""Row zeroing on the GPU against the oracle, bit for bit (needs the GPU):
the output memset (rows of tokens with a valid permuted index become zero)
and the padding zero-fill of dispatched rows."""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu
from workloads import WORKLOADS, build_inputs, routing

pytestmark = pytest.mark.gpu
DEV = gu.DEV


def _rand_rows(rng, n, shape_tail, dtype):
    if dtype == torch.uint8:
        return torch.from_numpy(rng.integers(1, 255, (n,) + shape_tail, dtype=np.uint8)).to(DEV)
    return torch.from_numpy(rng.standard_normal((n,) + shape_tail).astype(np.float32)) \
        .to(dtype).to(DEV)


@pytest.mark.parametrize("T,k,W,dtype", [
    (0, 8, 16, torch.bfloat16),
    (1, 1, 8, torch.bfloat16),
    (300, 8, 7168, torch.bfloat16),
    (77, 3, 13, torch.uint8),          # 13-byte rows: byte stores
    (50, 70, 100, torch.float32),      # topk > 64
    (40, 8, 20000, torch.float32),     # 80 KB rows: several column chunks
])
def test_output_memset(T, k, W, dtype):
    print("case: output memset", T, k, W, dtype, flush=True)
    rng = np.random.default_rng(T * 31 + k)
    out = _rand_rows(rng, T, (W,), dtype)
    perm = rng.integers(0, 1000, T * k).astype(np.int32)
    perm[rng.random(T * k) < 0.9] = -1                    # many tokens with no valid pick
    before = gu.bits(out)
    mx.moe_output_memset(out, torch.from_numpy(perm).to(DEV), k)
    torch.cuda.synchronize()
    want = oracle.output_memset(before, k, perm)
    np.testing.assert_array_equal(gu.bits(out), want)


def test_output_memset_misaligned_base():
    print("case: output memset misaligned", flush=True)
    rng = np.random.default_rng(4)
    T, k, W = 64, 4, 512
    big = _rand_rows(rng, T * W + 1, (), torch.bfloat16)
    out = big[1:].view(T, W)
    perm = rng.integers(-1, 3, T * k).astype(np.int32)
    before = gu.bits(out)
    mx.moe_output_memset(out, torch.from_numpy(perm).to(DEV), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.bits(out), oracle.output_memset(before, k, perm))


@pytest.mark.parametrize("T,E,k,A,W,dtype,with_offsets", [
    (100, 16, 4, 8, 256, torch.bfloat16, True),
    (100, 16, 4, 8, 256, torch.bfloat16, False),      # unused capacity zeroed too
    (500, 256, 8, 128, 7168, torch.bfloat16, True),
    (60, 7, 3, 5, 13, torch.uint8, True),
    (0, 8, 8, 16, 64, torch.bfloat16, True),
])
def test_zero_padding_rows(T, E, k, A, W, dtype, with_offsets):
    print("case: zero padding", T, E, k, A, W, dtype, with_offsets, flush=True)
    rng = np.random.default_rng(T + E + A)
    ids = routing.uniform_topk(rng, T, E, k) if T else np.zeros((0, k), np.int64)
    meta = gu.check_prepare(ids, E, A)
    t = meta["_t"]
    rows = _rand_rows(rng, t["input_permutation"].numel(), (W,), dtype)
    before = gu.bits(rows)
    mx.zero_padding_rows(rows, t["input_permutation"],
                         t["expert_offsets"] if with_offsets else None)
    torch.cuda.synchronize()
    want = oracle.zero_padding_rows(before, meta["input_permutation"],
                                    meta["expert_offsets"] if with_offsets else None)
    np.testing.assert_array_equal(gu.bits(rows), want)


def test_zeroing_full_size_uniform_T4096():
    """At the T=4096, H=7168 workload's size, launched as the benchmark
    launches it: padding rows of the full dispatched buffer and the output
    memset, each compared with the oracle on every byte."""
    w = WORKLOADS["uniform_T4096_H7168_E256_k8_pad128"]
    print("case: zeroing full", w.name, flush=True)
    inp = build_inputs(w, DEV)
    meta = gu.check_prepare(inp["ids"], w.E, w.row_align)
    t = meta["_t"]
    cap = t["input_permutation"].numel()
    xd = torch.empty(cap, w.H, dtype=torch.bfloat16, device=DEV)
    xd.view(torch.uint8).fill_(0x3C)
    mx.dispatch_rows(inp["x"], t["output_permutation"], w.k, xd)
    before = gu.bits(xd)
    mx.zero_padding_rows(xd, t["input_permutation"], t["expert_offsets"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(
        gu.bits(xd), oracle.zero_padding_rows(before, meta["input_permutation"],
                                              meta["expert_offsets"]))
    out = torch.randn(w.T, w.H, device=DEV).to(torch.bfloat16)
    before = gu.bits(out)
    mx.moe_output_memset(out, t["output_permutation"], w.k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.bits(out),
                                  oracle.output_memset(before, w.k, meta["output_permutation"]))
