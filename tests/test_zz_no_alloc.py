"""mx_prepare_moe_input_noalloc through the C ABI against mx_prepare_moe_input
(needs the GPU): bit-identical metadata on two calls in a row, the second
with a smaller input, so the second call reuses the library's scratch left
by the first."""

import ctypes

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from workloads import routing

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
        "output_permutation", "blockscale_offsets")


def _routing(T, k, E, A):
    r = mx.empty_routing(T, k, E, DEV, row_align=A, blockscale=True)
    for key in KEYS:
        r[key].fill_(-7)                      # poison: a missing write shows
    return r


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call(fn, ids, r, T, k, E, A, *tail):
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = fn(_ptr(ids), 5, T, k, E, 2 * 64, 32, 32, 64, A,
            _ptr(r["expert_offsets"]), _ptr(r["problem_sizes1"]), _ptr(r["problem_sizes2"]),
            _ptr(r["input_permutation"]), r["input_permutation"].numel(),
            _ptr(r["output_permutation"]), _ptr(r["blockscale_offsets"]), 128, *tail, stream)
    assert st == 0, mx.load_library().mx_status_string(st)


@pytest.mark.parametrize("sizes", [
    ((4096, 8, 256, 128), (1000, 8, 256, 128)),      # two-launch routing, then a smaller one
    ((65536, 8, 288, 1), (3000, 6, 100, 16)),        # the largest table, then another shape
    ((2048, 8, 256, 1), (40, 8, 256, 1)),            # then the one-launch path (no table)
])
def test_noalloc_matches_workspace_call_twice(sizes):
    lib = mx.load_library()
    rng = np.random.default_rng(sum(sum(s) for s in sizes))
    for T, k, E, A in sizes:
        print("case: noalloc", T, k, E, A, flush=True)
        ids_np = routing.uniform_topk(rng, T, E, k)
        ids_np[rng.random(ids_np.shape) < 0.01] = E + 3      # a few dropped picks
        ids = torch.from_numpy(ids_np).to(DEV)
        want = _routing(T, k, E, A)
        got = _routing(T, k, E, A)
        ws = torch.empty(max(lib.mx_prepare_workspace_size(T, k, E), 16), dtype=torch.uint8,
                         device=DEV)
        _call(lib.mx_prepare_moe_input, ids, want, T, k, E, A, _ptr(ws), ws.numel())
        _call(lib.mx_prepare_moe_input_noalloc, ids, got, T, k, E, A)
        torch.cuda.synchronize()
        for key in KEYS:
            assert torch.equal(got[key], want[key]), key
        # and the oracle agrees (same bar as the workspace call's parity tests)
        o = oracle.prepare_moe_input(ids_np, E, row_align=A, blockscale_align=128,
                                     gemm=(2 * 64, 32, 32, 64))
        for key in KEYS:
            np.testing.assert_array_equal(got[key].cpu().numpy().reshape(o[key].shape), o[key],
                                          err_msg=key)


def test_noalloc_binding_then_dispatch_and_combine():
    """The binding's prepare_moe_input_noalloc feeds dispatch and combine like
    the workspace form."""
    print("case: noalloc binding", flush=True)
    T, k, E, H = 512, 8, 64, 1024
    rng = np.random.default_rng(5)
    ids = torch.from_numpy(routing.uniform_topk(rng, T, E, k)).to(DEV)
    a, b = (mx.empty_routing(T, k, E, DEV, row_align=16) for _ in range(2))
    mx.prepare_moe_input(ids, a["expert_offsets"], a["problem_sizes1"], a["problem_sizes2"],
                         a["input_permutation"], a["output_permutation"], E, 64, H,
                         row_align=16, workspace=a["workspace"])
    mx.prepare_moe_input_noalloc(ids, b["expert_offsets"], b["problem_sizes1"],
                                 b["problem_sizes2"], b["input_permutation"],
                                 b["output_permutation"], E, 64, H, row_align=16)
    x = routing.normal_rows(T, H, "bf16", 6, device=DEV)
    outs = []
    for r in (a, b):
        rows = r["input_permutation"].numel()
        xd = torch.zeros((rows, H), dtype=torch.bfloat16, device=DEV)
        mx.dispatch_rows(x, r["output_permutation"], k, xd)
        out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
        mx.apply_shuffle_mul_sum(xd, out, r["output_permutation"])
        outs.append((xd, out))
    torch.cuda.synchronize()
    for key in ("expert_offsets", "input_permutation", "output_permutation"):
        assert torch.equal(a[key], b[key])
    for u, v in zip(*outs):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))
