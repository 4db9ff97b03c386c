"""prepare_dispatch (mx_prepare_dispatch) on the GPU, through the C ABI.

Every metadata array must equal the oracle's bit for bit, every used
dispatched row must equal the oracle's gather of its source token, rows no
pick lands on must keep a sentinel, and everything must equal what
prepare_moe_input followed by dispatch_rows writes.  The cases cover the one
launch path (up to 1024 picks, or 2048 with little padding; 16-byte rows and
bases; no side rows; at most 512 workgroups) and every input that leaves it.
"""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu
from workloads import routing

pytestmark = pytest.mark.gpu

DEV = gu.DEV
META = ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
        "output_permutation", "blockscale_offsets")


def _ids(rng, T, E, k, mode, bad):
    if mode == "dups":
        ids = rng.integers(0, E, (T, k))
    elif mode == "k_hot":
        ids = routing.k_hot_topk(rng, T, E, k, min(8, E), 0.8)
    else:
        ids = routing.uniform_topk(rng, T, E, k)
    if bad:
        m = rng.random(ids.shape) < bad
        ids = np.where(m, rng.choice([-1, -5, E, E + 77], size=ids.shape), ids)
    return ids.astype(np.int64)


def _routing(T, k, E, A):
    r = mx.empty_routing(T, k, E, DEV, row_align=A, blockscale=True)
    for key in META + ("workspace",):
        r[key].fill_(-7 if r[key].dtype == torch.int32 else 0x5A)
    return r


def _rows(cap, H, dtype, byte_offset=0):
    """A [cap, H] buffer filled with the sentinel; with byte_offset its base
    sits that many bytes into a larger allocation."""
    eb = torch.empty((), dtype=dtype).element_size()
    raw = torch.empty(cap * H * eb + byte_offset, dtype=torch.uint8, device=DEV)
    raw.fill_(gu.SENTINEL)
    return raw[byte_offset:].view(dtype).view(cap, H)


def _run(T, E, k, A, mode, bad, H, dtype, ids_dtype=torch.int64, dst_offset=0, seed=0):
    print("case: prepare_dispatch", T, E, k, A, mode, bad, H, dtype, ids_dtype, dst_offset,
          flush=True)
    rng = np.random.default_rng(seed * 1000 + T * 7 + E)
    ids = _ids(rng, T, E, k, mode, bad)
    t_ids = torch.from_numpy(ids).to(ids_dtype).to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed * 31 + T)
    x = torch.randn((T, H), generator=g, device=DEV).to(dtype)
    cap = mx.dispatch_capacity(T, k, E, A)
    n, kk = 64, 32

    r1, xd1 = _routing(T, k, E, A), _rows(cap, H, dtype, dst_offset)
    mx.prepare_dispatch(t_ids, r1["expert_offsets"], r1["problem_sizes1"], r1["problem_sizes2"],
                        r1["input_permutation"], r1["output_permutation"], E, n, kk, x, xd1,
                        r1["blockscale_offsets"], row_align=A, workspace=r1["workspace"])
    r2, xd2 = _routing(T, k, E, A), _rows(cap, H, dtype, dst_offset)
    mx.prepare_moe_input(t_ids, r2["expert_offsets"], r2["problem_sizes1"],
                         r2["problem_sizes2"], r2["input_permutation"], r2["output_permutation"],
                         E, n, kk, r2["blockscale_offsets"], row_align=A,
                         workspace=r2["workspace"])
    mx.dispatch_rows(x, r2["output_permutation"], k, xd2)
    torch.cuda.synchronize()

    o = oracle.prepare_moe_input(ids, E, row_align=A, blockscale_align=128,
                                 gemm=(2 * n, kk, kk, n))
    for key in META:
        got = r1[key].cpu().numpy().reshape(o[key].shape)
        np.testing.assert_array_equal(got, o[key], err_msg=key)
        np.testing.assert_array_equal(r2[key].cpu().numpy().reshape(o[key].shape), o[key],
                                      err_msg="two calls: " + key)
    if cap == 0:
        return
    inp = o["input_permutation"]
    used = inp >= 0
    want = oracle.shuffle_rows(gu.bits(x), inp)
    got = gu.bits(xd1)
    np.testing.assert_array_equal(got[used], want[used], err_msg="dispatched rows")
    raw = xd1.contiguous().view(torch.uint8).cpu().numpy().reshape(cap, -1)
    assert np.all(raw[~used] == gu.SENTINEL), "a row no pick lands on was written"
    assert torch.equal(xd1.view(torch.uint8), xd2.view(torch.uint8)), \
        "prepare_dispatch and prepare_moe_input + dispatch_rows differ"


@pytest.mark.parametrize("T,E,k,A,mode,bad,H,dtype", [
    (1, 8, 1, 1, "uniform", 0.0, 4096, torch.bfloat16),        # one pick
    (32, 256, 8, 1, "uniform", 0.0, 4096, torch.bfloat16),      # decode batch: 32 workgroups
    (33, 256, 8, 128, "uniform", 0.05, 7168, torch.bfloat16),   # padded, invalid ids, 2 chunks
    (128, 256, 8, 1, "k_hot", 0.0, 7168, torch.bfloat16),       # 1024 picks, 256 workgroups
    (256, 256, 8, 1, "uniform", 0.0, 7168, torch.bfloat16),     # 2048 picks, 512 workgroups
    (20, 33, 70, 3, "dups", 0.1, 1024, torch.float16),          # topk > 64
    (16, 1024, 8, 16, "uniform", 0.02, 2048, torch.float32),    # E = 1024
    (100, 4, 8, 1, "dups", 0.0, 512, torch.bfloat16),           # few experts, long segments
    (257, 256, 8, 1, "uniform", 0.0, 4096, torch.bfloat16),     # 2056 picks: two calls
    (200, 256, 8, 128, "uniform", 0.0, 4096, torch.bfloat16),   # heavy padding: two calls
    (64, 256, 8, 1, "uniform", 0.0, 40960, torch.bfloat16),     # 640 workgroups: two calls
    (8, 16, 4, 1, "uniform", 0.0, 100, torch.bfloat16),         # 200-byte rows: two calls
    (0, 256, 8, 1, "uniform", 0.0, 4096, torch.bfloat16),       # no tokens
])
@pytest.mark.parametrize("ids_dtype", [torch.int32, torch.int64])
def test_prepare_dispatch_matches_oracle(T, E, k, A, mode, bad, H, dtype, ids_dtype):
    _run(T, E, k, A, mode, bad, H, dtype, ids_dtype)


def test_prepare_dispatch_misaligned_destination_takes_two_calls():
    # row base 8 bytes past a 16-byte boundary: not the one-launch path
    _run(32, 256, 8, 1, "uniform", 0.0, 4096, torch.bfloat16, dst_offset=8)


def test_prepare_dispatch_short_destination_skips_rows():
    # num_dst_rows below the rows the routing places: those picks are skipped
    T, E, k = 16, 8, 4
    rng = np.random.default_rng(5)
    ids = routing.uniform_topk(rng, T, E, k).astype(np.int64)
    t_ids = torch.from_numpy(ids).to(DEV)
    x = torch.randn((T, 256), device=DEV).to(torch.bfloat16)
    r = _routing(T, k, E, 1)
    short = 20
    xd = _rows(short, 256, torch.bfloat16)
    mx.prepare_dispatch(t_ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                        r["input_permutation"], r["output_permutation"], E, 64, 32, x, xd,
                        r["blockscale_offsets"], workspace=r["workspace"])
    torch.cuda.synchronize()
    o = oracle.prepare_moe_input(ids, E)
    np.testing.assert_array_equal(r["output_permutation"].cpu().numpy(),
                                  o["output_permutation"])
    inp = o["input_permutation"][:short]
    want = oracle.shuffle_rows(gu.bits(x), inp)
    np.testing.assert_array_equal(gu.bits(xd)[inp >= 0], want[inp >= 0])


def test_prepare_dispatch_side_rows_take_two_calls():
    # fp8 rows with fp32 scale rows: the side rows go through dispatch_rows
    T, E, k, A = 48, 64, 8, 1
    rng = np.random.default_rng(9)
    ids = routing.uniform_topk(rng, T, E, k).astype(np.int64)
    t_ids = torch.from_numpy(ids).to(DEV)
    xq, sc = routing.fp8_blockscaled_rows(T, 1024, 11, device=DEV)
    cap = mx.dispatch_capacity(T, k, E, A)
    r = _routing(T, k, E, A)
    xd = torch.zeros((cap, 1024), dtype=xq.dtype, device=DEV)
    sd = torch.full((cap, sc.shape[1]), float("nan"), dtype=torch.float32, device=DEV)
    mx.prepare_dispatch(t_ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                        r["input_permutation"], r["output_permutation"], E, 64, 32, xq, xd,
                        r["blockscale_offsets"], side_input=sc, side_output=sd,
                        workspace=r["workspace"])
    torch.cuda.synchronize()
    o = oracle.prepare_moe_input(ids, E, blockscale_align=128, gemm=(128, 32, 32, 64))
    np.testing.assert_array_equal(r["input_permutation"].cpu().numpy(), o["input_permutation"])
    used = o["input_permutation"] >= 0
    np.testing.assert_array_equal(gu.bits(xd)[used],
                                  oracle.shuffle_rows(gu.bits(xq), o["input_permutation"])[used])
    np.testing.assert_array_equal(gu.bits(sd)[used],
                                  oracle.shuffle_rows(gu.bits(sc), o["input_permutation"])[used])


def test_prepare_dispatch_bound_call_repeats():
    # bind() once, call several times with new ids in place: each result exact
    T, E, k = 32, 256, 8
    t_ids = torch.empty((T, k), dtype=torch.int64, device=DEV)
    x = torch.randn((T, 4096), device=DEV).to(torch.bfloat16)
    cap = mx.dispatch_capacity(T, k, E, 1)
    r = _routing(T, k, E, 1)
    xd = _rows(cap, 4096, torch.bfloat16)
    call = mx.bind(mx.prepare_dispatch, t_ids, r["expert_offsets"], r["problem_sizes1"],
                   r["problem_sizes2"], r["input_permutation"], r["output_permutation"], E, 64,
                   32, x, xd, r["blockscale_offsets"], workspace=r["workspace"])
    for seed in range(3):
        print("case: bound prepare_dispatch, seed", seed, flush=True)
        ids = routing.uniform_topk(np.random.default_rng(seed), T, E, k).astype(np.int64)
        t_ids.copy_(torch.from_numpy(ids))
        assert call() is xd
        torch.cuda.synchronize()
        o = oracle.prepare_moe_input(ids, E)
        np.testing.assert_array_equal(r["output_permutation"].cpu().numpy(),
                                      o["output_permutation"])
        want = oracle.shuffle_rows(gu.bits(x), o["input_permutation"])
        used = o["input_permutation"] >= 0
        np.testing.assert_array_equal(gu.bits(xd)[used], want[used])
