"""Tile-padded sort with a local-expert window on the GPU against the oracle,
bit for bit, for every output (needs the GPU)."""

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

KEYS = ("expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
        "tile_idx_to_group_idx", "tile_idx_to_mn_limit")


def _check(ids, E, L0, EL, S, ids_dtype=torch.int64):
    got = mx.moe_sort(torch.from_numpy(np.ascontiguousarray(ids)).to(ids_dtype).to(DEV),
                      E, L0, EL, S)
    torch.cuda.synchronize()
    want = oracle.moe_sort(ids.astype(np.int64), E, L0, EL, S)
    for key in KEYS:
        np.testing.assert_array_equal(got[key].cpu().numpy(), want[key], err_msg=key)
    assert got["total_num_padded_tokens"].item() == want["total_num_padded_tokens"]
    assert got["num_non_exiting_tiles"].item() == want["num_non_exiting_tiles"]
    # expert offsets: the first row of every group = the oracle's padded prefix
    # sum over the window (its prepare_moe_input on the shifted ids)
    flat = ids.astype(np.int64) - L0
    shifted = np.where((flat >= 0) & (flat < EL), flat, -1).reshape(ids.shape)
    ref = oracle.prepare_moe_input(shifted, EL, row_align=S)
    np.testing.assert_array_equal(got["expert_offsets"].cpu().numpy(), ref["expert_offsets"])
    return got, want


@pytest.mark.parametrize("T,E,k,L0,EL,S,mode", [
    (0, 8, 8, 0, 8, 4, "uniform"),
    (4, 4, 2, 1, 2, 2, "dups"),
    (100, 64, 8, 16, 16, 8, "uniform"),
    (128, 256, 8, 0, 256, 128, "uniform"),        # one launch: 1024 picks
    (256, 64, 8, 0, 64, 1, "uniform"),            # one launch, unpadded: 2048 picks
    (257, 64, 8, 0, 64, 1, "uniform"),            # two launches: 2056 picks
    (1024, 256, 8, 0, 256, 128, "uniform"),       # two-launch path, 16 tiles
    (3001, 256, 8, 64, 32, 128, "uniform"),       # several tiles, ragged tail
    (5000, 256, 8, 0, 16, 64, "k_hot"),           # window holds the hot experts
    (5000, 256, 8, 128, 128, 256, "k_hot"),       # window holds only cold experts
    (4000, 128, 8, 100, 28, 1, "zipf"),           # tile of one row
    (700, 40, 70, 5, 30, 16, "dups"),             # topk > 64
    (2000, 1024, 8, 512, 512, 32, "uniform"),
    (9000, 256, 8, 32, 64, 128, "uniform"),      # tiles longer than 512 picks
])
@pytest.mark.parametrize("ids_dtype", [torch.int32, torch.int64])
def test_moe_sort_matches_oracle(T, E, k, L0, EL, S, mode, ids_dtype):
    print("case: moe_sort", T, E, k, L0, EL, S, mode, ids_dtype, flush=True)
    rng = np.random.default_rng(T + 13 * E + L0)
    if T == 0:
        ids = np.zeros((0, k), np.int64)
    elif mode == "dups":
        ids = rng.integers(-2, E + 2, (T, k))
    elif mode == "k_hot":
        ids = routing.k_hot_topk(rng, T, E, k, 8, 0.8)
    elif mode == "zipf":
        ids = routing.zipf_topk(rng, T, E, k, 1.2)
    else:
        ids = routing.uniform_topk(rng, T, E, k)
    _check(ids, E, L0, EL, S, ids_dtype)


def test_moe_sort_full_window_equals_prepare():
    """With the window covering every expert, the sort's pick -> row map is
    prepare_moe_input's output_permutation, and its row -> pick map divided
    by k is input_permutation (both on the GPU)."""
    print("case: moe_sort vs prepare", flush=True)
    rng = np.random.default_rng(3)
    ids = routing.uniform_topk(rng, 4096, 256, 8)
    got, _ = _check(ids, 256, 0, 256, 128)
    meta = gu.gpu_prepare(ids, 256, 128)
    np.testing.assert_array_equal(got["expanded_idx_to_permuted_idx"].cpu().numpy(),
                                  meta["output_permutation"])
    p2e = got["permuted_idx_to_expanded_idx"].cpu().numpy()
    np.testing.assert_array_equal(np.where(p2e >= 0, p2e // 8, -1), meta["input_permutation"])


def test_moe_sort_one_rank_of_288_slots():
    """One rank's share of the 288-slot workload at full size (T = 65536,
    top-8): slots [72, 108) of 8 ranks x 36 slots, tiles of 128 rows."""
    w = WORKLOADS["replica288_T65536_H7168_k8_f32out"]
    print("case: moe_sort rank share", w.name, flush=True)
    ids = routing_ids(w, np.random.default_rng(w.seed))
    _check(ids, w.E, 72, 36, 128)


def test_moe_sort_then_dispatch_is_the_permute():
    """The sort's outputs drive the row kernels: dispatch_rows with
    expanded_idx_to_permuted_idx writes row r = x[p2e[r] / k] for every row
    with p2e[r] >= 0 (the permute of the TensorRT-LLM page's MoE, in
    token-major form) and leaves padding and unused rows untouched; checked
    against the oracle's sort and gather, bit for bit."""
    print("case: moe_sort then dispatch", flush=True)
    rng = np.random.default_rng(57)
    T, E, k, L0, EL, S, H = 3000, 256, 8, 64, 32, 128, 2048
    ids = routing.uniform_topk(rng, T, E, k)
    got = mx.moe_sort(torch.from_numpy(ids).to(DEV), E, L0, EL, S)
    want = oracle.moe_sort(ids.astype(np.int64), E, L0, EL, S)
    p2e = want["permuted_idx_to_expanded_idx"]
    x = routing.normal_rows(T, H, "bf16", seed=58, device=DEV)
    rows = got["permuted_idx_to_expanded_idx"].numel()
    xd = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    xd.view(torch.uint8).fill_(gu.SENTINEL)
    mx.dispatch_rows(x, got["expanded_idx_to_permuted_idx"], k, xd)
    torch.cuda.synchronize()
    src = np.where(p2e >= 0, p2e // k, -1).astype(np.int32)
    used = src >= 0
    np.testing.assert_array_equal(gu.bits(xd)[used], oracle.shuffle_rows(gu.bits(x), src)[used])
    assert np.all(xd.view(torch.uint8).cpu().numpy()[~used] == gu.SENTINEL)
