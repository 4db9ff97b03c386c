"""Seeded random sweep of the whole path against the oracle (needs the GPU).

Each case draws its own shape from its seed: token count (empty, one, ragged
and several routing tiles), expert count (one expert up to 1024, powers of
two and not), top-k (including topk > E, where picks repeat an expert, and
topk > 64), segment padding, id width, share of invalid ids, row width and
element type.  On that draw it runs routing, dispatch (scatter and gather),
combine, the FP8 dispatch where the rows allow it, both zero-fills and the
tile-padded sort over a random expert window, and compares every output with
the oracle: bit for bit for metadata, rows and codes, and for the combine both
bit for bit and within rtol 1.6e-2 / atol 1e-2 (16-bit) or rtol 1e-5 (fp32).
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

SEEDS = range(160)
_FLOAT = (torch.bfloat16, torch.float16, torch.float32)


def draw(seed: int) -> dict:
    """The case for one seed (host only)."""
    rng = np.random.default_rng(90210 + seed)
    T = int(rng.choice([0, 1, rng.integers(2, 64), rng.integers(64, 1500),
                        rng.integers(1500, 6000), rng.integers(6000, 40000)],
                       p=[0.04, 0.04, 0.22, 0.4, 0.22, 0.08]))
    E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 128, 255, 256, 300, 1024]))
    k = int(rng.choice([1, 2, 4, 6, 8, 8, 8, 9, 70]))
    A = int(rng.choice([1, 1, 2, 3, 8, 16, 64, 128]))
    mode = str(rng.choice(["uniform", "k_hot", "zipf", "dups"]))
    if k > E or (mode == "k_hot" and E < 8):
        mode = "dups"
    bad = float(rng.choice([0.0, 0.0, 0.01, 0.1]))
    ids_dtype = torch.int32 if rng.random() < 0.5 else torch.int64
    dtype = [torch.bfloat16, torch.bfloat16, torch.float16, torch.float32,
             torch.uint8][int(rng.integers(0, 5))]
    H = int(rng.choice([1, 7, 8, 100, 128, 512, 1000, 2048, 4096, 7168]))
    cap = T * k + E * (A - 1)                             # dispatched rows
    while cap * H > (1 << 22) and H > 1:                  # keep the host copies small
        H //= 2
    out_dtype = _FLOAT[int(rng.integers(0, 3))]
    f_dtype = [None, torch.float32, torch.float32, torch.bfloat16, torch.float16][
        int(rng.integers(0, 5))]
    # tile-padded sort over a window [L0, L0 + EL) of the E experts
    L0 = int(rng.integers(0, E))
    EL = int(rng.integers(1, E - L0 + 1))
    S = int(rng.choice([1, 4, 16, 128]))
    return dict(seed=seed, T=T, E=E, k=k, A=A, mode=mode, bad=bad, ids_dtype=ids_dtype,
                dtype=dtype, H=H, out_dtype=out_dtype, f_dtype=f_dtype, L0=L0, EL=EL, S=S,
                rng=rng)


def _ids(c) -> np.ndarray:
    rng, T, E, k = c["rng"], c["T"], c["E"], c["k"]
    if T == 0:
        return np.zeros((0, k), np.int64)
    if c["mode"] == "dups":
        ids = rng.integers(0, E, (T, k))
    elif c["mode"] == "k_hot":
        ids = routing.k_hot_topk(rng, T, E, k, 8, 0.8)
    elif c["mode"] == "zipf":
        ids = routing.zipf_topk(rng, T, E, k, 1.2)
    else:
        ids = routing.uniform_topk(rng, T, E, k)
    if c["bad"]:
        m = rng.random(ids.shape) < c["bad"]
        ids = np.where(m, rng.choice([-1, -3, E, E + 9], size=ids.shape), ids)
    return ids.astype(np.int64)


def _rows(c, n, width, dtype, seed):
    if dtype == torch.uint8:
        return torch.from_numpy(c["rng"].integers(0, 256, (n, width), dtype=np.uint8)).to(DEV)
    return routing.normal_rows(n, width, gu.code(dtype), seed=seed, device=DEV)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(seed):
    c = draw(seed)
    print("case: sweep", {key: v for key, v in c.items() if key != "rng"}, flush=True)
    T, E, k, A, H, dtype = c["T"], c["E"], c["k"], c["A"], c["H"], c["dtype"]
    rng = c["rng"]
    ids = _ids(c)

    # routing metadata and permutations
    meta = gu.check_prepare(ids, E, A, c["ids_dtype"])
    t = meta["_t"]
    rows = t["input_permutation"].numel()

    # dispatch, scatter and gather forms
    x = _rows(c, T, H, dtype, seed)
    gu.check_dispatch(x, meta, k)

    # combine of expert outputs laid out as the dispatched rows
    ydt = dtype if dtype in _FLOAT else torch.bfloat16
    y = _rows(c, rows, H, ydt, seed + 1)
    f = None
    if c["f_dtype"] is not None:
        f = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(c["f_dtype"]).to(DEV)
    gu.check_combine(y, t["output_permutation"], f, c["out_dtype"], T)

    # FP8 dispatch of bf16 rows in 1x128 groups
    if dtype == torch.bfloat16 and H % 128 == 0:
        q = torch.full((rows, H), 0x55, dtype=torch.uint8, device=DEV)
        sc = torch.full((rows, H // 128), -3.0, dtype=torch.float32, device=DEV)
        mx.dispatch_rows_fp8(x, t["output_permutation"], k, q, sc)
        torch.cuda.synchronize()
        xq, xs = oracle.quantize_fp8_rows(gu.bits(x))
        inp = meta["input_permutation"]
        want_q = oracle.shuffle_rows(xq, inp, dst=np.full((rows, H), 0x55, np.uint8))
        want_s = oracle.shuffle_rows(xs, inp, dst=np.full((rows, H // 128), -3.0, np.float32))
        np.testing.assert_array_equal(gu.bits(q), want_q)
        np.testing.assert_array_equal(gu.bits(sc), want_s)

    # padding zero-fill of the dispatched rows, bounded by the padded total
    pad = _rows(c, rows, H, dtype, seed + 2)
    before = gu.bits(pad)
    mx.zero_padding_rows(pad, t["input_permutation"], t["expert_offsets"])
    torch.cuda.synchronize()
    want = oracle.zero_padding_rows(before, meta["input_permutation"], meta["expert_offsets"])
    np.testing.assert_array_equal(gu.bits(pad), want)

    # output memset of the tokens with a valid pick
    out = _rows(c, T, H, dtype, seed + 3)
    before = gu.bits(out)
    mx.moe_output_memset(out, t["output_permutation"], k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.bits(out),
                                  oracle.output_memset(before, k, meta["output_permutation"]))

    # tile-padded sort over the expert window
    L0, EL, S = c["L0"], c["EL"], c["S"]
    got = mx.moe_sort(torch.from_numpy(ids).to(c["ids_dtype"]).to(DEV), E, L0, EL, S)
    torch.cuda.synchronize()
    want = oracle.moe_sort(ids, E, L0, EL, S)
    for key in ("expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
                "tile_idx_to_group_idx", "tile_idx_to_mn_limit"):
        np.testing.assert_array_equal(got[key].cpu().numpy(), want[key], err_msg=key)
    assert got["total_num_padded_tokens"].item() == want["total_num_padded_tokens"]
    assert got["num_non_exiting_tiles"].item() == want["num_non_exiting_tiles"]
