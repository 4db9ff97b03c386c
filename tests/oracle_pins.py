"""Pins that tie the CPU oracle to something other than itself.

Each pin checks the oracle against hand-worked examples (tests/golden), a
library routine that computes the same thing by another algorithm (numpy
bincount / cumsum / stable argsort / fancy indexing, torch and numpy float
conversions), a closed form or invariant, a float64 sum with a rounding-error
bound, or brute force on tiny inputs.  The definitions pinned are those of the
sglang page "[jit_kernel] Add prepare_moe_input JIT kernels" (section
"Changes").

Every pin takes the oracle library handle, so the mutation test can run the
same pins against deliberately broken builds of the oracle and check that at
least one pin fails for each.
"""

from __future__ import annotations

import os

import numpy as np
import torch
import yaml

import oracle
from workloads import routing

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return yaml.safe_load(f)["cases"]


def _bf16_bits(a) -> np.ndarray:
    """float values -> bf16 bit patterns via torch's conversion (a library
    routine, independent of the oracle)."""
    return torch.tensor(np.asarray(a, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _bits_to_f32_torch(bits: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).float().numpy()


def _rand_ids(rng, T, E, k, mode, invalid_frac=0.0, dtype=np.int64):
    if mode == "uniform":
        ids = routing.uniform_topk(rng, T, E, k) if k <= E else rng.integers(0, E, (T, k))
    elif mode == "dups":                       # duplicates within a token allowed
        ids = rng.integers(0, E, (T, k))
    elif mode == "k_hot":
        ids = routing.k_hot_topk(rng, T, E, k, min(4, E), 0.9)
    elif mode == "zipf":
        ids = routing.zipf_topk(rng, T, E, k, 1.2)
    else:
        raise ValueError(mode)
    if invalid_frac:
        bad = rng.random(ids.shape) < invalid_frac
        junk = rng.choice(np.array([-1, -7, E, E + 3, 2**31 - 1]), size=ids.shape)
        ids = np.where(bad, junk, ids)
    return ids.astype(dtype)


def _round_up(v, a):
    return (v + a - 1) // a * a


# ---------------------------------------------------------------------------
# prepare_moe_input
# ---------------------------------------------------------------------------

def pin_golden_prepare(lib):
    """Hand-worked examples of counts, offsets and both permutations."""
    for case in _golden("prepare_small.yaml"):
        for dt in (np.int32, np.int64):
            ids = np.array(case["ids"], dtype=dt)
            m = oracle.prepare_moe_input(ids, case["num_experts"], row_align=case["row_align"],
                                         lib=lib)
            for key in ("expert_offsets", "output_permutation", "input_permutation",
                        "blockscale_offsets"):
                np.testing.assert_array_equal(m[key], np.array(case[key]),
                                              err_msg=f"{case['name']} {key}")
            np.testing.assert_array_equal(m["problem_sizes1"][:, 0], case["counts"])


def pin_prepare_vs_numpy(lib):
    """Unpadded metadata equals numpy's: counts = bincount of the valid ids,
    offsets = cumsum of counts, and the rows in order are numpy's stable
    argsort of the flat ids, so input_permutation = order // k and
    output_permutation is its inverse."""
    rng = np.random.default_rng(11)
    for T, E, k, mode in [(1, 1, 1, "uniform"), (7, 5, 3, "uniform"), (33, 64, 8, "uniform"),
                          (200, 256, 8, "k_hot"), (300, 128, 8, "zipf"), (50, 6, 9, "dups"),
                          (129, 288, 8, "uniform")]:
        for dt in (np.int32, np.int64):
            ids = _rand_ids(rng, T, E, k, mode, dtype=dt)
            m = oracle.prepare_moe_input(ids, E, row_align=1, lib=lib)
            flat = ids.ravel().astype(np.int64)
            counts = np.bincount(flat, minlength=E)
            np.testing.assert_array_equal(m["problem_sizes1"][:, 0], counts)
            assert counts.sum() == T * k                      # closed form, all ids valid
            np.testing.assert_array_equal(m["expert_offsets"],
                                          np.concatenate([[0], np.cumsum(counts)]))
            order = np.argsort(flat, kind="stable")
            np.testing.assert_array_equal(m["input_permutation"], order // k)
            inv = np.empty_like(order)
            inv[order] = np.arange(order.size)
            np.testing.assert_array_equal(m["output_permutation"], inv)


def pin_prepare_padding_layout(lib):
    """With row_align A: segment e has ceil(count/A)*A rows starting at the
    running sum; its first count rows hold the expert's picks in ascending
    flat index (one row per pick: a bijection between valid picks and used
    rows), and every other row of the capacity is -1."""
    rng = np.random.default_rng(12)
    for T, E, k, A, mode, bad in [(40, 16, 4, 8, "uniform", 0.0), (100, 64, 8, 128, "k_hot", 0.0),
                                  (64, 32, 8, 3, "zipf", 0.1), (17, 5, 2, 1, "dups", 0.3),
                                  (0, 8, 8, 128, "uniform", 0.0)]:
        ids = _rand_ids(rng, T, E, k, mode, invalid_frac=bad) if T else np.zeros((0, k), np.int64)
        m = oracle.prepare_moe_input(ids, E, row_align=A, lib=lib)
        flat = ids.ravel()
        valid = (flat >= 0) & (flat < E)
        counts = np.bincount(flat[valid], minlength=E)
        seg = _round_up(counts, A)
        eo = m["expert_offsets"]
        np.testing.assert_array_equal(eo, np.concatenate([[0], np.cumsum(seg)]))
        assert np.all(np.diff(eo) >= 0)
        cap = T * k + E * (A - 1)
        assert eo[-1] <= cap and m["input_permutation"].size == cap
        inp, outp = m["input_permutation"], m["output_permutation"]
        np.testing.assert_array_equal(outp[~valid], -1)
        expected_inp = np.full(cap, -1, np.int64)
        for e in range(E):
            picks = np.nonzero(valid & (flat == e))[0]          # ascending flat index
            rows = eo[e] + np.arange(picks.size)
            np.testing.assert_array_equal(outp[picks], rows)
            expected_inp[rows] = picks // k
        np.testing.assert_array_equal(inp, expected_inp)


def pin_prepare_bruteforce(lib):
    """Tiny inputs against a different algorithm in pure Python: for each
    expert in turn, scan all picks and append the matching ones (an O(N*E)
    selection, not a counting sort)."""
    rng = np.random.default_rng(13)
    for trial in range(30):
        T = int(rng.integers(0, 6))
        k = int(rng.integers(1, 4))
        E = int(rng.integers(1, 6))
        A = int(rng.integers(1, 5))
        ids = rng.integers(-1, E + 1, (T, k)).astype(np.int64)
        m = oracle.prepare_moe_input(ids, E, row_align=A, lib=lib)
        flat = [int(v) for v in ids.ravel()]
        rows_of_pick = [-1] * len(flat)
        token_of_row = [-1] * (T * k + E * (A - 1))
        offsets = [0]
        r = 0
        for e in range(E):
            start = r
            for i, v in enumerate(flat):
                if v == e:
                    rows_of_pick[i] = r
                    token_of_row[r] = i // k
                    r += 1
            while (r - start) % A:
                r += 1
            offsets.append(r)
        assert list(m["expert_offsets"]) == offsets, trial
        assert list(m["output_permutation"]) == rows_of_pick, trial
        assert list(m["input_permutation"]) == token_of_row, trial


def pin_blockscale_and_problem_sizes(lib):
    """Block-scale offsets: running sum of each count rounded up to B
    (numpy cumsum).  Problem sizes: (count, N, K) per expert with the given
    N, K; the counts are numpy's bincount."""
    rng = np.random.default_rng(14)
    # with row_align > 1 the block-scale sum must still round the raw counts,
    # not the row-padded ones (they differ when the padding crosses a B step)
    for T, E, k, B, A in [(300, 128, 8, 128, 1), (50, 7, 3, 16, 1), (5, 4, 2, 1, 1),
                          (300, 16, 8, 4, 3), (1000, 64, 8, 128, 64), (40, 5, 3, 2, 7)]:
        ids = _rand_ids(rng, T, E, k, "zipf" if E >= 8 else "dups", invalid_frac=0.05)
        m = oracle.prepare_moe_input(ids, E, row_align=A, blockscale_align=B,
                                     gemm=(2 * 512, 256, 256, 512), lib=lib)
        flat = ids.ravel()
        counts = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
        np.testing.assert_array_equal(m["blockscale_offsets"],
                                      np.concatenate([[0], np.cumsum(_round_up(counts, B))]))
        np.testing.assert_array_equal(m["problem_sizes1"],
                                      np.stack([counts, np.full(E, 1024), np.full(E, 256)], 1))
        np.testing.assert_array_equal(m["problem_sizes2"],
                                      np.stack([counts, np.full(E, 256), np.full(E, 512)], 1))


def pin_prepare_edges(lib):
    """Degenerate shapes: no tokens, one expert, every id invalid, a
    too-small capacity is refused."""
    m = oracle.prepare_moe_input(np.zeros((0, 8), np.int64), 256, row_align=128, lib=lib)
    assert not m["expert_offsets"].any() and m["output_permutation"].size == 0
    assert np.all(m["input_permutation"] == -1)
    m = oracle.prepare_moe_input(np.zeros((9, 1), np.int32), 1, lib=lib)
    np.testing.assert_array_equal(m["expert_offsets"], [0, 9])
    np.testing.assert_array_equal(m["input_permutation"], np.arange(9))
    m = oracle.prepare_moe_input(np.full((4, 2), 7, np.int64), 7, row_align=2, lib=lib)
    assert np.all(m["output_permutation"] == -1) and not m["expert_offsets"].any()
    try:
        oracle.prepare_moe_input(np.zeros((4, 2), np.int64), 2, row_align=4, r_max=3, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("capacity smaller than the padded rows was accepted")


# ---------------------------------------------------------------------------
# shuffle_rows
# ---------------------------------------------------------------------------

def pin_shuffle_vs_numpy(lib):
    """Row gather equals numpy fancy indexing, byte for byte, for any row
    width; rows whose index is out of range are left untouched."""
    rng = np.random.default_rng(15)
    for n_src, width, n_dst in [(10, 7, 25), (33, 128, 100), (1, 1, 3), (64, 4096 + 3, 40)]:
        src = rng.integers(0, 256, (n_src, width), dtype=np.uint8)
        idx = rng.integers(-2, n_src + 2, n_dst).astype(np.int32)
        init = rng.integers(0, 256, (n_dst, width), dtype=np.uint8)
        got = oracle.shuffle_rows(src, idx, dst=init.copy(), lib=lib)
        ok = (idx >= 0) & (idx < n_src)
        np.testing.assert_array_equal(got[ok], src[idx[ok]])
        np.testing.assert_array_equal(got[~ok], init[~ok])


# ---------------------------------------------------------------------------
# apply_shuffle_mul_sum
# ---------------------------------------------------------------------------

def pin_golden_combine(lib):
    """Hand-worked sums, including exact ties that must round to even."""
    for case in _golden("combine_small.yaml"):
        y = np.array(case["y"], np.float32)
        k = case["k"]
        perm = np.array(case["permutation"], np.int32)
        T = perm.size // k
        fac = None if case["factors"] is None else np.array(case["factors"], np.float32)
        yb = _bf16_bits(y)
        np.testing.assert_array_equal(_bits_to_f32_torch(yb, "bf16"), y)   # exact inputs
        o32 = oracle.apply_shuffle_mul_sum(yb, "bf16", perm, fac, "f32", T, k, "f32", lib=lib)
        np.testing.assert_array_equal(o32, np.array(case["out_f32"], np.float32),
                                      err_msg=case["name"])
        ob = oracle.apply_shuffle_mul_sum(yb, "bf16", perm, fac, "f32", T, k, "bf16", lib=lib)
        np.testing.assert_array_equal(ob, np.array(case["out_bf16_bits"], np.uint16),
                                      err_msg=case["name"])


def _dispatch_identity(x_bits: np.ndarray, ids: np.ndarray, E: int, A: int, lib):
    m = oracle.prepare_moe_input(ids, E, row_align=A, lib=lib)
    xd = oracle.shuffle_rows(x_bits, m["input_permutation"], lib=lib)
    return m, xd


def pin_combine_identity(lib):
    """Identity experts (y = dispatched x) reproduce x bit-exactly when
    (i) k = 1 with unit weight, and (ii) k = 8 with every weight 1/8: each
    partial sum m*x/8 (m <= 8) of a bf16 or fp16 x needs at most 14
    significant bits, so the fp32 sum is exact and rounds back to x."""
    rng = np.random.default_rng(16)
    T, H, E = 37, 40, 19
    for dtype in ("bf16", "f16", "f32"):
        x = rng.standard_normal((T, H)).astype(np.float32) * 3
        if dtype == "bf16":
            xb = _bf16_bits(x)
        elif dtype == "f16":
            xb = x.astype(np.float16).view(np.uint16)
        else:
            xb = x
        ids1 = _rand_ids(rng, T, E, 1, "uniform")
        m, xd = _dispatch_identity(xb, ids1, E, 4, lib)
        out = oracle.apply_shuffle_mul_sum(xd, dtype, m["output_permutation"], None, "f32",
                                           T, 1, dtype, lib=lib)
        np.testing.assert_array_equal(out, xb)
        if dtype == "f32":
            continue        # a 24-bit significand times m/8 is not exact in fp32
        ids8 = _rand_ids(rng, T, E, 8, "uniform")
        m, xd = _dispatch_identity(xb, ids8, E, 1, lib)
        w = np.full((T, 8), 0.125, np.float32)
        out = oracle.apply_shuffle_mul_sum(xd, dtype, m["output_permutation"], w, "f32",
                                           T, 8, dtype, lib=lib)
        np.testing.assert_array_equal(out, xb)


def pin_combine_softmax_identity(lib):
    """Identity experts with softmax weights (summing to 1 within rounding)
    give back x within the bf16 tolerance rtol 1.6e-2 / atol 1e-2, and within
    a few fp32 ulps for fp32 output."""
    rng = np.random.default_rng(17)
    T, H, E, k = 64, 96, 32, 8
    x = rng.standard_normal((T, H)).astype(np.float32)
    xb = _bf16_bits(x)
    ids = _rand_ids(rng, T, E, k, "uniform")
    w = routing.softmax_weights(rng, T, k)
    m, xd = _dispatch_identity(xb, ids, E, 1, lib)
    out = oracle.apply_shuffle_mul_sum(xd, "bf16", m["output_permutation"], w, "f32", T, k,
                                       "bf16", lib=lib)
    xf = _bits_to_f32_torch(xb, "bf16")
    np.testing.assert_allclose(_bits_to_f32_torch(out, "bf16"), xf, rtol=1.6e-2, atol=1e-2)
    out32 = oracle.apply_shuffle_mul_sum(xd, "bf16", m["output_permutation"], w, "f32", T, k,
                                         "f32", lib=lib)
    np.testing.assert_allclose(out32, xf, rtol=1e-5, atol=1e-6)


def pin_combine_f64_bound(lib):
    """fp32 output against the exact (float64) weighted sum: the error of k
    fused multiply-adds is at most gamma_k * sum_j |w_j y_j| with
    gamma_k = k u / (1 - k u), u = 2^-24.  Factors in bf16 are widened
    exactly.  Also checks that a wrong operand (a transposed y, a wrong
    permutation entry) would be caught: the bound is far tighter than the
    values' spread."""
    rng = np.random.default_rng(18)
    u = 2.0 ** -24
    for T, H, k, R, fdt in [(20, 33, 8, 200, "f32"), (9, 64, 3, 40, "bf16"), (5, 8, 1, 7, "f32")]:
        y32 = rng.standard_normal((R, H)).astype(np.float32)
        yb = _bf16_bits(y32)
        yf = _bits_to_f32_torch(yb, "bf16").astype(np.float64)
        perm = rng.integers(0, R, T * k).astype(np.int32)
        w32 = rng.standard_normal((T, k)).astype(np.float32)
        if fdt == "bf16":
            wb = _bf16_bits(w32)
            wf = _bits_to_f32_torch(wb, "bf16").astype(np.float64)
            warg = wb
        else:
            wf = w32.astype(np.float64)
            warg = w32
        prods = yf[perm.reshape(T, k)] * wf[:, :, None]          # [T, k, H]
        exact = prods.sum(axis=1)
        bound = k * u / (1 - k * u) * np.abs(prods).sum(axis=1)
        got = oracle.apply_shuffle_mul_sum(yb, "bf16", perm, warg, fdt, T, k, "f32", lib=lib)
        assert np.all(np.abs(got.astype(np.float64) - exact) <= bound), "fp32 sum out of bound"


def pin_combine_f16_factors_and_out(lib):
    """fp16 expert output, fp16 factors and fp16 output against numpy's
    float16 conversions of the float64 sum: the result is within one fp16
    ulp (the fp32 sum is far more accurate than fp16)."""
    rng = np.random.default_rng(19)
    T, H, k, R = 16, 24, 4, 50
    y = rng.standard_normal((R, H)).astype(np.float16)
    w = rng.random((T, k)).astype(np.float16)
    perm = rng.integers(0, R, T * k).astype(np.int32)
    exact = (y.astype(np.float64)[perm.reshape(T, k)] * w.astype(np.float64)[:, :, None]).sum(1)
    got = oracle.apply_shuffle_mul_sum(y.view(np.uint16), "f16", perm, w.view(np.uint16), "f16",
                                       T, k, "f16", lib=lib).view(np.float16).astype(np.float64)
    ulp = np.spacing(np.abs(exact).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(got - exact) <= ulp), "fp16 combine off by more than one ulp"


def pin_conversions(lib):
    """The oracle's number-format conversions against library routines:
    fp32 -> bf16 against torch, fp32 -> fp16 against numpy (both round to
    nearest even), and the widenings against torch / numpy on every bf16
    and fp16 bit pattern."""
    rng = np.random.default_rng(20)
    special = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                        1e-45, -1e-45, 1.1754942e-38, 65504.0, 65519.99, 65520.0, 65536.0,
                        6.1035156e-05, 6.1e-05, 5.96e-08, 2.98e-08, 2.99e-08, 1e-10],
                       dtype=np.float32)
    # exact bf16 ties: low 16 bits = 0x8000 with both parities of bit 16
    ties = (rng.integers(0, 2**15, 200, dtype=np.uint32) << 17 | np.uint32(0x8000)) \
        | (rng.integers(0, 2, 200, dtype=np.uint32) << 16)
    ties = ties.astype(np.uint32).view(np.float32)
    # exact fp16 ties: fp32 values with 13 dropped fraction bits = 1 0000 0000 0000
    f16ties = ((rng.integers(113, 142, 200, dtype=np.uint32) << 23)
               | (rng.integers(0, 2**10, 200, dtype=np.uint32) << 13) | np.uint32(1 << 12))
    f16ties = f16ties.astype(np.uint32).view(np.float32)
    vals = np.concatenate([special, -special, ties, f16ties,
                           (rng.standard_normal(2000) * 10.0 ** rng.integers(-8, 6, 2000)).astype(np.float32),
                           rng.integers(0, 2**32, 2000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    vals = vals.astype(np.float32)
    vals = vals[~np.isnan(vals)]
    np.testing.assert_array_equal(oracle.f32_to_bf16(vals, lib=lib), _bf16_bits(vals))
    with np.errstate(over="ignore"):
        want16 = vals.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16(vals, lib=lib), want16)
    # NaN stays NaN (a reading: payloads are not unique).  Patterns whose
    # payload lies only in the low 16 bits would become infinities if the
    # narrowing merely truncated, so they are included with the random NaNs.
    nans = np.concatenate([
        np.array([0x7fc00000, 0xffc00000, 0x7f800001, 0xff800001, 0x7f80ffff, 0x7f810000,
                  0x7fbfffff, 0xffffffff], np.uint32).view(np.float32),
        rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32).view(np.float32)])
    nans = nans[np.isnan(nans)]
    assert nans.size > 8
    assert np.isnan(_bits_to_f32_torch(oracle.f32_to_bf16(nans, lib=lib), "bf16")).all()
    assert np.isnan(oracle.f32_to_f16(nans, lib=lib).view(np.float16)).all()
    all16 = np.arange(2**16, dtype=np.uint32).astype(np.uint16)
    fin = ~np.isnan(all16.view(np.float16))
    np.testing.assert_array_equal(oracle.f16_to_f32(all16, lib=lib)[fin],
                                  all16.view(np.float16).astype(np.float32)[fin])
    assert np.isnan(oracle.f16_to_f32(all16, lib=lib)[~fin]).all()
    bf_ref = _bits_to_f32_torch(all16, "bf16")
    finb = ~np.isnan(bf_ref)
    np.testing.assert_array_equal(oracle.bf16_to_f32(all16, lib=lib)[finb], bf_ref[finb])
    assert np.isnan(oracle.bf16_to_f32(all16, lib=lib)[~finb]).all()


# ---------------------------------------------------------------------------
# zeroing rows in place
# ---------------------------------------------------------------------------

def _golden_doc(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return yaml.safe_load(f)


def pin_golden_zeroing(lib):
    """Hand-worked output memset and padding zero-fill."""
    doc = _golden_doc("prepare_small.yaml")
    for case in doc["memset_cases"]:
        before = np.array(case["rows_before"], np.float32)
        k = len(case["output_permutation"]) // len(before)
        got = oracle.output_memset(before, k, np.array(case["output_permutation"]), lib=lib)
        np.testing.assert_array_equal(got, np.array(case["rows_after"], np.float32))
    for case in doc["padding_cases"]:
        inp = np.array(case["input_permutation"], np.int32)
        rows = np.arange(1, inp.size + 1, dtype=np.float32)[:, None] * np.ones((1, 3), np.float32)
        got = oracle.zero_padding_rows(rows, inp, np.array(case["expert_offsets"]), lib=lib)
        zeroed = np.nonzero((got == 0).all(axis=1))[0]
        np.testing.assert_array_equal(zeroed, case["zeroed_rows"])
        np.testing.assert_array_equal(got[(got != 0).any(axis=1)], rows[(got != 0).any(axis=1)])


def pin_zeroing_vs_numpy(lib):
    """Row masks computed with numpy: a token row is zeroed iff any of its
    picks has an index >= 0; a dispatched row below the padded total is
    zeroed iff its source index is negative; every other byte is kept."""
    rng = np.random.default_rng(21)
    for T, k, W in [(50, 8, 7), (1, 1, 16), (33, 3, 1), (0, 4, 5)]:
        perm = rng.integers(-1, 30, T * k).astype(np.int32)
        perm[rng.random(T * k) < 0.5] = -1
        before = rng.integers(1, 255, (T, W)).astype(np.uint8)
        got = oracle.output_memset(before, k, perm, lib=lib)
        mask = (perm.reshape(T, k) >= 0).any(axis=1) if T else np.zeros(0, bool)
        np.testing.assert_array_equal(got, np.where(mask[:, None], 0, before))
    for T, E, k, A in [(40, 16, 4, 8), (100, 64, 8, 128), (5, 3, 2, 1)]:
        ids = routing.uniform_topk(rng, T, E, k)
        m = oracle.prepare_moe_input(ids, E, row_align=A, lib=lib)
        inp, eo = m["input_permutation"], m["expert_offsets"]
        rows = rng.integers(1, 255, (inp.size, 6)).astype(np.uint8)
        got = oracle.zero_padding_rows(rows, inp, eo, lib=lib)
        mask = (inp < 0) & (np.arange(inp.size) < eo[-1])
        np.testing.assert_array_equal(got, np.where(mask[:, None], 0, rows))
        got = oracle.zero_padding_rows(rows, inp, None, lib=lib)
        np.testing.assert_array_equal(got, np.where((inp < 0)[:, None], 0, rows))


# ---------------------------------------------------------------------------
# tile-padded sort with a local-expert window
# ---------------------------------------------------------------------------

_SORT_KEYS = ("expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
              "tile_idx_to_group_idx", "tile_idx_to_mn_limit")


def pin_golden_moe_sort(lib):
    """Hand-worked tile-padded sort metadata (tests/golden/moe_sort_small.yaml)."""
    for case in _golden("moe_sort_small.yaml"):
        for dt in (np.int32, np.int64):
            m = oracle.moe_sort(np.array(case["ids"], dt), case["num_experts"],
                                case["local_expert_offset"], case["num_local_experts"],
                                case["tile_size"], lib=lib)
            for key in _SORT_KEYS:
                np.testing.assert_array_equal(m[key], case[key], err_msg=f"{case['name']} {key}")
            assert m["total_num_padded_tokens"] == case["total_num_padded_tokens"]
            assert m["num_non_exiting_tiles"] == case["num_non_exiting_tiles"]


def sort_reference_numpy(ids, E, L0, EL, S):
    """The same metadata assembled from numpy library routines (stable
    argsort, bincount, cumsum, repeat)."""
    flat = ids.ravel().astype(np.int64)
    g = flat - L0
    local = (g >= 0) & (g < EL) & (flat < E)
    counts = np.bincount(g[local], minlength=EL)
    tiles = -(-counts // S)
    first = np.concatenate([[0], np.cumsum(tiles * S)])
    cap = flat.size + EL * (S - 1)
    max_tiles = -(-cap // S)
    li = np.nonzero(local)[0]
    order = li[np.argsort(g[li], kind="stable")]               # local picks by group, stable
    rank = np.arange(order.size) - np.concatenate([[0], np.cumsum(counts)])[g[order]]
    rows = first[g[order]] + rank
    e2p = np.full(flat.size, -1, np.int64)
    e2p[order] = rows
    p2e = np.full(cap, -1, np.int64)
    p2e[rows] = order
    tg = np.full(max_tiles, -1, np.int64)
    tl = np.full(max_tiles, -1, np.int64)
    ntile = int(tiles.sum())
    tg[:ntile] = np.repeat(np.arange(EL), tiles)
    tl[:ntile] = np.repeat(first[:-1] + counts, tiles)
    return {"expanded_idx_to_permuted_idx": e2p, "permuted_idx_to_expanded_idx": p2e,
            "tile_idx_to_group_idx": tg, "tile_idx_to_mn_limit": tl,
            "total_num_padded_tokens": int(first[-1]), "num_non_exiting_tiles": ntile}


def pin_moe_sort_vs_numpy(lib):
    """Random routings, windows and tile sizes against the numpy assembly."""
    rng = np.random.default_rng(22)
    for T, E, k, L0, EL, S, mode in [(64, 16, 4, 4, 8, 8, "uniform"), (200, 256, 8, 32, 32, 128, "k_hot"),
                                     (300, 128, 8, 0, 128, 16, "zipf"), (50, 9, 3, 2, 7, 1, "dups"),
                                     (1, 4, 1, 3, 1, 4, "uniform"), (0, 8, 8, 0, 8, 4, "uniform")]:
        ids = _rand_ids(rng, T, E, k, mode, invalid_frac=0.05) if T else np.zeros((0, k), np.int64)
        m = oracle.moe_sort(ids, E, L0, EL, S, lib=lib)
        want = sort_reference_numpy(ids, E, L0, EL, S)
        for key in _SORT_KEYS:
            np.testing.assert_array_equal(m[key], want[key], err_msg=key)
        assert m["total_num_padded_tokens"] == want["total_num_padded_tokens"]
        assert m["num_non_exiting_tiles"] == want["num_non_exiting_tiles"]


# ---------------------------------------------------------------------------
# FP8 quantization
# ---------------------------------------------------------------------------

def _e4m3_torch(v: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn bytes by torch's conversion (round to nearest even),
    after clamping to the finite range so torch does not produce NaN."""
    t = torch.from_numpy(np.clip(np.asarray(v, np.float32), -448.0, 448.0))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_conversion(lib):
    """The oracle's fp32 -> e4m3fn rounding against torch's on every e4m3
    value, every midpoint between neighbours (ties to even), random values
    over the whole range, subnormals, and values past 448 (saturation)."""
    codes = np.arange(256, dtype=np.uint8)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    finite = np.isfinite(vals)
    v = np.unique(vals[finite])
    mids = ((v[1:].astype(np.float64) + v[:-1]) / 2).astype(np.float32)   # exact in fp32
    rng = np.random.default_rng(23)
    rand = (rng.standard_normal(4000) * 10.0 ** rng.uniform(-4, 2.7, 4000)).astype(np.float32)
    tiny = (rng.random(500) * 2.0 ** -6).astype(np.float32)
    test = np.concatenate([v, mids, -mids, rand, tiny, -tiny,
                           np.array([0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 1e9, -1e9], np.float32)])
    np.testing.assert_array_equal(oracle.f32_to_e4m3(test, lib=lib), _e4m3_torch(test))
    assert oracle.f32_to_e4m3(np.array([np.nan], np.float32), lib=lib)[0] == 0x7f


def pin_quantize_rows(lib):
    """Per 1x128 group: the scale is amax / 448 in fp32 and the codes are the
    e4m3 rounding of x / scale (torch's conversion of numpy's fp32 quotient);
    dequantized values are within half an e4m3 ulp (relative 2^-4) of x;
    an all-zero group gets scale 1 and zero codes."""
    rng = np.random.default_rng(24)
    T, H = 17, 512
    x = rng.standard_normal((T, H)).astype(np.float32) * 10.0 ** rng.uniform(-3, 3, (T, 1))
    x[3, 128:256] = 0.0
    xb = _bf16_bits(x)
    xf = _bits_to_f32_torch(xb, "bf16").reshape(T, H // 128, 128)
    q, sc = oracle.quantize_fp8_rows(xb, lib=lib)
    amax = np.abs(xf).max(axis=2)
    want_sc = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    np.testing.assert_array_equal(sc, want_sc)
    quot = (xf / want_sc[:, :, None]).astype(np.float32)
    np.testing.assert_array_equal(q, _e4m3_torch(quot).reshape(T, H))
    deq = torch.from_numpy(q).view(torch.float8_e4m3fn).float().numpy().reshape(T, H // 128, 128)
    deq = deq * sc[:, :, None]
    assert np.all(np.abs(deq - xf) <= np.abs(xf) * 2.0 ** -4 + sc[:, :, None] * 2.0 ** -10)
    assert np.all(q[3, 128:256] == 0) and sc[3, 1] == 1.0


def pin_quantize_non_finite(lib):
    """Non-finite inputs (the pages are silent; the reading taken): amax is
    numpy's fmax reduction from 0 (IEEE maxNum, which skips NaN), an
    infinite element makes the scale infinite, the codes are torch's
    conversion of numpy's fp32 quotient with every NaN coded 0x7f, and a
    group of NaN only gets scale 1."""
    T, H = 2, 128 * 5
    x = np.linspace(-3, 3, T * H, dtype=np.float32).reshape(T, H)
    x[0, 5] = np.nan                       # group 0: NaN among normals
    x[0, 130] = np.inf                     # group 1: +inf
    x[0, 260] = -np.inf                    # group 2: -inf and a NaN
    x[0, 300] = np.nan
    x[1, 384:512] = np.nan                 # row 1 group 3: NaN only
    xb = _bf16_bits(x)
    G = H // 128
    xf = _bits_to_f32_torch(xb, "bf16").reshape(T, G, 128)
    q, sc = oracle.quantize_fp8_rows(xb, lib=lib)
    amax = np.fmax.reduce(np.concatenate([np.zeros((T, G, 1), np.float32), np.abs(xf)], axis=2),
                          axis=2)
    want_sc = np.where(amax > 0, (amax / np.float32(448.0)).astype(np.float32), np.float32(1.0))
    np.testing.assert_array_equal(sc, want_sc)
    assert np.isinf(sc[0, 1]) and np.isinf(sc[0, 2]) and sc[1, 3] == 1.0
    with np.errstate(invalid="ignore"):
        quot = (xf / want_sc[:, :, None]).astype(np.float32)
    want_q = _e4m3_torch(quot)
    want_q[np.isnan(quot)] = 0x7f
    np.testing.assert_array_equal(q, want_q.reshape(T, H))


ALL_PINS = [
    pin_golden_prepare,
    pin_prepare_vs_numpy,
    pin_prepare_padding_layout,
    pin_prepare_bruteforce,
    pin_blockscale_and_problem_sizes,
    pin_prepare_edges,
    pin_shuffle_vs_numpy,
    pin_golden_combine,
    pin_combine_identity,
    pin_combine_softmax_identity,
    pin_combine_f64_bound,
    pin_combine_f16_factors_and_out,
    pin_conversions,
    pin_golden_zeroing,
    pin_zeroing_vs_numpy,
    pin_golden_moe_sort,
    pin_moe_sort_vs_numpy,
    pin_e4m3_conversion,
    pin_quantize_rows,
    pin_quantize_non_finite,
]


def run_all(lib_path: str) -> None:
    """Run every pin against the oracle build at ``lib_path`` (raises on the
    first failing pin)."""
    lib = oracle.load(lib_path)
    for pin in ALL_PINS:
        pin(lib)
