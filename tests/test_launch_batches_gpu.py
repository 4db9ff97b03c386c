"""Calls whose rows need more than one kernel launch (needs the GPU).

The row kernels put at most 2^31 work-items in one launch, so a call with
more rows goes out as several launches over consecutive row ranges.  With
16-byte rows (and with 128-element rows in the FP8 dispatch) a row is one
64-thread workgroup, so 2^25 rows fill a launch.  These cases use 2^25 + 1000
rows and check the rows on both sides of that boundary, the first and last
rows and a random sample against the oracle, and every row through a
whole-array property of the definition.
"""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

DEV = gu.DEV
B = 1 << 25           # rows of one launch at 64 threads per row
N = B + 1000


def _print_case(*args):
    print("case:", *args, flush=True)


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _sample(n, seed):
    rng = np.random.default_rng(seed)
    s = np.concatenate([np.arange(B - 300, B + 300), rng.choice(n, 1000, replace=False), [0, n - 1]])
    return np.unique(s)


def _rows(t, idx):
    return gu.bits(t[torch.from_numpy(idx.astype(np.int64)).to(DEV)])


def test_shuffle_rows_over_launches():
    _print_case("shuffle_rows", N, "rows of 16 B")
    n_src = 1 << 20
    g = _gen(1)
    src = torch.randint(-2**31, 2**31 - 1, (n_src, 4), dtype=torch.int32, device=DEV, generator=g)
    m = torch.randint(-1, n_src + 1, (N,), dtype=torch.int32, device=DEV, generator=g)
    dst = torch.full((N, 4), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    mx.shuffle_rows(src, m, dst)
    torch.cuda.synchronize()
    s = _sample(N, 1)
    m_s = gu.bits(m)[s]
    want = oracle.shuffle_rows(gu.bits(src), m_s, dst=np.full((s.size, 4), 0x5A5A5A5A, np.int32))
    np.testing.assert_array_equal(_rows(dst, s), want)
    ok = (m >= 0) & (m < n_src)
    assert torch.equal(dst[ok], src[m[ok].long()])
    assert bool((dst[~ok] == 0x5A5A5A5A).all())


def test_dispatch_rows_over_launches():
    _print_case("dispatch_rows", N, "tokens, k=1, rows of 16 B")
    g = _gen(2)
    x = torch.randint(-2**31, 2**31 - 1, (N, 4), dtype=torch.int32, device=DEV, generator=g)
    perm = torch.randperm(N, device=DEV, generator=g).to(torch.int32)
    xd = torch.zeros((N, 4), dtype=torch.int32, device=DEV)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for e in ev:
        e.record()
    mx.dispatch_rows(x, perm, 1, xd, kernel_events=ev)    # start with the first launch, stop with the last
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) > 0.0
    s = _sample(N, 2)                                  # tokens
    p_s = gu.bits(perm)[s]
    inv = np.argsort(p_s)                              # sampled destination rows, in row order
    want = oracle.shuffle_rows(_rows(x, s), inv.astype(np.int32))
    np.testing.assert_array_equal(_rows(xd, p_s[inv]), want)
    assert torch.equal(xd[perm.long()], x)


def test_combine_over_launches():
    _print_case("apply_shuffle_mul_sum", N, "tokens, k=1, hidden 8 bf16")
    g = _gen(3)
    y = torch.randn((N, 8), dtype=torch.float32, device=DEV, generator=g).to(torch.bfloat16)
    perm = torch.randperm(N, device=DEV, generator=g).to(torch.int32)
    f = torch.rand((N, 1), dtype=torch.float32, device=DEV, generator=g) + 0.5
    out = torch.empty((N, 8), dtype=torch.bfloat16, device=DEV)
    mx.apply_shuffle_mul_sum(y, out, perm, f)
    torch.cuda.synchronize()
    s = _sample(N, 3)
    p_s = gu.bits(perm)[s]
    sub_y = _rows(y, p_s)                              # the sampled tokens' rows, in token order
    want = oracle.apply_shuffle_mul_sum(sub_y, "bf16", np.arange(s.size, dtype=np.int32),
                                        gu.bits(f)[s], "f32", s.size, 1, "bf16")
    np.testing.assert_array_equal(_rows(out, s), want)
    # one pick: fma(v, w, +0) is v * w rounded once to fp32 (+0 for a zero
    # product), then rounded to bf16
    ref = (y[perm.long()].float() * f + 0.0).to(torch.bfloat16)
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_output_memset_over_launches():
    _print_case("moe_output_memset", N, "tokens, k=1, rows of 16 B")
    g = _gen(4)
    out = torch.full((N, 4), 0x33333333, dtype=torch.int32, device=DEV)
    perm = torch.randint(-1, 2, (N,), dtype=torch.int32, device=DEV, generator=g)
    mx.moe_output_memset(out, perm, 1)
    torch.cuda.synchronize()
    s = _sample(N, 4)
    want = oracle.output_memset(np.full((s.size, 4), 0x33333333, np.int32), 1, gu.bits(perm)[s])
    np.testing.assert_array_equal(_rows(out, s), want)
    hit = perm >= 0
    assert bool((out[hit] == 0).all()) and bool((out[~hit] == 0x33333333).all())


def test_zero_padding_over_launches():
    _print_case("zero_padding_rows", N, "rows of 16 B, no expert offsets")
    g = _gen(5)
    rows = torch.full((N, 4), 0x66666666, dtype=torch.int32, device=DEV)
    inp = torch.randint(-1, 2, (N,), dtype=torch.int32, device=DEV, generator=g)
    mx.zero_padding_rows(rows, inp)
    torch.cuda.synchronize()
    s = _sample(N, 5)
    want = oracle.zero_padding_rows(np.full((s.size, 4), 0x66666666, np.int32), gu.bits(inp)[s])
    np.testing.assert_array_equal(_rows(rows, s), want)
    pad = inp < 0
    assert bool((rows[pad] == 0).all()) and bool((rows[~pad] == 0x66666666).all())


def test_dispatch_fp8_over_launches():
    _print_case("dispatch_rows_fp8", N, "tokens, k=1, hidden 128")
    g = _gen(6)
    x = torch.randn((N, 128), dtype=torch.float32, device=DEV, generator=g).to(torch.bfloat16)
    perm = torch.randperm(N, device=DEV, generator=g).to(torch.int32)
    q = torch.zeros((N, 128), dtype=torch.uint8, device=DEV)
    sc = torch.zeros((N, 1), dtype=torch.float32, device=DEV)
    mx.dispatch_rows_fp8(x, perm, 1, q, sc)
    torch.cuda.synchronize()
    s = _sample(N, 6)
    p_s = gu.bits(perm)[s]
    want_q, want_s = oracle.quantize_fp8_rows(_rows(x, s))
    np.testing.assert_array_equal(_rows(q, p_s), want_q)
    np.testing.assert_array_equal(_rows(sc, p_s), want_s)
    # every destination row was written: a group of N(0,1) values has a
    # positive amax, so its scale is positive
    assert bool((sc > 0).all())
