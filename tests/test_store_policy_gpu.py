"""Calls on both sides of the 256 MiB store-policy switch (needs the GPU).

The row dispatch stores its destination rows streaming while the source rows
fit in 256 MiB and allocating beyond; the combine stores its output rows
allocating while the output fits in 256 MiB and streaming beyond.  Each side
is a different kernel instantiation, so each case here runs one call just
below and one just above the switch and checks sampled rows against the
oracle and every row against a whole-array property of the definition.
"""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
DEV = gu.DEV
SWITCH = 256 << 20
H = 7168


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _rows(t, idx):
    return gu.bits(t[torch.from_numpy(idx.astype(np.int64)).to(DEV)])


# 14 336-byte bf16 rows: 18 724 rows are just under 256 MiB, 18 725 just over.
@pytest.mark.parametrize("T", [18724, 18725])
def test_dispatch_either_side_of_switch(T):
    print("case: dispatch_rows at the policy switch", T, "tokens, k=1", flush=True)
    assert (T * H * 2 > SWITCH) == (T == 18725)
    g = _gen(T)
    x = torch.randn((T, H), dtype=torch.float32, device=DEV, generator=g).to(torch.bfloat16)
    perm = torch.randperm(T, device=DEV, generator=g).to(torch.int32)
    xd = torch.zeros((T, H), dtype=torch.bfloat16, device=DEV)
    mx.dispatch_rows(x, perm, 1, xd)
    torch.cuda.synchronize()
    s = np.unique(np.random.default_rng(T).choice(T, 400, replace=False))
    p_s = gu.bits(perm)[s]
    inv = np.argsort(p_s)
    want = oracle.shuffle_rows(_rows(x, s), inv.astype(np.int32))
    np.testing.assert_array_equal(_rows(xd, p_s[inv]), want)
    assert torch.equal(xd[perm.long()].view(torch.int16), x.view(torch.int16))


# fp32 output rows of 28 672 bytes: 9 362 tokens are just under 256 MiB,
# 9 363 just over.
@pytest.mark.parametrize("T", [9362, 9363])
def test_combine_either_side_of_switch(T):
    print("case: apply_shuffle_mul_sum at the policy switch", T, "tokens, k=1, fp32 out",
          flush=True)
    assert (T * H * 4 > SWITCH) == (T == 9363)
    g = _gen(T + 1)
    y = torch.randn((T, H), dtype=torch.float32, device=DEV, generator=g).to(torch.bfloat16)
    perm = torch.randperm(T, device=DEV, generator=g).to(torch.int32)
    f = torch.rand((T, 1), dtype=torch.float32, device=DEV, generator=g) + 0.5
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device=DEV)
    mx.apply_shuffle_mul_sum(y, out, perm, f)
    torch.cuda.synchronize()
    s = np.unique(np.random.default_rng(T).choice(T, 200, replace=False))
    p_s = gu.bits(perm)[s]
    want = oracle.apply_shuffle_mul_sum(_rows(y, p_s), "bf16", np.arange(s.size, dtype=np.int32),
                                        gu.bits(f)[s], "f32", s.size, 1, "f32")
    np.testing.assert_array_equal(_rows(out, s), want)
    # one pick: fma(v, w, +0) is v * w rounded once to fp32 (+0 for a zero product)
    ref = y[perm.long()].float() * f + 0.0
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32))
