"""The custom operators (torch.ops.mxmoe.*) on the GPU: each must write
exactly what the binding's call writes, bit for bit, and a step built from
them must trace whole under torch.compile (eager backend, no graph break) and
give the same bits as the eager step."""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import combine_topk_ids_expert_amd.ops  # noqa: F401  (registers torch.ops.mxmoe)
from tests import gpu_util as gu
from workloads import routing

pytestmark = pytest.mark.gpu

DEV = gu.DEV
T, E, K, H, A = 300, 64, 8, 1024, 16
META = ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
        "output_permutation", "blockscale_offsets")


def _inputs(seed=0):
    rng = np.random.default_rng(seed)
    ids = torch.from_numpy(routing.uniform_topk(rng, T, E, K)).to(DEV)
    w = torch.from_numpy(routing.softmax_weights(rng, T, K)).to(DEV)
    x = routing.normal_rows(T, H, "bf16", seed=seed + 1, device=DEV)
    return ids, w, x


def _routing():
    r = mx.empty_routing(T, K, E, DEV, row_align=A, blockscale=True)
    for v in r.values():
        v.fill_(-7 if v.dtype == torch.int32 else 0x5A)
    return r


def _same(a, b, what):
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8)), what


def _op_prepare(ids, r):
    torch.ops.mxmoe.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"],
                                      r["problem_sizes2"], r["input_permutation"],
                                      r["output_permutation"], E, 64, 32, r["blockscale_offsets"],
                                      A, 128, r["workspace"])


def _bind_prepare(ids, r):
    mx.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                         r["input_permutation"], r["output_permutation"], E, 64, 32,
                         r["blockscale_offsets"], row_align=A, workspace=r["workspace"])


def test_ops_write_what_the_binding_writes():
    print("case: torch.ops.mxmoe against the binding", flush=True)
    ids, w, x = _inputs()
    r1, r2 = _routing(), _routing()
    _op_prepare(ids, r1)
    _bind_prepare(ids, r2)
    for key in META:
        _same(r1[key], r2[key], key)
    cap = r1["input_permutation"].numel()
    perm, inp = r1["output_permutation"], r1["input_permutation"]

    def rows(dtype=torch.bfloat16, width=H):
        return torch.full((cap, width), float("nan"), device=DEV).to(dtype)

    a, b = rows(), rows()
    torch.ops.mxmoe.dispatch_rows(x, perm, K, a, None, None)
    mx.dispatch_rows(x, perm, K, b)
    _same(a, b, "dispatch_rows")
    a, b = rows(), rows()
    torch.ops.mxmoe.shuffle_rows(x, inp, a)
    mx.shuffle_rows(x, inp, b)
    _same(a, b, "shuffle_rows")

    y = routing.normal_rows(cap, H, "bf16", seed=5, device=DEV)
    o1 = torch.full((T, H), float("nan"), device=DEV)
    o2 = o1.clone()
    torch.ops.mxmoe.apply_shuffle_mul_sum(y, o1, perm, w)
    mx.apply_shuffle_mul_sum(y, o2, perm, w)
    _same(o1, o2, "apply_shuffle_mul_sum")

    o1, o2 = o1.fill_(3.0), o2.fill_(3.0)
    torch.ops.mxmoe.moe_output_memset(o1, perm, K)
    mx.moe_output_memset(o2, perm, K)
    _same(o1, o2, "moe_output_memset")

    a, b = rows(), rows()
    a.fill_(2.0)
    b.fill_(2.0)
    torch.ops.mxmoe.zero_padding_rows(a, inp, r1["expert_offsets"])
    mx.zero_padding_rows(b, inp, r1["expert_offsets"])
    _same(a, b, "zero_padding_rows")

    qa, qb = rows(torch.uint8), rows(torch.uint8)
    sa = torch.full((cap, H // 128), float("nan"), device=DEV)
    sb = sa.clone()
    torch.ops.mxmoe.dispatch_rows_fp8(x, perm, K, qa, sa)
    mx.dispatch_rows_fp8(x, perm, K, qb, sb)
    _same(qa, qb, "dispatch_rows_fp8 codes")
    _same(sa, sb, "dispatch_rows_fp8 scales")

    r3, r4 = _routing(), _routing()
    xa, xb = rows(), rows()
    torch.ops.mxmoe.prepare_dispatch(ids, r3["expert_offsets"], r3["problem_sizes1"],
                                     r3["problem_sizes2"], r3["input_permutation"],
                                     r3["output_permutation"], E, 64, 32, x, xa,
                                     r3["blockscale_offsets"], None, None, A, 128,
                                     r3["workspace"])
    mx.prepare_dispatch(ids, r4["expert_offsets"], r4["problem_sizes1"], r4["problem_sizes2"],
                        r4["input_permutation"], r4["output_permutation"], E, 64, 32, x, xb,
                        r4["blockscale_offsets"], row_align=A, workspace=r4["workspace"])
    for key in META:
        _same(r3[key], r4[key], "prepare_dispatch " + key)
    _same(xa, xb, "prepare_dispatch rows")

    tile, off, nl = 16, 8, 32
    s1 = mx.moe_sort(ids, E, off, nl, tile)
    s2 = {k_: torch.full_like(v, -7) for k_, v in s1.items()}
    ws = torch.empty(max(mx.prepare_workspace_size(T, K, nl), 4), dtype=torch.uint8, device=DEV)
    torch.ops.mxmoe.moe_sort(ids, E, off, nl, tile, s2["expanded_idx_to_permuted_idx"],
                             s2["permuted_idx_to_expanded_idx"], s2["tile_idx_to_group_idx"],
                             s2["tile_idx_to_mn_limit"], s2["total_num_padded_tokens"],
                             s2["num_non_exiting_tiles"], s2["expert_offsets"], ws)
    torch.cuda.synchronize()
    for k_ in s1:
        _same(s1[k_], s2[k_], "moe_sort " + k_)


def _step(ids, w, x, r, xd, y, out):
    torch.ops.mxmoe.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"],
                                      r["problem_sizes2"], r["input_permutation"],
                                      r["output_permutation"], E, 64, 32, r["blockscale_offsets"],
                                      A, 128, r["workspace"])
    torch.ops.mxmoe.dispatch_rows(x, r["output_permutation"], K, xd, None, None)
    y.copy_(xd)            # stands in for the expert GEMMs
    torch.ops.mxmoe.apply_shuffle_mul_sum(y, out, r["output_permutation"], w)
    return out


def test_step_traces_whole_under_torch_compile():
    print("case: torch.compile (eager backend, fullgraph) over the operators", flush=True)
    ids, w, x = _inputs(3)
    bufs = []
    for _ in range(2):
        r = _routing()
        cap = r["input_permutation"].numel()
        xd = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
        y = torch.zeros_like(xd)
        out = torch.full((T, H), float("nan"), device=DEV)
        bufs.append((r, xd, y, out))
    torch._dynamo.reset()
    compiled = torch.compile(_step, backend="eager", fullgraph=True)
    got = compiled(ids, w, x, *bufs[0])
    want = _step(ids, w, x, *bufs[1])
    torch.cuda.synchronize()
    _same(got, want, "compiled step")
    for key in META:
        _same(bufs[0][0][key], bufs[1][0][key], key)


def test_opcheck_on_the_row_operators():
    print("case: torch.library.opcheck", flush=True)
    ids, w, x = _inputs(7)
    r = _routing()
    _bind_prepare(ids, r)
    torch.cuda.synchronize()
    cap = r["input_permutation"].numel()
    y = routing.normal_rows(cap, H, "bf16", seed=9, device=DEV)
    out = torch.zeros((T, H), device=DEV)
    torch.library.opcheck(torch.ops.mxmoe.apply_shuffle_mul_sum.default,
                          (y, out, r["output_permutation"], w))
    xd = torch.zeros((cap, H), dtype=torch.bfloat16, device=DEV)
    torch.library.opcheck(torch.ops.mxmoe.dispatch_rows.default,
                          (x, r["output_permutation"], K, xd, None, None))
