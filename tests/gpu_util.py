"""Helpers for the GPU parity tests: run the HIP path through the binding and
the oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import numpy as np
import torch

import combine_topk_ids_expert_amd as mx
import oracle

DEV = "cuda:0"
SENTINEL = 0xA5

_TORCH_CODE = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's elements as raw bit patterns (float32 stays
    float32 values, 16-bit floats become uint16, fp8 uint8)."""
    t = t.detach().contiguous().cpu()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def code(dtype: torch.dtype) -> str:
    return _TORCH_CODE[dtype]


def gpu_prepare(ids: np.ndarray, E: int, row_align: int = 1, blockscale: bool = True,
                ids_dtype=torch.int64, n: int = 64, k: int = 32) -> dict:
    T, topk = ids.shape
    r = mx.empty_routing(T, topk, E, DEV, row_align=row_align, blockscale=blockscale)
    # poison every output so a missing write shows
    for key in ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
                "output_permutation", "blockscale_offsets", "workspace"):
        if r[key] is not None:
            r[key].fill_(-7 if r[key].dtype == torch.int32 else 0x5A)
    t_ids = torch.from_numpy(np.ascontiguousarray(ids)).to(ids_dtype).to(DEV)
    mx.prepare_moe_input(t_ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                         r["input_permutation"], r["output_permutation"], E, n, k,
                         r["blockscale_offsets"], row_align=row_align, workspace=r["workspace"])
    torch.cuda.synchronize()
    out = {key: (v.cpu().numpy() if v is not None else None) for key, v in r.items()
           if key != "workspace"}
    out["_t"] = r
    return out


def check_prepare(ids: np.ndarray, E: int, row_align: int = 1, ids_dtype=torch.int64,
                  n: int = 64, k: int = 32) -> dict:
    """GPU metadata == oracle metadata, bit for bit, for every output array."""
    g = gpu_prepare(ids, E, row_align, True, ids_dtype, n, k)
    o = oracle.prepare_moe_input(ids.astype(np.int64), E, row_align=row_align,
                                 blockscale_align=128, gemm=(2 * n, k, k, n))
    for key in ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
                "output_permutation", "blockscale_offsets"):
        np.testing.assert_array_equal(g[key].reshape(o[key].shape), o[key], err_msg=key)
    return g


def check_dispatch(x: torch.Tensor, meta: dict, topk: int, scales: torch.Tensor | None = None):
    """dispatch_rows and shuffle_rows write exactly the oracle's rows (bit for
    bit) and leave padding / unused rows untouched."""
    inp_t = meta["_t"]["input_permutation"]
    outp_t = meta["_t"]["output_permutation"]
    rows = inp_t.numel()
    inp = meta["input_permutation"]
    used = inp >= 0
    x_host = bits(x)
    want = oracle.shuffle_rows(x_host, inp)
    for mode in ("scatter", "gather"):
        xd = torch.empty((rows,) + tuple(x.shape[1:]), dtype=x.dtype, device=DEV)
        xd.view(torch.uint8).fill_(SENTINEL)
        sd = None
        if scales is not None:
            sd = torch.full((rows,) + tuple(scales.shape[1:]), float("nan"), dtype=scales.dtype,
                            device=DEV)
        if mode == "scatter":
            mx.dispatch_rows(x, outp_t, topk, xd, scales, sd)
        else:
            mx.shuffle_rows(x, inp_t, xd)
            if scales is not None:
                mx.shuffle_rows(scales, inp_t, sd)
        torch.cuda.synchronize()
        got = bits(xd)
        np.testing.assert_array_equal(got[used], want[used], err_msg=mode)
        raw = xd.view(torch.uint8).cpu().numpy().reshape(rows, int(np.prod(xd.shape[1:])) * xd.element_size())
        assert np.all(raw[~used] == SENTINEL), f"{mode} wrote a padding row"
        if scales is not None:
            sw = oracle.shuffle_rows(bits(scales), inp)
            sg = bits(sd)
            np.testing.assert_array_equal(sg[used], sw[used], err_msg=mode + " scales")
            assert np.all(np.isnan(sg[~used]))


def check_combine(y: torch.Tensor, perm: torch.Tensor, factors: torch.Tensor | None,
                  out_dtype: torch.dtype, T: int, exact: bool = True):
    """apply_shuffle_mul_sum == oracle: bit-exact (same fma order and rounding)
    and, stated separately, within the bar: rtol 1.6e-2 / atol 1e-2 for 16-bit
    outputs, rtol 1e-5 for fp32."""
    H = y.shape[1]
    out = torch.full((T, H), float("nan"), dtype=out_dtype, device=DEV)
    mx.apply_shuffle_mul_sum(y, out, perm, factors)
    torch.cuda.synchronize()
    topk = perm.numel() // T if T else 1
    fd = code(factors.dtype) if factors is not None else "f32"
    want = oracle.apply_shuffle_mul_sum(bits(y), code(y.dtype), bits(perm),
                                        bits(factors) if factors is not None else None, fd,
                                        T, topk, code(out_dtype))
    got = bits(out)
    if out_dtype == torch.float32:
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=0)
    else:
        gf = out.float().cpu().numpy()
        wf = torch.from_numpy(want.view(np.int16)).view(
            torch.bfloat16 if out_dtype == torch.bfloat16 else torch.float16).float().numpy()
        np.testing.assert_allclose(gf, wf, rtol=1.6e-2, atol=1e-2)
    if exact:
        np.testing.assert_array_equal(got, want)
    return out
