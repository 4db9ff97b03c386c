"""HIP path against the CPU oracle, element by element (needs the GPU).

Metadata, permutations and dispatched rows must match bit for bit; the
combine must be within rtol 1.6e-2 / atol 1e-2 (16-bit output) or rtol 1e-5
(fp32 output), and is also expected to match bit for bit because both sides
take the same fused multiply-add order.  Sizes span several routing tiles
(512 to 4096 picks each) with ragged tails, rows wider than one workgroup chunk,
and every workload's real shape at a reduced token count; at full size every
metadata entry, every dispatched row and every combined token is compared.
"""

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
import oracle
from tests import gpu_util as gu
from workloads import WORKLOADS, build_inputs, routing
from workloads.configs import expert_output

pytestmark = pytest.mark.gpu

DEV = gu.DEV


def _print_case(*args):
    print("case:", *args, flush=True)


# --------------------------------------------------------------------------
# prepare_moe_input
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,A,mode,bad", [
    (0, 256, 8, 1, "uniform", 0.0),
    (1, 256, 8, 1, "uniform", 0.0),
    (7, 5, 3, 4, "dups", 0.2),
    (32, 256, 8, 1, "uniform", 0.0),
    (128, 256, 8, 128, "uniform", 0.0),         # one launch, padded: 1024 picks
    (129, 256, 8, 128, "uniform", 0.0),         # medium path, heavy padding: 1032 picks, 3 tiles
    (256, 256, 8, 1, "uniform", 0.0),           # one launch, unpadded: 2048 picks
    (257, 256, 8, 1, "uniform", 0.0),           # medium path: 2056 picks, 5 tiles
    (1000, 256, 8, 128, "uniform", 0.0),        # medium path, 16 tiles, padded
    (1024, 1024, 8, 1, "uniform", 0.05),       # medium path at its limit: 8192 picks, E = 1024
    (1000, 1, 8, 1, "dups", 0.0),               # medium path, every pick on one expert
    (900, 8, 8, 2, "dups", 0.02),               # medium path, 8 experts
    (1025, 256, 8, 1, "uniform", 0.0),          # two launches from 8200 picks, ragged last tile
    (8192, 256, 8, 1, "uniform", 0.0),          # 65536 picks, E = 256: 64 tiles of 1024
    (8193, 256, 8, 128, "uniform", 0.02),       # tiles grow past 1024 picks
    (8192, 128, 8, 1, "uniform", 0.0),          # 65536 picks, E = 128: 128 tiles of 512
    (8193, 128, 8, 1, "uniform", 0.0),          # 65 tiles of 1024: table rows of 17 vectors
    (9000, 1024, 8, 1, "uniform", 0.01),        # tile count held up by the one-round floor
    (3000, 1000, 8, 4, "uniform", 0.05),        # E not a power of two, invalid ids
    (2000, 100, 8, 8, "k_hot", 0.0),
    (4000, 8, 4, 1, "dups", 0.0),               # few experts, many duplicates
    (3001, 256, 8, 128, "uniform", 0.05),       # several tiles, ragged tail, invalid ids
    (4096, 256, 8, 128, "uniform", 0.0),
    (5000, 256, 8, 1, "k_hot", 0.0),
    (4000, 128, 8, 1, "zipf", 0.0),
    (3000, 1024, 8, 16, "uniform", 0.0),        # largest expert count
    (2500, 1, 4, 1, "dups", 0.0),               # one expert takes everything
    (700, 33, 70, 3, "dups", 0.1),              # topk > 64
])
@pytest.mark.parametrize("ids_dtype", [torch.int32, torch.int64])
def test_prepare_matches_oracle(T, E, k, A, mode, bad, ids_dtype):
    _print_case("prepare", T, E, k, A, mode, bad, ids_dtype)
    rng = np.random.default_rng(T * 7 + E)
    if mode == "dups":
        ids = rng.integers(0, E, (T, k))
    elif mode == "k_hot":
        ids = routing.k_hot_topk(rng, T, E, k, 8, 0.8)
    elif mode == "zipf":
        ids = routing.zipf_topk(rng, T, E, k, 1.2)
    else:
        ids = routing.uniform_topk(rng, T, E, k)
    if bad:
        m = rng.random(ids.shape) < bad
        ids = np.where(m, rng.choice([-1, -5, E, E + 77], size=ids.shape), ids)
    gu.check_prepare(ids, E, A, ids_dtype)


def test_prepare_all_invalid_and_int64_extremes():
    _print_case("prepare invalid")
    ids = np.full((5000, 8), 300, np.int64)
    ids[::3, 1] = -(2**40)
    ids[::5, 2] = 2**40
    gu.check_prepare(ids, 256, 128, torch.int64)


def test_prepare_deterministic_across_calls():
    _print_case("prepare twice")
    rng = np.random.default_rng(5)
    ids = routing.k_hot_topk(rng, 6000, 256, 8, 8, 0.8)
    a = gu.gpu_prepare(ids, 256, 128)
    b = gu.gpu_prepare(ids, 256, 128)
    for key in ("expert_offsets", "input_permutation", "output_permutation"):
        np.testing.assert_array_equal(a[key], b[key])


def test_prepare_workspace_of_another_dtype():
    """A workspace tensor is sized in bytes whatever its dtype: an int32
    tensor of exactly the bytes mx_prepare_workspace_size asks for is enough,
    and one byte fewer is refused."""
    _print_case("prepare with an int32 workspace")
    T, E, k = 4096, 256, 8
    need = mx.prepare_workspace_size(T, k, E)
    assert need > 0 and need % 4 == 0
    rng = np.random.default_rng(12)
    ids = routing.uniform_topk(rng, T, E, k).astype(np.int64)
    t_ids = torch.from_numpy(ids).to(DEV)
    r = mx.empty_routing(T, k, E, DEV)
    ws = torch.empty(need // 4, dtype=torch.int32, device=DEV)
    mx.prepare_moe_input(t_ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                         r["input_permutation"], r["output_permutation"], E, 64, 32,
                         workspace=ws)
    torch.cuda.synchronize()
    o = oracle.prepare_moe_input(ids, E)
    np.testing.assert_array_equal(r["output_permutation"].cpu().numpy(), o["output_permutation"])
    np.testing.assert_array_equal(r["input_permutation"].cpu().numpy(), o["input_permutation"])
    short = torch.empty(need - 1, dtype=torch.uint8, device=DEV)
    with pytest.raises(mx.MxError) as err:
        mx.prepare_moe_input(t_ids, r["expert_offsets"], None, None, r["input_permutation"],
                             r["output_permutation"], E, 64, 32, workspace=short)
    assert err.value.status == 4


# --------------------------------------------------------------------------
# dispatch rows (scatter and gather)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,dtype,E,k,A", [
    (37, 7168, torch.bfloat16, 64, 8, 128),     # 14 KiB rows
    (300, 4096, torch.bfloat16, 256, 8, 1),
    (50, 100, torch.bfloat16, 16, 4, 8),        # 200 B rows: 8-byte accesses
    (40, 7, torch.bfloat16, 8, 3, 1),           # 14 B rows: 2-byte accesses
    (33, 13, torch.uint8, 8, 2, 4),             # 13 B rows: byte accesses
    (20, 20000, torch.float32, 16, 2, 1),       # 80 KB rows: several column chunks
    (64, 1024, torch.float16, 32, 70, 1),       # topk > 64
])
def test_dispatch_matches_oracle(T, H, dtype, E, k, A):
    _print_case("dispatch", T, H, dtype, E, k, A)
    rng = np.random.default_rng(T + H)
    ids = rng.integers(-1, E + 1, (T, k))
    meta = gu.check_prepare(ids, E, A)
    if dtype == torch.uint8:
        x = torch.from_numpy(rng.integers(0, 256, (T, H), dtype=np.uint8)).to(DEV)
    else:
        x = routing.normal_rows(T, H, gu.code(dtype), seed=T, device=DEV)
    gu.check_dispatch(x, meta, k)


def test_shuffle_rows_takes_an_output_shape():
    """sglang's shuffle_rows takes the output's shape; so does this one."""
    _print_case("shuffle_rows with an output shape")
    rng = np.random.default_rng(4)
    x = torch.randn((50, 384), device=DEV).to(torch.bfloat16)
    m = torch.from_numpy(rng.integers(-2, 52, 70).astype(np.int32)).to(DEV)
    got = mx.shuffle_rows(x, m, (70, 384))
    torch.cuda.synchronize()
    assert got.shape == (70, 384) and got.dtype == torch.bfloat16
    want = oracle.shuffle_rows(gu.bits(x), m.cpu().numpy())
    used = (m.cpu().numpy() >= 0) & (m.cpu().numpy() < 50)
    np.testing.assert_array_equal(gu.bits(got)[used], want[used])


def test_dispatch_misaligned_base():
    """A base pointer off the 16-byte grid takes a narrower access width and
    still copies exactly."""
    _print_case("dispatch misaligned")
    T, H, E, k = 64, 512, 32, 4
    rng = np.random.default_rng(9)
    meta = gu.check_prepare(routing.uniform_topk(rng, T, E, k), E, 1)
    big = routing.normal_rows(T * H + 1, 1, "bf16", seed=3, device=DEV).view(-1)
    x = big[1:].view(T, H)                               # 2-byte offset
    assert x.data_ptr() % 16 != 0
    gu.check_dispatch(x, meta, k)


def test_calls_follow_the_current_stream():
    """The binding launches on torch's current stream: inside a side-stream
    context the raw handle it passes is that stream's, and prepare, dispatch
    and combine queued there (with the poisoning fills of their outputs on
    the same stream) still match the oracle."""
    _print_case("side stream")
    dev = torch.device(DEV)
    assert mx._stream(dev) == torch.cuda.current_stream(dev).cuda_stream
    side = torch.cuda.Stream(device=dev)
    rng = np.random.default_rng(77)
    T, E, k, H = 3001, 256, 8, 1024
    ids = routing.uniform_topk(rng, T, E, k)
    with torch.cuda.stream(side):
        assert mx._stream(dev) == side.cuda_stream
        assert side.cuda_stream != torch.cuda.default_stream(dev).cuda_stream
        meta = gu.check_prepare(ids, E, 128)
        gu.check_dispatch(routing.normal_rows(T, H, "bf16", seed=5, device=DEV), meta, k)
        y = routing.normal_rows(meta["input_permutation"].size, H, "bf16", seed=6, device=DEV)
        f = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(DEV)
        gu.check_combine(y, meta["_t"]["output_permutation"], f, torch.bfloat16, T)


def test_dispatch_fp8_with_scale_rows():
    _print_case("dispatch fp8")
    w = WORKLOADS["zipf1.2_T16384_H4096fp8_E128_k8"]
    inp = build_inputs(w, DEV, T=1500)
    meta = gu.check_prepare(inp["ids"], w.E, 1)
    gu.check_dispatch(inp["x"], meta, w.k, inp["scales"])


def _raw(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy().reshape(t.shape[0], -1)


@pytest.mark.parametrize("T,H,E,k,side_cols,side_dtype", [
    (77, 256, 16, 8, 56, torch.float32),     # 224-byte side rows, 14 vectors of 16 bytes
    (130, 512, 32, 10, 3, torch.float32),    # 12-byte side rows (4-byte vectors), k > 8
    (65, 1024, 8, 3, 7, torch.uint8),        # 7-byte side rows (single bytes)
    (40, 128, 16, 8, 600, torch.float32),    # side rows wider than the workgroup
    (20, 16400, 8, 8, 56, torch.float32),    # 17 column chunks per row
    (50, 256, 8, 1, 32, torch.float32),      # k = 1
    (1, 64, 4, 2, 32, torch.float32),        # one token
])
def test_dispatch_side_row_shapes(T, H, E, k, side_cols, side_dtype):
    """dispatch_rows with side rows of several widths, where some picks are
    dropped (-1 in the output permutation): row and side row of token t land
    in every destination t*k + j names, bit for bit as the oracle's gather
    with the inverse map, and no other row is written."""
    _print_case("dispatch side rows", T, H, E, k, side_cols, side_dtype)
    rng = np.random.default_rng(T * 31 + side_cols)
    ids = routing.uniform_topk(rng, T, E, k)
    meta = gu.check_prepare(ids, E, 1)
    outp = meta["_t"]["output_permutation"].clone()
    outp.view(T, k)[::5] = -1                          # tokens with no pick kept
    outp.view(-1)[3::7] = -1                           # and single dropped picks
    rows = meta["_t"]["input_permutation"].numel()
    outp_h = outp.cpu().numpy().reshape(-1)
    d2s = np.full(rows, -1, dtype=np.int32)
    for i, r in enumerate(outp_h):
        if r >= 0:
            d2s[r] = i // k
    used = d2s >= 0
    x = routing.normal_rows(T, H, "bf16", seed=T + 1, device=DEV)
    if side_dtype == torch.uint8:
        side = torch.from_numpy(rng.integers(0, 256, (T, side_cols), dtype=np.uint8)).to(DEV)
    else:
        side = torch.from_numpy(rng.standard_normal((T, side_cols)).astype(np.float32)).to(DEV)
    xd = torch.empty((rows, H), dtype=x.dtype, device=DEV)
    sd = torch.empty((rows, side_cols), dtype=side.dtype, device=DEV)
    xd.view(torch.uint8).fill_(gu.SENTINEL)
    sd.view(torch.uint8).fill_(gu.SENTINEL)
    mx.dispatch_rows(x, outp, k, xd, side, sd)
    torch.cuda.synchronize()
    for got, src, what in ((xd, x, "rows"), (sd, side, "side rows")):
        want = oracle.shuffle_rows(_raw(src), d2s)
        g = _raw(got)
        np.testing.assert_array_equal(g[used], want[used], err_msg=what)
        assert np.all(g[~used] == gu.SENTINEL), f"{what}: a row no pick names was written"


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ydt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float16, torch.float32])
@pytest.mark.parametrize("fdt", [None, torch.float32, torch.bfloat16, torch.float16])
def test_combine_dtypes(ydt, odt, fdt):
    _print_case("combine", ydt, odt, fdt)
    T, H, k, R = 150, 512, 8, 1500
    rng = np.random.default_rng(42)
    y = routing.normal_rows(R, H, gu.code(ydt), seed=11, device=DEV)
    perm = torch.from_numpy(rng.integers(0, R, T * k).astype(np.int32)).to(DEV)
    f = None
    if fdt is not None:
        f = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(fdt).to(DEV)
    gu.check_combine(y, perm, f, odt, T)


@pytest.mark.parametrize("T,H,k,R", [
    (33, 7168, 8, 400),        # 896 threads per token
    (20, 16400, 8, 200),       # two column chunks with a ragged end
    (50, 104, 8, 300),         # short rows, vector path
    (40, 77, 3, 90),           # H % 8 != 0: scalar path
    (30, 256, 9, 300),         # pick batch remainder
    (25, 64, 70, 500),         # topk > 64
    (1, 8, 1, 1),
])
def test_combine_shapes(T, H, k, R):
    _print_case("combine shape", T, H, k, R)
    rng = np.random.default_rng(T * H)
    y = routing.normal_rows(R, H, "bf16", seed=R, device=DEV)
    p = rng.integers(0, R, T * k).astype(np.int32)
    p[rng.random(p.size) < 0.1] = -1
    p[rng.random(p.size) < 0.05] = R + 3                 # out of range: skipped
    perm = torch.from_numpy(p).to(DEV)
    f = torch.from_numpy(rng.standard_normal((T, k)).astype(np.float32)).to(DEV)
    gu.check_combine(y, perm, f, torch.bfloat16, T)
    gu.check_combine(y, perm, f, torch.float32, T)


@pytest.mark.parametrize("ydt,odt", [
    (torch.bfloat16, torch.bfloat16), (torch.bfloat16, torch.float16),
    (torch.float32, torch.float32), (torch.float16, torch.bfloat16),
])
def test_combine_non_finite(ydt, odt):
    """NaN stays NaN and infinities propagate: y rows holding NaN, +inf and
    -inf (so some sums are inf - inf), and finite values large enough that
    the weighted sum overflows the output format to +-inf.  NaN payloads are
    not unique (the hardware conversion may pick another quiet NaN), so the
    NaN positions must agree and every other output must match bit for bit."""
    _print_case("combine non-finite", ydt, odt)
    T, H, k, R = 40, 256, 4, 60
    rng = np.random.default_rng(31)
    big = {torch.float16: 6e4, torch.bfloat16: 3e38, torch.float32: 3e38}[ydt]
    yh = rng.standard_normal((R, H)).astype(np.float32)
    yh[rng.random((R, H)) < 0.03] = np.nan
    yh[rng.random((R, H)) < 0.03] = np.inf
    yh[rng.random((R, H)) < 0.03] = -np.inf
    yh[rng.random((R, H)) < 0.05] = big
    y = torch.from_numpy(yh).to(ydt).to(DEV)
    perm = torch.from_numpy(rng.integers(0, R, T * k).astype(np.int32)).to(DEV)
    f = torch.from_numpy(rng.uniform(0.5, 2.0, (T, k)).astype(np.float32)).to(DEV)
    out = torch.zeros(T, H, dtype=odt, device=DEV)
    mx.apply_shuffle_mul_sum(y, out, perm, f)
    torch.cuda.synchronize()
    want = oracle.apply_shuffle_mul_sum(gu.bits(y), gu.code(ydt), gu.bits(perm), gu.bits(f), "f32",
                                        T, k, gu.code(odt))
    got = gu.bits(out)
    got_nan = torch.isnan(out.float()).cpu().numpy()
    if odt == torch.float32:
        want_nan = np.isnan(want)
    else:
        want_nan = torch.isnan(torch.from_numpy(want.view(np.int16)).view(odt).float()).numpy()
    assert want_nan.any() and np.isinf(out.float().cpu().numpy()).any()
    np.testing.assert_array_equal(got_nan, want_nan)
    np.testing.assert_array_equal(got[~got_nan], want[~want_nan])


def test_combine_misaligned_base():
    _print_case("combine misaligned")
    T, H, k, R = 16, 256, 4, 64
    rng = np.random.default_rng(3)
    big = routing.normal_rows(R * H + 1, 1, "bf16", seed=5, device=DEV).view(-1)
    y = big[1:].view(R, H)
    perm = torch.from_numpy(rng.integers(0, R, T * k).astype(np.int32)).to(DEV)
    gu.check_combine(y, perm, None, torch.bfloat16, T)


def test_combine_identity_experts_reproduce_x():
    """Closed form on the GPU: identity experts with weights 1/8 give x back
    bit for bit (the partial sums are exact)."""
    _print_case("combine identity")
    T, H, E, k = 500, 1024, 64, 8
    rng = np.random.default_rng(8)
    ids = routing.uniform_topk(rng, T, E, k)
    meta = gu.gpu_prepare(ids, E, 128)
    x = routing.normal_rows(T, H, "bf16", seed=1, device=DEV)
    xd = torch.empty(meta["_t"]["input_permutation"].numel(), H, dtype=torch.bfloat16, device=DEV)
    mx.dispatch_rows(x, meta["_t"]["output_permutation"], k, xd)
    out = torch.empty_like(x)
    mx.apply_shuffle_mul_sum(xd, out, meta["_t"]["output_permutation"],
                             torch.full((T, k), 0.125, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


# --------------------------------------------------------------------------
# every workload end to end at a reduced token count (same E, H, k, routing)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_end_to_end_reduced(name):
    w = WORKLOADS[name]
    T = min(w.T, 2048)
    _print_case("workload reduced", name, T)
    inp = build_inputs(w, DEV, T=T)
    meta = gu.check_prepare(inp["ids"], w.E, w.row_align)
    gu.check_dispatch(inp["x"], meta, w.k, inp["scales"])
    rows = meta["_t"]["input_permutation"].numel()
    y = expert_output(w, rows, DEV)
    f = torch.from_numpy(inp["weights"]).to(DEV)
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.out_dtype]
    gu.check_combine(y, meta["_t"]["output_permutation"], f, odt, T)


# --------------------------------------------------------------------------
# full sizes, launched as the benchmark launches them: every metadata entry,
# every dispatched row and every combined token against the oracle
# --------------------------------------------------------------------------

def _oracle_combine_all(y, perm_all, weights, T, k, out_dtype, chunk=2048):
    """The oracle's combine over all T tokens, in token chunks: each chunk
    reads only the y rows its picks name (gathered on the device and copied
    to the host, then renumbered), so the host never holds all of y.  The
    chunks run on threads (the C oracle releases the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    rows = y.shape[0]
    perm_all = perm_all.reshape(T, k)
    outs = {}

    def host_chunk(t0):
        t1 = min(T, t0 + chunk)
        perm = perm_all[t0:t1]
        need = np.unique(perm[perm >= 0])
        remap = np.full(rows, -1, np.int64)
        remap[need] = np.arange(need.size)
        sub_perm = np.where(perm >= 0, remap[np.maximum(perm, 0)], -1).astype(np.int32).ravel()
        sub_y = gu.bits(y[torch.from_numpy(need).to(DEV)])
        return t0, t1, sub_y, sub_perm

    def run(args):
        t0, t1, sub_y, sub_perm = args
        outs[t0] = oracle.apply_shuffle_mul_sum(sub_y, gu.code(y.dtype), sub_perm,
                                                weights[t0:t1], "f32", t1 - t0, k, out_dtype)

    with ThreadPoolExecutor(max_workers=8) as pool:
        futs = []
        for t0 in range(0, T, chunk):
            futs.append(pool.submit(run, host_chunk(t0)))   # device gathers stay on this thread
            if len(futs) >= 16:
                futs.pop(0).result()
        for f in futs:
            f.result()
    return np.concatenate([outs[t0] for t0 in sorted(outs)])


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workload_full_size(name):
    w = WORKLOADS[name]
    _print_case("workload full", name, w.T)
    inp = build_inputs(w, DEV)
    T, k = w.T, w.k
    meta = gu.check_prepare(inp["ids"], w.E, w.row_align)     # metadata: every entry
    t = meta["_t"]
    rows = t["input_permutation"].numel()
    x = inp["x"]
    xd = torch.empty((rows, w.H), dtype=x.dtype, device=DEV)
    sd = None
    if inp["scales"] is not None:
        sd = torch.empty((rows, inp["scales"].shape[1]), dtype=torch.float32, device=DEV)
    mx.dispatch_rows(x, t["output_permutation"], k, xd, inp["scales"], sd)
    y = expert_output(w, rows, DEV)
    f = torch.from_numpy(inp["weights"]).to(DEV)
    odt = {"bf16": torch.bfloat16, "f32": torch.float32}[w.out_dtype]
    out = torch.empty((T, w.H), dtype=odt, device=DEV)
    mx.apply_shuffle_mul_sum(y, out, t["output_permutation"], f)
    torch.cuda.synchronize()

    rng = np.random.default_rng(123)
    inp_perm = meta["input_permutation"]
    used = np.nonzero(inp_perm >= 0)[0]
    # dispatched rows: 512 sampled rows against the oracle's gather
    sample = np.sort(rng.choice(used, size=min(512, used.size), replace=False))
    x_host = gu.bits(x)
    want = oracle.shuffle_rows(x_host, inp_perm[sample])
    got = gu.bits(xd[torch.from_numpy(sample).to(DEV)])
    np.testing.assert_array_equal(got, want)
    if sd is not None:
        np.testing.assert_array_equal(gu.bits(sd[torch.from_numpy(sample).to(DEV)]),
                                      oracle.shuffle_rows(gu.bits(inp["scales"]),
                                                          inp_perm[sample]))
    # every used row holds its source token's bytes (exact, in chunks): with
    # the metadata equal to the oracle's, this is the oracle's gather
    for c0 in range(0, used.size, 16384):
        idx = torch.from_numpy(used[c0:c0 + 16384]).to(DEV)
        src = torch.from_numpy(inp_perm[used[c0:c0 + 16384]].astype(np.int64)).to(DEV)
        assert torch.equal(xd[idx].view(torch.uint8), x[src].view(torch.uint8))
        if sd is not None:
            assert torch.equal(sd[idx], inp["scales"][src])
    del xd, sd
    # combine: every token through the oracle
    _print_case("workload full combine", name, T)
    want = _oracle_combine_all(y, meta["output_permutation"], inp["weights"], T, k,
                               w.out_dtype)
    got = gu.bits(out)
    if w.out_dtype == "f32":
        np.testing.assert_allclose(got, want, rtol=1e-5, atol=0)
    else:
        wt = torch.from_numpy(want.view(np.int16)).view(odt).float().numpy()
        np.testing.assert_allclose(out.float().cpu().numpy(), wt, rtol=1.6e-2, atol=1e-2)
    np.testing.assert_array_equal(got, want)


def test_bound_calls_match_plain_calls():
    """bind(): checked and marshalled once, each call of the BoundCall gives
    the plain call's bytes (and the timed form's), on the stream current at
    the time of the call."""
    _print_case("bound calls", 512, 4096)
    T, k, E, H = 512, 8, 64, 4096
    rng = np.random.default_rng(41)
    ids = torch.from_numpy(routing.uniform_topk(rng, T, E, k)).to(DEV)
    x = routing.normal_rows(T, H, "bf16", seed=42, device=DEV)
    f = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(DEV)
    outs = []
    for use_bind in (False, True):
        r = mx.empty_routing(T, k, E, DEV, row_align=16, blockscale=True)
        rows = r["input_permutation"].numel()
        xd = torch.zeros((rows, H), dtype=torch.bfloat16, device=DEV)
        xg = torch.zeros_like(xd)
        y = routing.normal_rows(rows, H, "bf16", seed=43, device=DEV)
        out = torch.empty((T, H), dtype=torch.float32, device=DEV)
        args_p = (ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                  r["input_permutation"], r["output_permutation"], E, 256, H,
                  r["blockscale_offsets"])
        kw_p = dict(row_align=16, workspace=r["workspace"])
        if use_bind:
            calls = [mx.bind(mx.prepare_moe_input, *args_p, **kw_p),
                     mx.bind(mx.dispatch_rows, x, r["output_permutation"], k, xd),
                     mx.bind(mx.shuffle_rows, x, r["input_permutation"], xg),
                     mx.bind(mx.apply_shuffle_mul_sum, y, out, r["output_permutation"], f)]
            assert calls[1].result is xd and calls[2].result is xg
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):                  # the stream current at call time
                for c in calls:
                    c()
            torch.cuda.current_stream().wait_stream(side)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
            for e in evs:
                e.record()
            out.fill_(float("nan"))
            calls[0](kernel_events=(evs[0], evs[1]))        # timed forms, same bytes again
            calls[1](kernel_events=(evs[2], evs[3]))
            calls[3](kernel_events=(evs[4], evs[5]))
            with pytest.raises(ValueError):
                calls[2](kernel_events=(evs[0], evs[1]))    # shuffle_rows has no timed form
        else:
            mx.prepare_moe_input(*args_p, **kw_p)
            mx.dispatch_rows(x, r["output_permutation"], k, xd)
            mx.shuffle_rows(x, r["input_permutation"], xg)
            mx.apply_shuffle_mul_sum(y, out, r["output_permutation"], f)
        torch.cuda.synchronize()
        outs.append([r[key].clone() for key in ("expert_offsets", "input_permutation",
                                                "output_permutation", "blockscale_offsets",
                                                "problem_sizes1")] + [xd, xg, out])
    for a, b in zip(*outs):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    with pytest.raises(TypeError):
        mx.bind(mx.moe_sort, ids, E, 0, E, 16)


def test_timed_forms_match_and_time_the_kernels():
    """mx_dispatch_rows_timed / mx_apply_shuffle_mul_sum_timed: the same bytes
    as the plain calls, and kernel events that lie inside the stage events
    recorded on the stream around the call."""
    _print_case("timed forms", 1024, 7168)
    w = WORKLOADS["uniform_T4096_H7168_E256_k8_pad128"]
    T, k, E, H = 1024, w.k, w.E, w.H
    rng = np.random.default_rng(31)
    ids = routing.uniform_topk(rng, T, E, k)
    meta = gu.gpu_prepare(ids, E, row_align=128)
    perm = meta["_t"]["output_permutation"]
    rows = meta["_t"]["input_permutation"].numel()
    x = routing.normal_rows(T, H, "bf16", seed=32, device=DEV)
    y = routing.normal_rows(rows, H, "bf16", seed=33, device=DEV)
    f = torch.from_numpy(routing.softmax_weights(rng, T, k)).to(DEV)
    stream = torch.cuda.current_stream()
    kd = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    kc = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    st = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for e in (*kd, *kc):
        e.record(stream)
    xd1 = torch.full((rows, H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    xd2 = xd1.clone()
    o1 = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    o2 = torch.empty_like(o1)
    mx.dispatch_rows(x, perm, k, xd1)
    mx.apply_shuffle_mul_sum(y, o1, perm, f)
    st[0].record(stream)
    mx.dispatch_rows(x, perm, k, xd2, kernel_events=kd)
    st[1].record(stream)
    mx.apply_shuffle_mul_sum(y, o2, perm, f, kernel_events=kc)
    st[2].record(stream)
    torch.cuda.synchronize()
    assert torch.equal(xd1.view(torch.int16), xd2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    for (a, b), (s0, s1) in ((kd, (st[0], st[1])), (kc, (st[1], st[2]))):
        kernel, stage = a.elapsed_time(b), s0.elapsed_time(s1)
        assert 0.0 < kernel <= stage
        assert s0.elapsed_time(a) >= 0.0 and b.elapsed_time(s1) >= 0.0


@pytest.mark.parametrize("T,one_call", [(1500, False), (1500, True), (100, True)])
def test_graph_capture_replays_match_eager(T, one_call):
    """The calls enqueue kernels only (no allocation, no memset), so a HIP
    graph can capture prepare, dispatch and combine (with one_call, routing
    and dispatch through prepare_dispatch, one launch at T = 100).  The graph
    is replayed three times on new inputs copied into its static tensors,
    with eager work and synchronisations between replays; every replay must
    equal the eager calls on the same inputs, bit for bit."""
    if mx.library_path() == mx.CHECKED_LIBRARY:
        pytest.skip("the bounds-checked library refuses stream capture")
    _print_case("graph capture", T, one_call)
    dev = torch.device(DEV)
    E, k, H, A = 64, 8, 1024, 16
    r = mx.empty_routing(T, k, E, dev, row_align=A)
    cap = r["input_permutation"].numel()
    ids = torch.empty(T, k, dtype=torch.int64, device=dev)
    x = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    y = torch.empty(cap, H, dtype=torch.bfloat16, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    xd = torch.zeros(cap, H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def step():
        if one_call:
            mx.prepare_dispatch(ids, r["expert_offsets"], r["problem_sizes1"],
                                r["problem_sizes2"], r["input_permutation"],
                                r["output_permutation"], E, 64, 32, x, xd, row_align=A,
                                workspace=r["workspace"])
        else:
            mx.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"],
                                 r["problem_sizes2"], r["input_permutation"],
                                 r["output_permutation"], E, 64, 32, row_align=A,
                                 workspace=r["workspace"])
            mx.dispatch_rows(x, r["output_permutation"], k, xd)
        mx.apply_shuffle_mul_sum(y, out, r["output_permutation"], w)

    def load(seed):
        rng = np.random.default_rng(seed)
        ids.copy_(torch.from_numpy(routing.uniform_topk(rng, T, E, k)))
        x.copy_(routing.normal_rows(T, H, "bf16", seed=seed, device=DEV))
        y.copy_(routing.normal_rows(cap, H, "bf16", seed=seed + 1, device=DEV))
        w.copy_(torch.from_numpy(routing.softmax_weights(rng, T, k)))

    def snapshot():
        used = r["input_permutation"] >= 0
        return [r["expert_offsets"].clone(), r["input_permutation"].clone(),
                r["output_permutation"].clone(), xd[used].clone(), out.clone()]

    load(100)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        step()                                         # warm-up off the default stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for seed in (101, 102, 103):
        load(seed)
        torch.cuda.synchronize()
        step()                                         # eager on these inputs
        torch.cuda.synchronize()
        want = snapshot()
        xd.zero_()
        out.fill_(float("nan"))
        r["input_permutation"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), seed


@pytest.mark.parametrize("name", ["uniform_T4096_H7168_E256_k8_pad128", "khot8_T8192_H7168_E256_k8"])
def test_repeat_runs_identical(name):
    """Determinism at full size: the whole step (prepare, dispatch, combine)
    run twice on the same inputs, with every output poisoned in between,
    gives identical bits; the K-hot workload puts most picks on 8 experts,
    so many lanes of a wave count into the same LDS counters."""
    w = WORKLOADS[name]
    _print_case("repeat runs", name)
    dev = torch.device(DEV)
    inp = build_inputs(w, DEV)
    T, k, E, H = w.T, w.k, w.E, w.H
    r = mx.empty_routing(T, k, E, dev, row_align=w.row_align, blockscale=True)
    cap = r["input_permutation"].numel()
    ids = torch.from_numpy(inp["ids"]).to(dev)
    wts = torch.from_numpy(inp["weights"]).to(dev)
    y = expert_output(w, cap, dev)
    xd = torch.empty(cap, H, dtype=inp["x"].dtype, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    runs = []
    for _ in range(2):
        for key in ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
                    "output_permutation", "blockscale_offsets"):
            r[key].fill_(-7)
        xd.view(torch.uint8).fill_(0xA5)
        out.fill_(float("nan"))
        mx.prepare_moe_input(ids, r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
                             r["input_permutation"], r["output_permutation"], E, 2048, H,
                             r["blockscale_offsets"], row_align=w.row_align,
                             workspace=r["workspace"])
        mx.dispatch_rows(inp["x"], r["output_permutation"], k, xd)
        mx.apply_shuffle_mul_sum(y, out, r["output_permutation"], wts)
        torch.cuda.synchronize()
        runs.append([r[key].clone() for key in ("expert_offsets", "problem_sizes1",
                                                "problem_sizes2", "input_permutation",
                                                "output_permutation", "blockscale_offsets")]
                    + [xd.view(torch.uint8).clone(), out.view(torch.int16).clone()])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


def test_out_of_range_indices_are_skipped():
    """Index data is never trusted: destinations of dispatch_rows and
    dispatch_rows_fp8 outside [0, rows) and sources of shuffle_rows outside
    [0, T) are skipped, rows nobody targets keep their contents, and every
    in-range row matches the oracle's gather bit for bit."""
    _print_case("out-of-range indices")
    rng = np.random.default_rng(71)
    T, k, H, rows = 300, 4, 1024, 1500
    x = routing.normal_rows(T, H, "bf16", seed=72, device=DEV)
    perm = rng.permutation(rows)[:T * k].astype(np.int64)       # distinct rows
    bad = rng.random(T * k)
    perm[bad < 0.05] = -1
    perm[(bad >= 0.05) & (bad < 0.10)] = rows
    perm[(bad >= 0.10) & (bad < 0.15)] = rows + 5
    perm[(bad >= 0.15) & (bad < 0.17)] = 2**31 - 1
    perm = perm.astype(np.int32)
    src = np.full(rows, -1, np.int32)                            # the gather map it implies
    ok = (perm >= 0) & (perm < rows)
    src[perm[ok]] = (np.nonzero(ok)[0] // k).astype(np.int32)
    used = src >= 0
    t_perm = torch.from_numpy(perm).to(DEV)
    # scatter form
    xd = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    xd.view(torch.uint8).fill_(gu.SENTINEL)
    mx.dispatch_rows(x, t_perm, k, xd)
    torch.cuda.synchronize()
    want = oracle.shuffle_rows(gu.bits(x), src)
    np.testing.assert_array_equal(gu.bits(xd)[used], want[used])
    assert np.all(xd.view(torch.uint8).cpu().numpy()[~used] == gu.SENTINEL)
    # gather form with sources out of range
    src_bad = src.copy()
    src_bad[rng.random(rows) < 0.1] = T
    src_bad[rng.random(rows) < 0.05] = T + 9
    used_g = (src_bad >= 0) & (src_bad < T)
    xg = torch.empty(rows, H, dtype=torch.bfloat16, device=DEV)
    xg.view(torch.uint8).fill_(gu.SENTINEL)
    mx.shuffle_rows(x, torch.from_numpy(src_bad).to(DEV), xg)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gu.bits(xg)[used_g],
                                  oracle.shuffle_rows(gu.bits(x), src_bad)[used_g])
    assert np.all(xg.view(torch.uint8).cpu().numpy()[~used_g] == gu.SENTINEL)
    # FP8 dispatch: codes and scales of in-range rows, others untouched
    q = torch.full((rows, H), 0x55, dtype=torch.uint8, device=DEV)
    sc = torch.full((rows, H // 128), -3.0, dtype=torch.float32, device=DEV)
    mx.dispatch_rows_fp8(x, t_perm, k, q, sc)
    torch.cuda.synchronize()
    xq, xs = oracle.quantize_fp8_rows(gu.bits(x))
    np.testing.assert_array_equal(q.cpu().numpy()[used], oracle.shuffle_rows(xq, src)[used])
    np.testing.assert_array_equal(sc.cpu().numpy()[used], oracle.shuffle_rows(xs, src)[used])
    assert np.all(q.cpu().numpy()[~used] == 0x55) and np.all(sc.cpu().numpy()[~used] == -3.0)
