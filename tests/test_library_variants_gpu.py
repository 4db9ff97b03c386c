"""The two test builds of the library on the GPU, against libmxmoe.so.

libmxmoe_checked.so checks every global load and store of the kernels against
the arrays of the call that launched them (include/mxmoe.h,
mx_bounds_checked): a call whose kernels stayed inside them returns MX_OK, one
whose kernels did not returns MX_ERR_OUT_OF_BOUNDS after skipping the
accesses outside.  libmxmoe_altgrid.so is built with other tile sizes, path
limits and workgroup widths (build.py), so the same calls run on other grids
and, for routing, other paths; deterministic kernels give the same bits.

Every entry point runs through both builds on inputs that reach each kernel
path (each routing path, the tile sort, the no-allocation routing, routing
and dispatch in one launch, each vector width of the row copies, side rows,
both combine paths, both zeroing kernels, the FP8 dispatch), with ragged
tails and invalid ids, and must return MX_OK with outputs byte-identical to
libmxmoe.so's.  Last, the checked build is shown outputs described as shorter
than they are: it catches a write past an end, skips it and reports where it
was.
"""

import contextlib

import numpy as np
import pytest
import torch

import combine_topk_ids_expert_amd as mx
from tests import gpu_util as gu
from workloads import routing

pytestmark = pytest.mark.gpu

DEV = gu.DEV
SITE_ROW_DST = 11       # CheckSite codes of the library's sources
SITE_COMBINE_OUT = 15


@pytest.fixture(scope="module")
def libs():
    return {"product": mx.load_library(), "checked": mx.open_library(mx.CHECKED_LIBRARY),
            "altgrid": mx.open_library(mx.ALTGRID_LIBRARY)}


@pytest.fixture(params=["checked", "altgrid"])
def variant(request):
    return request.param


@contextlib.contextmanager
def _using(lib):
    saved = mx._lib
    mx._lib = lib
    try:
        yield
    finally:
        mx._lib = saved


def _both(libs, variant, make, run):
    """make() returns a dict of fresh tensors (seeded inputs, sentinel-filled
    outputs); run(bufs) calls the binding.  Runs libmxmoe.so and the variant
    build on their own copies (the checked build must count nothing) and
    returns the two dicts."""
    results = []
    for name in ("product", variant):
        with _using(libs[name]):       # workspace sizes come from the library that runs
            bufs = make()
            torch.cuda.synchronize()
            if name == "checked":
                assert mx.bounds_checked()
                mx.bounds_report(clear=True)
            try:
                run(bufs)
            except mx.MxError as err:
                if err.status != 7:
                    raise
                pytest.fail(f"{err}: {mx.bounds_report(clear=True)}")
            torch.cuda.synchronize()
            if name == "checked":
                rep = mx.bounds_report(clear=True)
                assert rep["loads"] == 0 and rep["stores"] == 0, rep
        results.append(bufs)
    return results


def _same(a: dict, b: dict):
    for key in a:
        if key == "workspace":          # scratch: its size and use depend on the build
            continue
        if isinstance(a[key], torch.Tensor):
            ua = a[key].contiguous().view(torch.uint8)
            ub = b[key].contiguous().view(torch.uint8)
            assert torch.equal(ua, ub), f"{key} differs between the two libraries"


def _ids(T, E, k, mode, bad, seed, dtype=torch.int64):
    rng = np.random.default_rng(seed)
    if mode == "dups":
        ids = rng.integers(0, E, (T, k))
    else:
        ids = routing.uniform_topk(rng, T, E, k)
    if bad:
        m = rng.random(ids.shape) < bad
        ids = np.where(m, rng.choice([-1, E, E + 9], size=ids.shape), ids)
    return torch.from_numpy(ids.astype(np.int64)).to(dtype).to(DEV)


def _routing(T, k, E, A, ids):
    r = mx.empty_routing(T, k, E, DEV, row_align=A, blockscale=True)
    for key, v in r.items():
        if v is not None:
            v.fill_(-7 if v.dtype == torch.int32 else 0x5A)
    r["ids"] = ids
    return r


def _prepare(r, E, A, noalloc=False):
    args = (r["ids"], r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
            r["input_permutation"], r["output_permutation"], E, 64, 32, r["blockscale_offsets"])
    if noalloc:
        mx.prepare_moe_input_noalloc(*args, row_align=A)
    else:
        mx.prepare_moe_input(*args, row_align=A, workspace=r["workspace"])


@pytest.mark.parametrize("T,E,k,A,mode,bad,ids_dtype", [
    (32, 256, 8, 1, "uniform", 0.0, torch.int64),      # one workgroup
    (256, 256, 8, 1, "uniform", 0.0, torch.int32),     # one workgroup, 2048 picks
    (200, 256, 8, 128, "uniform", 0.05, torch.int64),  # heavy padding: one launch, every tile
    (1000, 64, 8, 1, "dups", 0.0, torch.int64),        # 8000 picks, one launch
    (4096, 256, 8, 128, "uniform", 0.0, torch.int64),  # two launches, 64 tiles
    (8192, 128, 8, 1, "uniform", 0.01, torch.int32),   # two launches, 128 tiles
    (100, 1000, 8, 16, "uniform", 0.1, torch.int64),   # 1000 experts
    (20, 33, 70, 3, "dups", 0.1, torch.int64),         # topk 70
])
def test_variant_prepare_moe_input(libs, variant, T, E, k, A, mode, bad, ids_dtype):
    print(f"case: {variant} prepare_moe_input", T, E, k, A, mode, flush=True)
    a, b = _both(libs, variant, lambda: _routing(T, k, E, A, _ids(T, E, k, mode, bad, T, ids_dtype)),
                 lambda r: _prepare(r, E, A))
    _same(a, b)


def test_variant_prepare_noalloc(libs, variant):
    T, E, k = 8192, 128, 8
    print(f"case: {variant} prepare_moe_input_noalloc", T, E, k, flush=True)
    a, b = _both(libs, variant, lambda: _routing(T, k, E, 1, _ids(T, E, k, "uniform", 0.0, 3)),
                 lambda r: _prepare(r, E, 1, noalloc=True))
    _same(a, b)


@pytest.mark.parametrize("T,E,k,off,n_local,tile", [
    (64, 8, 4, 2, 4, 16),        # one workgroup, ids outside the window
    (4096, 288, 8, 36, 36, 128),  # two launches
])
def test_variant_moe_sort(libs, variant, T, E, k, off, n_local, tile):
    print(f"case: {variant} moe_sort", T, E, k, off, n_local, tile, flush=True)

    def make():
        cap = mx.dispatch_capacity(T, k, n_local, tile)
        mt = -(-cap // tile)
        out = {"ids": _ids(T, E, k, "uniform", 0.0, 11)}
        for name, numel in [("expanded_idx_to_permuted_idx", T * k),
                            ("permuted_idx_to_expanded_idx", cap),
                            ("tile_idx_to_group_idx", mt), ("tile_idx_to_mn_limit", mt),
                            ("total_num_padded_tokens", 1), ("num_non_exiting_tiles", 1),
                            ("expert_offsets", n_local + 1)]:
            out[name] = torch.full((numel,), -7, dtype=torch.int32, device=DEV)
        return out

    a, b = _both(libs, variant, make, lambda r: mx.moe_sort(
        r["ids"], E, off, n_local, tile, out={k_: v for k_, v in r.items() if k_ != "ids"}))
    _same(a, b)


@pytest.mark.parametrize("T,E,k,H", [(32, 256, 8, 4096), (257, 256, 8, 4096)])
def test_variant_prepare_dispatch(libs, variant, T, E, k, H):
    print(f"case: {variant} prepare_dispatch", T, E, k, H, flush=True)
    cap = mx.dispatch_capacity(T, k, E, 1)

    def make():
        r = _routing(T, k, E, 1, _ids(T, E, k, "uniform", 0.0, 5))
        g = torch.Generator(device=DEV)
        g.manual_seed(T)
        r["x"] = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
        r["xd"] = torch.empty((cap, H), dtype=torch.bfloat16, device=DEV)
        r["xd"].view(torch.uint8).fill_(gu.SENTINEL)
        return r

    a, b = _both(libs, variant, make, lambda r: mx.prepare_dispatch(
        r["ids"], r["expert_offsets"], r["problem_sizes1"], r["problem_sizes2"],
        r["input_permutation"], r["output_permutation"], E, 64, 32, r["x"], r["xd"],
        r["blockscale_offsets"], workspace=r["workspace"]))
    _same(a, b)


def _routed(T, E, k, A, seed):
    """Metadata from the normal library, shared by both runs of a row kernel."""
    r = _routing(T, k, E, A, _ids(T, E, k, "uniform", 0.05, seed))
    _prepare(r, E, A)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("row_bytes", [14336, 200, 100, 50, 25])
def test_variant_row_copies(libs, variant, row_bytes):
    # 16-, 8-, 4-, 2- and 1-byte vectors; a ragged token count
    T, E, k, A = 77, 16, 4, 8
    print(f"case: {variant} dispatch_rows / shuffle_rows, row bytes", row_bytes, flush=True)
    r = _routed(T, E, k, A, 21)
    cap = r["input_permutation"].numel()

    def make():
        g = torch.Generator(device=DEV)
        g.manual_seed(row_bytes)
        x = torch.randint(0, 256, (T, row_bytes), generator=g, device=DEV, dtype=torch.uint8)
        xd = torch.full((cap, row_bytes), gu.SENTINEL, dtype=torch.uint8, device=DEV)
        xs = torch.full((cap, row_bytes), gu.SENTINEL, dtype=torch.uint8, device=DEV)
        return {"x": x, "xd": xd, "xs": xs}

    def run(b):
        mx.dispatch_rows(b["x"], r["output_permutation"], k, b["xd"])
        mx.shuffle_rows(b["x"], r["input_permutation"], b["xs"])

    a, b = _both(libs, variant, make, run)
    _same(a, b)


def test_variant_dispatch_with_side_rows_and_fp8(libs, variant):
    T, E, k, H = 48, 64, 8, 1024
    print(f"case: {variant} dispatch with scale rows, fp8 dispatch", flush=True)
    r = _routed(T, E, k, 1, 31)
    cap = r["input_permutation"].numel()

    def make():
        xq, sc = routing.fp8_blockscaled_rows(T, H, 11, device=DEV)
        g = torch.Generator(device=DEV)
        g.manual_seed(7)
        xb = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
        return {"xq": xq, "sc": sc, "xb": xb,
                "xd": torch.zeros((cap, H), dtype=xq.dtype, device=DEV),
                "sd": torch.full((cap, sc.shape[1]), float("nan"), device=DEV),
                "q": torch.zeros((cap, H), dtype=torch.uint8, device=DEV),
                "qs": torch.full((cap, H // 128), float("nan"), device=DEV)}

    def run(b):
        mx.dispatch_rows(b["xq"], r["output_permutation"], k, b["xd"], side_input=b["sc"],
                         side_output=b["sd"])
        mx.dispatch_rows_fp8(b["xb"], r["output_permutation"], k, b["q"], b["qs"])

    a, b = _both(libs, variant, make, run)
    _same(a, b)


@pytest.mark.parametrize("ydt,odt,fdt,H", [
    (torch.bfloat16, torch.bfloat16, torch.float32, 7168),   # vector path
    (torch.float32, torch.float32, torch.bfloat16, 1024),    # fp32 rows: two column sets
    (torch.bfloat16, torch.float32, None, 2048),             # unit weights
    (torch.float16, torch.float16, torch.float16, 1000),     # scalar path
])
def test_variant_combine(libs, variant, ydt, odt, fdt, H):
    T, E, k = 61, 32, 8
    print(f"case: {variant} combine", ydt, odt, fdt, H, flush=True)
    r = _routed(T, E, k, 4, 41)
    cap = r["input_permutation"].numel()

    def make():
        g = torch.Generator(device=DEV)
        g.manual_seed(H)
        y = torch.randn((cap, H), generator=g, device=DEV).to(ydt)
        w = None if fdt is None else torch.rand((T, k), generator=g, device=DEV).to(fdt)
        out = torch.full((T, H), float("nan"), device=DEV).to(odt)
        return {"y": y, "w": w, "out": out}

    a, b = _both(libs, variant, make, lambda b: mx.apply_shuffle_mul_sum(
        b["y"], b["out"], r["output_permutation"], b["w"]))
    _same(a, b)


def test_variant_zeroing(libs, variant):
    T, E, k, A, H = 90, 16, 4, 32, 1024
    print(f"case: {variant} zero_padding_rows, moe_output_memset", flush=True)
    r = _routed(T, E, k, A, 51)
    cap = r["input_permutation"].numel()
    outp = r["output_permutation"].clone()
    outp.view(T, k)[::5] = -1                         # some tokens with no valid pick

    def make():
        return {"rows": torch.full((cap, H), 3.0, device=DEV).to(torch.bfloat16),
                "rows2": torch.full((cap, H), 3.0, device=DEV).to(torch.bfloat16),
                "out": torch.full((T, H), 5.0, device=DEV).to(torch.bfloat16)}

    def run(b):
        mx.zero_padding_rows(b["rows"], r["input_permutation"], r["expert_offsets"])
        mx.zero_padding_rows(b["rows2"], r["input_permutation"])
        mx.moe_output_memset(b["out"], outp, k)

    a, b = _both(libs, variant, make, run)
    _same(a, b)


def test_checked_catches_writes_past_the_end(libs):
    """Outputs described 16 bytes short: the last 16-byte store of each call is
    counted, skipped (its bytes keep their old contents) and reported."""
    T, H = 16, 1024
    g = torch.Generator(device=DEV)
    g.manual_seed(1)
    x = torch.randn((T, H), generator=g, device=DEV).to(torch.bfloat16)
    perm = torch.arange(T, dtype=torch.int32, device=DEV)      # row t -> row t
    xd = torch.full((T, H), float("nan"), device=DEV).to(torch.bfloat16)
    out = torch.full((T, H), float("nan"), device=DEV)
    with _using(libs["checked"]):
        mx.bounds_report(clear=True)
        mx.bounds_shrink_outputs(16)
        try:
            print("case: checked dispatch_rows with a planted short destination", flush=True)
            with pytest.raises(mx.MxError) as err:
                mx.dispatch_rows(x, perm, 1, xd)
            assert err.value.status == 7
            torch.cuda.synchronize()
            rep = mx.bounds_report(clear=True)
            assert rep["loads"] == 0 and rep["stores"] == 1, rep
            assert rep["first_site"] == SITE_ROW_DST
            assert rep["first_address"] == xd.data_ptr() + xd.numel() * 2 - 16
            got = xd.view(torch.int16).view(-1)
            want = x.view(torch.int16).view(-1)
            assert torch.equal(got[:-8], want[:-8])
            assert torch.isnan(xd.view(-1)[-8:].float()).all()     # the skipped store

            print("case: checked combine with a planted short output", flush=True)
            with pytest.raises(mx.MxError) as err:
                mx.apply_shuffle_mul_sum(xd, out, perm)
            assert err.value.status == 7
            torch.cuda.synchronize()
            rep = mx.bounds_report(clear=True)
            assert rep["stores"] == 1 and rep["first_site"] == SITE_COMBINE_OUT, rep
            assert rep["first_address"] == out.data_ptr() + out.numel() * 4 - 16
            assert torch.isnan(out.view(-1)[-4:]).all()
        finally:
            mx.bounds_shrink_outputs(0)
        # the true extents again: the same calls are clean
        mx.dispatch_rows(x, perm, 1, xd)
        mx.apply_shuffle_mul_sum(xd, out, perm)
        torch.cuda.synchronize()
        rep = mx.bounds_report(clear=True)
        assert rep["loads"] == 0 and rep["stores"] == 0, rep
    assert torch.equal(xd.view(torch.int16), x.view(torch.int16))
    assert torch.equal(out, x.float())
