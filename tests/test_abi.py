"""The C ABI on the host (no GPU): the library loads, exports every entry
point include/mxmoe.h declares, and rejects bad arguments with the
documented status before making any HIP call (fake device addresses are
never dereferenced on these paths).  Every test runs against the loaded
library and against the bounds-checked build, whose host checks are the
same code."""

import ctypes
import os
import re

import pytest

import combine_topk_ids_expert_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxmoe.h")

OK, INVALID, DTYPE, MISALIGNED, WORKSPACE, CAPACITY, HIP, OUT_OF_BOUNDS = range(8)
F32, F16, BF16, FP8, I32, I64 = range(6)
P = 0x10000          # a fake, 64 KiB-aligned "device" address, never dereferenced
S = None             # stream (never reached)


@pytest.fixture(scope="module", params=["loaded", "checked"])
def lib(request):
    if request.param == "loaded":
        return mx.load_library()
    return mx.open_library(mx.CHECKED_LIBRARY)


def test_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(mx_\w+)\s*\(", text))
    assert declared == set(mx.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    for path in (mx.library_path(), mx.CHECKED_LIBRARY, mx.ALTGRID_LIBRARY):
        ext = ctypes.CDLL(path)
        for name in declared:
            getattr(ext, name)
    assert mx.open_library(mx.ALTGRID_LIBRARY).mx_bounds_checked() == 0


def test_status_strings(lib):
    for code in range(8):
        assert lib.mx_status_string(code) != b"unknown status"
    assert lib.mx_status_string(99) == b"unknown status"


def test_bounds_check_calls(lib):
    checked = lib.mx_bounds_checked()
    assert checked == (1 if lib._name == mx.CHECKED_LIBRARY else 0)
    report = (ctypes.c_uint64 * 4)(7, 7, 7, 7)
    assert lib.mx_bounds_report(report, 1) == OK
    assert list(report) == [0, 0, 0, 0]          # no kernel ran
    assert lib.mx_bounds_report(None, 0) == INVALID
    assert lib.mx_bounds_shrink_outputs(-1) == INVALID
    assert lib.mx_bounds_shrink_outputs(0) == OK
    assert lib.mx_bounds_shrink_outputs(16) == (OK if checked else INVALID)
    assert lib.mx_bounds_shrink_outputs(0) == OK


def test_capacity_and_workspace(lib):
    assert lib.mx_dispatch_capacity(4096, 8, 256, 128) == 4096 * 8 + 256 * 127
    assert lib.mx_dispatch_capacity(0, 8, 256, 1) == 0
    assert lib.mx_dispatch_capacity(2**31, 1, 1, 1) == -1
    assert lib.mx_dispatch_capacity(2**28, 8, 1, 1) == -1
    assert lib.mx_dispatch_capacity(10, 0, 1, 1) == -1
    assert lib.mx_dispatch_capacity(10, 1, 1, 0) == -1
    assert lib.mx_prepare_workspace_size(32, 8, 256) == 0          # one-launch path
    big = lib.mx_prepare_workspace_size(65536, 8, 288)
    assert big >= 288 * 4 * (65536 * 8 // 4096)
    assert lib.mx_prepare_workspace_size(10, 8, 2000) == 0


def _prep(lib, **kw):
    a = dict(ids=P, dt=I32, T=64, k=8, E=256, g=(1, 2, 3, 4), A=1, eo=P, ps1=P, ps2=P,
             inp=P, inp_len=64 * 8, outp=P, bso=None, bsa=128, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.mx_prepare_moe_input(a["ids"], a["dt"], a["T"], a["k"], a["E"], *a["g"], a["A"],
                                    a["eo"], a["ps1"], a["ps2"], a["inp"], a["inp_len"],
                                    a["outp"], a["bso"], a["bsa"], a["ws"], a["wsb"], S)


def test_prepare_rejects(lib):
    assert _prep(lib, dt=F32) == DTYPE
    assert _prep(lib, E=0) == INVALID
    assert _prep(lib, E=1025) == INVALID
    assert _prep(lib, k=0) == INVALID
    assert _prep(lib, T=-1) == INVALID
    assert _prep(lib, A=0) == INVALID
    assert _prep(lib, T=2**31, k=1) == INVALID
    assert _prep(lib, eo=None) == INVALID
    assert _prep(lib, ids=None) == INVALID
    assert _prep(lib, outp=None) == INVALID
    assert _prep(lib, inp=None) == INVALID
    assert _prep(lib, inp_len=64 * 8 - 1) == CAPACITY
    assert _prep(lib, A=128, inp_len=64 * 8) == CAPACITY
    assert _prep(lib, bso=P, bsa=0) == INVALID
    assert _prep(lib, ids=P + 2) == MISALIGNED
    assert _prep(lib, ids=P + 4, dt=I64) == MISALIGNED
    assert _prep(lib, outp=P + 1) == MISALIGNED
    assert _prep(lib, T=65536, inp_len=65536 * 8, ws=None) == WORKSPACE
    assert _prep(lib, T=65536, inp_len=65536 * 8, wsb=16) == WORKSPACE
    # the count table is read with 16-byte loads: a 4-aligned workspace is refused
    assert _prep(lib, T=65536, inp_len=65536 * 8, ws=P + 4) == MISALIGNED
    assert _prep(lib, T=65536, inp_len=65536 * 8, ws=P + 8) == MISALIGNED


def test_timed_prepare_checks_like_the_plain_call(lib):
    def prep_timed(**kw):
        a = dict(ids=P, dt=I32, T=64, k=8, E=256, A=1, inp_len=64 * 8, ws=P)
        a.update(kw)
        return lib.mx_prepare_moe_input_timed(a["ids"], a["dt"], a["T"], a["k"], a["E"],
                                              1, 2, 3, 4, a["A"], P, P, P, P, a["inp_len"], P,
                                              None, 128, a["ws"], 1 << 20, None, None, S)
    assert prep_timed(dt=F32) == DTYPE
    assert prep_timed(E=0) == INVALID
    assert prep_timed(inp_len=64 * 8 - 1) == CAPACITY
    assert prep_timed(ids=P + 2) == MISALIGNED
    assert prep_timed(T=65536, inp_len=65536 * 8, ws=P + 4) == MISALIGNED


def test_shuffle_rejects(lib):
    f = lib.mx_shuffle_rows
    assert f(P, 10, 0, P, 10, P, S) == INVALID
    assert f(P, -1, 16, P, 10, P, S) == INVALID
    assert f(P, 10, 16, None, 10, P, S) == INVALID
    assert f(P, 10, 16, P, 10, None, S) == INVALID
    assert f(P, 10, 16, P + 2, 10, P, S) == MISALIGNED
    assert f(P, 10, 65535 * 1024 + 1, P, 10, P, S) == INVALID
    assert f(P, 10, 16, P, 0, P, S) == OK            # nothing to do, nothing launched


def test_dispatch_rejects(lib):
    f = lib.mx_dispatch_rows
    assert f(P, 10, 0, 16, P, P, 80, None, 0, None, S) == INVALID
    assert f(P, 10, 8, 0, P, P, 80, None, 0, None, S) == INVALID
    assert f(P, 10, 8, 65535 * 1024 + 1, P, P, 80, None, 0, None, S) == INVALID
    assert f(P, 10, 8, 16, P, P, 80, P, 0, P, S) == INVALID          # side rows of 0 bytes
    assert f(P, 10, 8, 16, P, P, 80, P, 16, None, S) == INVALID      # side without destination
    assert f(P, 10, 8, 16, P, P, 80, None, 16, None, S) == INVALID   # side bytes without arrays
    assert f(None, 10, 8, 16, P, P, 80, None, 0, None, S) == INVALID
    assert f(P, 10, 8, 16, P + 1, P, 80, None, 0, None, S) == MISALIGNED
    assert f(P, 0, 8, 16, P, P, 80, None, 0, None, S) == OK


def test_timed_forms_check_like_the_plain_calls(lib):
    d = lib.mx_dispatch_rows_timed
    assert d(P, 10, 0, 16, P, P, 80, None, 0, None, None, None, S) == INVALID
    assert d(P, 10, 8, 16, P + 1, P, 80, None, 0, None, None, None, S) == MISALIGNED
    assert d(P, 10, 8, 16, P, P, 80, P, 16, None, None, None, S) == INVALID
    assert d(P, 0, 8, 16, P, P, 80, None, 0, None, P, P, S) == OK        # nothing launched
    c = lib.mx_apply_shuffle_mul_sum_timed
    assert c(P, I32, 10, 8, P, None, 0, 4, 2, P, BF16, None, None, S) == DTYPE
    assert c(P, BF16, 10, 8, P, None, 0, 4, 0, P, BF16, None, None, S) == INVALID
    assert c(P + 1, BF16, 10, 8, P, None, 0, 4, 2, P, BF16, None, None, S) == MISALIGNED
    assert c(P, BF16, 10, 8, P, None, 0, 0, 2, P, BF16, P, P, S) == OK   # nothing launched


def test_combine_rejects(lib):
    f = lib.mx_apply_shuffle_mul_sum
    assert f(P, I32, 10, 8, P, None, 0, 4, 2, P, BF16, S) == DTYPE
    assert f(P, BF16, 10, 8, P, None, 0, 4, 2, P, FP8, S) == DTYPE
    assert f(P, BF16, 10, 8, P, P, I64, 4, 2, P, BF16, S) == DTYPE
    assert f(P, BF16, 10, 8, P, None, 0, 4, 0, P, BF16, S) == INVALID
    assert f(P, BF16, -1, 8, P, None, 0, 4, 2, P, BF16, S) == INVALID
    assert f(P, BF16, 10, 8, None, None, 0, 4, 2, P, BF16, S) == INVALID
    assert f(P, BF16, 10, 8, P, None, 0, 4, 2, None, BF16, S) == INVALID
    assert f(P + 1, BF16, 10, 8, P, None, 0, 4, 2, P, BF16, S) == MISALIGNED
    assert f(P, BF16, 10, 8, P, None, 0, 4, 2, P + 2, F32, S) == MISALIGNED
    assert f(P, BF16, 10, 8, P, P + 2, F32, 4, 2, P, BF16, S) == MISALIGNED
    assert f(P, BF16, 10, 8, P, None, 0, 0, 2, P, BF16, S) == OK
    assert f(P, BF16, 10, 0, P, None, 0, 4, 2, P, BF16, S) == OK


def test_binding_refuses_cpu_tensors():
    import torch
    ids = torch.zeros(4, 2, dtype=torch.int32)
    r = {k: torch.zeros(3, dtype=torch.int32) for k in ("a", "b", "c", "d")}
    with pytest.raises(ValueError):
        mx.prepare_moe_input(ids, r["a"], None, None, r["b"], r["c"], 2, 1, 1)
    with pytest.raises(ValueError):
        mx.shuffle_rows(torch.zeros(4, 8), torch.zeros(4, dtype=torch.int32))


def test_zeroing_rejects(lib):
    f = lib.mx_moe_output_memset
    assert f(P, 10, 0, 16, P, S) == INVALID
    assert f(P, 10, 8, 0, P, S) == INVALID
    assert f(None, 10, 8, 16, P, S) == INVALID
    assert f(P, 10, 8, 16, None, S) == INVALID
    assert f(P, 10, 8, 16, P + 2, S) == MISALIGNED
    assert f(P, 0, 8, 16, P, S) == OK
    g = lib.mx_zero_padding_rows
    assert g(P, 10, 0, P, None, 0, S) == INVALID
    assert g(P, -1, 16, P, None, 0, S) == INVALID
    assert g(None, 10, 16, P, None, 0, S) == INVALID
    assert g(P, 10, 16, None, None, 0, S) == INVALID
    assert g(P, 10, 16, P, P, 0, S) == INVALID          # offsets without an expert count
    assert g(P, 10, 16, P, P, 1025, S) == INVALID
    assert g(P, 10, 16, P + 1, None, 0, S) == MISALIGNED
    assert g(P, 10, 16, P, P + 2, 4, S) == MISALIGNED
    assert g(P, 0, 16, P, None, 0, S) == OK


def _sort(lib, **kw):
    a = dict(ids=P, dt=I64, T=64, k=8, E=256, L0=32, EL=32, S=128, e2p=P, p2e=P,
             cap=64 * 8 + 32 * 127, tg=P, tl=P, mt=(64 * 8 + 32 * 127 + 127) // 128, tot=P, nt=P,
             eo=None, ws=P, wsb=1 << 20)
    a.update(kw)
    return lib.mx_moe_sort(a["ids"], a["dt"], a["T"], a["k"], a["E"], a["L0"], a["EL"], a["S"],
                           a["e2p"], a["p2e"], a["cap"], a["tg"], a["tl"], a["mt"], a["tot"],
                           a["nt"], a["eo"], a["ws"], a["wsb"], S)


def test_moe_sort_rejects(lib):
    assert _sort(lib, dt=F16) == DTYPE
    assert _sort(lib, L0=-1) == INVALID
    assert _sort(lib, EL=0) == INVALID
    assert _sort(lib, L0=250, EL=32) == INVALID          # window past the expert count
    assert _sort(lib, EL=1025, E=2000, L0=0) == INVALID
    assert _sort(lib, S=0) == INVALID
    assert _sort(lib, e2p=None) == INVALID
    assert _sort(lib, p2e=None) == INVALID
    assert _sort(lib, tg=None) == INVALID
    assert _sort(lib, tot=None) == INVALID
    assert _sort(lib, nt=None) == INVALID
    assert _sort(lib, cap=64 * 8) == CAPACITY
    assert _sort(lib, mt=3) == CAPACITY
    assert _sort(lib, ids=P + 4) == MISALIGNED
    assert _sort(lib, tl=P + 2) == MISALIGNED
    assert _sort(lib, T=65536, cap=65536 * 8 + 32 * 127, mt=(65536 * 8 + 32 * 127) // 128 + 1,
                 ws=None) == WORKSPACE
    assert _sort(lib, T=65536, cap=65536 * 8 + 32 * 127, mt=(65536 * 8 + 32 * 127) // 128 + 1,
                 ws=P + 4) == MISALIGNED


def test_dispatch_fp8_rejects(lib):
    f = lib.mx_dispatch_rows_fp8
    assert f(P, F16, 10, 8, 4096, P, P, P, 80, S) == DTYPE
    assert f(P, BF16, 10, 0, 4096, P, P, P, 80, S) == INVALID
    assert f(P, BF16, 10, 8, 100, P, P, P, 80, S) == INVALID       # not a multiple of 128
    assert f(P, BF16, 10, 8, 0, P, P, P, 80, S) == INVALID
    assert f(None, BF16, 10, 8, 4096, P, P, P, 80, S) == INVALID
    assert f(P, BF16, 10, 8, 4096, P, None, P, 80, S) == INVALID
    assert f(P, BF16, 10, 8, 4096, P, P, None, 80, S) == INVALID
    assert f(P + 8, BF16, 10, 8, 4096, P, P, P, 80, S) == MISALIGNED
    assert f(P, BF16, 10, 8, 4096, P, P + 8, P, 80, S) == MISALIGNED
    assert f(P, BF16, 10, 8, 4096, P + 2, P, P, 80, S) == MISALIGNED
    assert f(P, BF16, 0, 8, 4096, P, P, P, 80, S) == OK



def test_noalloc_prepare_checks_like_the_plain_call(lib):
    """The no-alloc routing entry point refuses what the plain call refuses,
    before any HIP call (so no device address is looked up here)."""
    def prep_na(**kw):
        a = dict(ids=P, dt=I32, T=64, k=8, E=256, A=1, inp_len=64 * 8)
        a.update(kw)
        return lib.mx_prepare_moe_input_noalloc(a["ids"], a["dt"], a["T"], a["k"], a["E"],
                                                1, 2, 3, 4, a["A"], P, P, P, P, a["inp_len"], P,
                                                None, 128, S)
    assert prep_na(dt=F32) == DTYPE
    assert prep_na(E=0) == INVALID
    assert prep_na(E=1025) == INVALID
    assert prep_na(inp_len=64 * 8 - 1) == CAPACITY
    assert prep_na(ids=P + 2) == MISALIGNED
    assert prep_na(T=2**31, k=1) == INVALID
    # every size the call accepts fits the scratch: the largest workspace is
    # 128 tiles x 1024 experts x 4 bytes
    assert lib.mx_prepare_workspace_size(2**31 // 8 - 1, 8, 1024) <= 512 * 1024
    assert lib.mx_prepare_workspace_size(65536, 8, 1024) <= 512 * 1024


def test_prepare_dispatch_checks_both_halves(lib):
    """prepare_dispatch refuses what prepare_moe_input or dispatch_rows would
    refuse, before anything is launched."""
    def pd(**kw):
        a = dict(ids=P, dt=I32, T=64, k=8, E=256, A=1, inp_len=64 * 8, outp=P, ws=P,
                 src=P, rb=16, dst=P, nd=64 * 8, ss=None, srb=0, sd=None)
        a.update(kw)
        return lib.mx_prepare_dispatch(a["ids"], a["dt"], a["T"], a["k"], a["E"], 1, 2, 3, 4,
                                       a["A"], P, P, P, P, a["inp_len"], a["outp"], None, 128,
                                       a["ws"], 1 << 20, a["src"], a["rb"], a["dst"], a["nd"],
                                       a["ss"], a["srb"], a["sd"], S)
    # the routing half
    assert pd(dt=F32) == DTYPE
    assert pd(E=0) == INVALID
    assert pd(E=1025) == INVALID
    assert pd(A=0) == INVALID
    assert pd(ids=None) == INVALID
    assert pd(inp_len=64 * 8 - 1) == CAPACITY
    assert pd(ids=P + 2) == MISALIGNED
    assert pd(T=65536, inp_len=65536 * 8, nd=65536 * 8, ws=None) == WORKSPACE
    assert pd(T=65536, inp_len=65536 * 8, nd=65536 * 8, ws=P + 4) == MISALIGNED
    # the dispatch half
    assert pd(rb=0) == INVALID
    assert pd(rb=65535 * 1024 + 1) == INVALID
    assert pd(src=None) == INVALID
    assert pd(dst=None) == INVALID
    assert pd(nd=-1) == INVALID
    assert pd(outp=None) == INVALID
    assert pd(outp=P + 1) == MISALIGNED
    assert pd(ss=P, srb=0, sd=P) == INVALID                  # side rows of 0 bytes
    assert pd(ss=P, srb=16, sd=None) == INVALID              # side without destination
    assert pd(srb=16) == INVALID                             # side bytes without arrays
