"""CPU oracle for MoE token dispatch and combine -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It wraps ``oracle.c`` (plain C, built with gcc) with
numpy in and numpy out; it shares no code with the HIP path.

What each function computes is the plain definition of the three calls on the
sglang page "[jit_kernel] Add prepare_moe_input JIT kernels" (section
"Changes"); ``oracle.c`` states the readings taken where the page is silent.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# The oracle's own element-type numbering (see oracle.c).
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}

_lib = None


def build(out_path: str | None = None, src_path: str | None = None,
          extra_flags: list[str] | None = None) -> str:
    """Compile the oracle with gcc; returns the library path.  ``extra_flags``
    are appended (the sanitizer test builds an instrumented copy)."""
    out_path = out_path or _LIB_PATH
    src_path = src_path or _SRC
    tmp = f"{out_path}.{os.getpid()}.tmp"
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-Wall",
           "-Werror", "-fPIC", "-shared", *(extra_flags or []), src_path, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def load(path: str | None = None):
    """Load (building first if absent) the oracle library.  With ``path``,
    load that build instead of the default one (used by the mutation tests)."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _declare(ctypes.CDLL(_LIB_PATH))
    return _lib


def _declare(lib):
    c_i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_prepare_moe_input.restype = ctypes.c_int
    lib.oracle_prepare_moe_input.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32,
        c_i32p, c_i32p, c_i32p, c_i32p, ctypes.c_int64, c_i32p, c_i32p]
    lib.oracle_shuffle_rows.restype = None
    lib.oracle_shuffle_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, c_i32p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_apply_shuffle_mul_sum.restype = None
    lib.oracle_apply_shuffle_mul_sum.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, c_i32p, ctypes.c_void_p, ctypes.c_int,
        ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_output_memset.restype = None
    lib.oracle_output_memset.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int64, c_i32p]
    lib.oracle_zero_padding_rows.restype = None
    lib.oracle_zero_padding_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             c_i32p, c_i32p, ctypes.c_int32]
    lib.oracle_moe_sort.restype = ctypes.c_int
    lib.oracle_moe_sort.argtypes = [
        ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, c_i32p, c_i32p, ctypes.c_int64,
        c_i32p, c_i32p, ctypes.c_int64, c_i32p, c_i32p]
    lib.oracle_f32_to_e4m3.restype = ctypes.c_uint8
    lib.oracle_f32_to_e4m3.argtypes = [ctypes.c_uint32]
    lib.oracle_quantize_fp8_rows.restype = None
    lib.oracle_quantize_fp8_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    # scalar conversions take and return fp32 bit patterns (no trip through a
    # double, which would quiet signalling NaNs)
    for name in ("oracle_f32_to_bf16", "oracle_f32_to_f16"):
        getattr(lib, name).restype = ctypes.c_uint16
        getattr(lib, name).argtypes = [ctypes.c_uint32]
    for name in ("oracle_bf16_to_f32", "oracle_f16_to_f32"):
        getattr(lib, name).restype = ctypes.c_uint32
        getattr(lib, name).argtypes = [ctypes.c_uint16]
    return lib


def _i32p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def capacity_rows(T: int, k: int, E: int, row_align: int) -> int:
    """Rows a dispatched buffer needs for any routing: every pick plus at most
    row_align - 1 padding rows per expert."""
    return T * k + E * (row_align - 1)


def prepare_moe_input(ids: np.ndarray, num_experts: int, row_align: int = 1,
                      blockscale_align: int = 128, gemm: tuple = (0, 0, 0, 0),
                      r_max: int | None = None, lib=None) -> dict:
    """Routing metadata for top-k ids [T, k] (int32 or int64)."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids)
    if ids.dtype not in (np.int32, np.int64) or ids.ndim != 2:
        raise TypeError("ids must be a 2-D int32 or int64 array")
    T, k = ids.shape
    E = int(num_experts)
    if r_max is None:
        r_max = capacity_rows(T, k, E, row_align)
    eo = np.zeros(E + 1, np.int32)
    ps1 = np.zeros((E, 3), np.int32)
    ps2 = np.zeros((E, 3), np.int32)
    inp = np.zeros(r_max, np.int32)
    outp = np.zeros(T * k, np.int32)
    bso = np.zeros(E + 1, np.int32)
    rc = lib.oracle_prepare_moe_input(
        ids.ctypes.data, ids.dtype.itemsize, T, k, E, *[int(g) for g in gemm],
        row_align, blockscale_align, _i32p(eo), _i32p(ps1), _i32p(ps2), _i32p(inp), r_max,
        _i32p(outp), _i32p(bso))
    if rc != 0:
        raise ValueError(f"oracle_prepare_moe_input failed with {rc}")
    return {"expert_offsets": eo, "problem_sizes1": ps1, "problem_sizes2": ps2,
            "input_permutation": inp, "output_permutation": outp,
            "blockscale_offsets": bso}


def shuffle_rows(src: np.ndarray, dst2src: np.ndarray, num_dst_rows: int | None = None,
                 dst: np.ndarray | None = None, lib=None) -> np.ndarray:
    """dst[r] = src[dst2src[r]] byte for byte (src is [n, ...] of any dtype).
    Rows whose index is out of range keep the contents of ``dst`` (zeros when
    ``dst`` is not given)."""
    lib = lib or load()
    src = np.ascontiguousarray(src)
    dst2src = np.ascontiguousarray(dst2src, dtype=np.int32)
    n_dst = len(dst2src) if num_dst_rows is None else num_dst_rows
    row_bytes = src[0:1].nbytes if len(src) else int(np.prod(src.shape[1:])) * src.itemsize
    if dst is None:
        dst = np.zeros((n_dst,) + src.shape[1:], dtype=src.dtype)
    assert dst.flags.c_contiguous and dst.dtype == src.dtype
    lib.oracle_shuffle_rows(src.ctypes.data, len(src), row_bytes, _i32p(dst2src), n_dst,
                            dst.ctypes.data)
    return dst


def _elem_array(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    want = np.float32 if dtype == "f32" else np.uint16
    if a.dtype != want:
        a = a.view(want)
    return a


def apply_shuffle_mul_sum(y: np.ndarray, y_dtype: str, permutation: np.ndarray,
                          factors: np.ndarray | None, factors_dtype: str, T: int, k: int,
                          out_dtype: str, lib=None) -> np.ndarray:
    """out[t] = round(sum_j factors[t, j] * y[permutation[t*k + j]]) in fp32.

    bf16 / f16 arrays are passed as their 16-bit patterns (uint16 / int16
    views); f32 as float32.  Returns float32 for "f32", else uint16 patterns.
    """
    lib = lib or load()
    y = _elem_array(y, y_dtype)
    H = y.shape[1] if y.ndim == 2 else 0
    perm = np.ascontiguousarray(permutation, dtype=np.int32)
    assert perm.size == T * k
    f = _elem_array(factors, factors_dtype) if factors is not None else None
    out = np.zeros((T, H), dtype=np.float32 if out_dtype == "f32" else np.uint16)
    lib.oracle_apply_shuffle_mul_sum(
        y.ctypes.data, DTYPES[y_dtype], len(y), _i32p(perm),
        f.ctypes.data if f is not None else None, DTYPES[factors_dtype], T, k, H,
        out.ctypes.data, DTYPES[out_dtype])
    return out


def _row_bytes(a: np.ndarray) -> int:
    return int(np.prod(a.shape[1:], dtype=np.int64)) * a.itemsize


def output_memset(out: np.ndarray, topk: int, expanded_to_permuted: np.ndarray,
                  lib=None) -> np.ndarray:
    """In place on a copy of ``out`` [T, ...]: row t becomes zero bytes iff one
    of its picks has a permuted index >= 0.  Returns the new array."""
    lib = lib or load()
    res = np.ascontiguousarray(out).copy()
    perm = np.ascontiguousarray(expanded_to_permuted, dtype=np.int32)
    assert perm.size == len(res) * topk
    lib.oracle_output_memset(res.ctypes.data, len(res), topk, _row_bytes(res), _i32p(perm))
    return res


def zero_padding_rows(rows: np.ndarray, input_permutation: np.ndarray,
                      expert_offsets: np.ndarray | None = None, lib=None) -> np.ndarray:
    """On a copy of ``rows`` [R, ...]: rows below the padded total whose
    input_permutation entry is negative become zero bytes."""
    lib = lib or load()
    res = np.ascontiguousarray(rows).copy()
    inp = np.ascontiguousarray(input_permutation, dtype=np.int32)
    assert inp.size >= len(res)
    eo = None if expert_offsets is None else np.ascontiguousarray(expert_offsets, dtype=np.int32)
    lib.oracle_zero_padding_rows(res.ctypes.data, len(res), _row_bytes(res), _i32p(inp),
                                 _i32p(eo), 0 if eo is None else eo.size - 1)
    return res


def moe_sort(ids: np.ndarray, num_experts: int, local_expert_offset: int,
             num_local_experts: int, tile_size: int, lib=None) -> dict:
    """Tile-padded sort metadata for the local experts (see oracle.c)."""
    lib = lib or load()
    ids = np.ascontiguousarray(ids)
    if ids.dtype not in (np.int32, np.int64) or ids.ndim != 2:
        raise TypeError("ids must be a 2-D int32 or int64 array")
    T, k = ids.shape
    cap = T * k + num_local_experts * (tile_size - 1)
    max_tiles = -(-cap // tile_size)
    e2p = np.zeros(T * k, np.int32)
    p2e = np.zeros(cap, np.int32)
    tg = np.zeros(max_tiles, np.int32)
    tl = np.zeros(max_tiles, np.int32)
    total = np.zeros(1, np.int32)
    ntiles = np.zeros(1, np.int32)
    rc = lib.oracle_moe_sort(ids.ctypes.data, ids.dtype.itemsize, T, k, num_experts,
                             local_expert_offset, num_local_experts, tile_size, _i32p(e2p),
                             _i32p(p2e), cap, _i32p(tg), _i32p(tl), max_tiles, _i32p(total),
                             _i32p(ntiles))
    if rc != 0:
        raise ValueError(f"oracle_moe_sort failed with {rc}")
    return {"expanded_idx_to_permuted_idx": e2p, "permuted_idx_to_expanded_idx": p2e,
            "tile_idx_to_group_idx": tg, "tile_idx_to_mn_limit": tl,
            "total_num_padded_tokens": int(total[0]), "num_non_exiting_tiles": int(ntiles[0])}


def f32_to_e4m3(x: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    bits = np.asarray(x, np.float32).ravel().view(np.uint32)
    return np.array([lib.oracle_f32_to_e4m3(int(v)) for v in bits], dtype=np.uint8)


def quantize_fp8_rows(x_bf16_bits: np.ndarray, block: int = 128, lib=None):
    """bf16 rows (uint16 patterns [T, H]) -> (e4m3fn bytes uint8 [T, H],
    float32 scales [T, H / block])."""
    lib = lib or load()
    x = np.ascontiguousarray(x_bf16_bits).view(np.uint16)
    T, H = x.shape
    assert H % block == 0
    q = np.zeros((T, H), np.uint8)
    sc = np.zeros((T, H // block), np.float32)
    lib.oracle_quantize_fp8_rows(x.ctypes.data, T, H, block, q.ctypes.data, sc.ctypes.data)
    return q, sc


def f32_to_bf16(x: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    bits = np.asarray(x, np.float32).ravel().view(np.uint32)
    return np.array([lib.oracle_f32_to_bf16(int(v)) for v in bits], dtype=np.uint16)


def f32_to_f16(x: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    bits = np.asarray(x, np.float32).ravel().view(np.uint32)
    return np.array([lib.oracle_f32_to_f16(int(v)) for v in bits], dtype=np.uint16)


def bf16_to_f32(h: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    return np.array([lib.oracle_bf16_to_f32(int(v)) for v in np.asarray(h, np.uint16).ravel()],
                    dtype=np.uint32).view(np.float32)


def f16_to_f32(h: np.ndarray, lib=None) -> np.ndarray:
    lib = lib or load()
    return np.array([lib.oracle_f16_to_f32(int(v)) for v in np.asarray(h, np.uint16).ravel()],
                    dtype=np.uint32).view(np.float32)
