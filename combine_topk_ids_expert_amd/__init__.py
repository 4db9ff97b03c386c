"""MoE token dispatch and combine on one AMD MI355X (gfx950).

A thin ctypes binding over ``libmxmoe.so`` (HIP kernels behind the C ABI in
``include/mxmoe.h``).  Every function here only checks and marshals
arguments: torch tensors supply device pointers and the current HIP stream,
and all work runs in the library's kernels.  There is no fallback: without
the built library every call raises.

The calls follow the sglang page "[jit_kernel] Add prepare_moe_input JIT
kernels" (section "Changes"): ``prepare_moe_input`` (routing metadata),
``shuffle_rows`` (row gather), ``apply_shuffle_mul_sum`` (gather, scale,
fp32 sum); ``dispatch_rows`` is the token-major form of the row gather.
Outputs are written in place, as the page's custom-op registration marks.

``bind(fn, *args, **kwargs)`` runs the checks and the marshalling of one call
once and returns a ``BoundCall``; calling that enqueues the same work again
with no Python-side checks, for small batches where a call is bound by host
time.

With ``MXMOE_LIBRARY=checked`` in the environment the binding loads
``libmxmoe_checked.so`` instead: the same kernels with every global access
checked against the call's arrays (``bounds_checked``, ``bounds_report``), a
debugging library that synchronises around every call.  ``MXMOE_LIBRARY=
altgrid`` loads ``libmxmoe_altgrid.so``, the same sources built with other
tile sizes and workgroup widths, whose results must be the same bits.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # loads the HIP runtime this library must share; keep before CDLL

__all__ = [
    "prepare_moe_input", "shuffle_rows", "dispatch_rows", "apply_shuffle_mul_sum",
    "prepare_dispatch",
    "moe_output_memset", "zero_padding_rows", "moe_sort", "dispatch_rows_fp8",
    "prepare_moe_input_noalloc", "dispatch_capacity", "prepare_workspace_size",
    "empty_routing", "MxError",
    "library_path", "load_library", "open_library", "EXPORTED_SYMBOLS", "bind", "BoundCall",
    "bounds_checked", "bounds_report", "bounds_shrink_outputs",
    "PRODUCT_LIBRARY", "CHECKED_LIBRARY", "ALTGRID_LIBRARY",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
PRODUCT_LIBRARY = os.path.join(_PKG, "libmxmoe.so")
CHECKED_LIBRARY = os.path.join(_PKG, "libmxmoe_checked.so")
ALTGRID_LIBRARY = os.path.join(_PKG, "libmxmoe_altgrid.so")


def _library_from_env() -> str:
    which = os.environ.get("MXMOE_LIBRARY", "")
    if which in ("", "product"):
        return PRODUCT_LIBRARY
    if which == "checked":
        return CHECKED_LIBRARY
    if which == "altgrid":
        return ALTGRID_LIBRARY
    raise ImportError(f"MXMOE_LIBRARY={which!r}: expected 'product', 'checked' or 'altgrid'")


_LIB_PATH = _library_from_env()

# mx_dtype codes of mxmoe.h
MX_F32, MX_F16, MX_BF16, MX_FP8_E4M3, MX_I32, MX_I64 = range(6)
_FLOAT_CODES = {torch.float32: MX_F32, torch.float16: MX_F16, torch.bfloat16: MX_BF16}
MAX_EXPERTS = 1024

EXPORTED_SYMBOLS = (
    "mx_status_string", "mx_last_hip_error", "mx_dispatch_capacity",
    "mx_prepare_workspace_size", "mx_prepare_moe_input", "mx_shuffle_rows",
    "mx_dispatch_rows", "mx_apply_shuffle_mul_sum", "mx_moe_output_memset",
    "mx_zero_padding_rows", "mx_moe_sort", "mx_dispatch_rows_fp8",
    "mx_dispatch_rows_timed", "mx_apply_shuffle_mul_sum_timed", "mx_prepare_moe_input_timed",
    "mx_prepare_moe_input_noalloc", "mx_prepare_dispatch",
    "mx_bounds_checked", "mx_bounds_report", "mx_bounds_shrink_outputs",
)


class MxError(RuntimeError):
    def __init__(self, status: int, what: str):
        lib = load_library()
        msg = lib.mx_status_string(status).decode()
        if status == 6:
            msg += f" (hipError_t {lib.mx_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmxmoe.so (built by ``python -m combine_topk_ids_expert_amd.build``),
    or libmxmoe_checked.so with ``MXMOE_LIBRARY=checked``; every call of this
    module goes to the library loaded here."""
    global _lib
    if _lib is None:
        _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path: str):
    """A ctypes handle of the library at ``path`` (libmxmoe.so or its checked
    twin) with every entry point's argument types set."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m combine_topk_ids_expert_amd.build`; there is no fallback")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.mx_status_string.restype = ctypes.c_char_p
    lib.mx_status_string.argtypes = [ctypes.c_int]
    lib.mx_last_hip_error.restype = ctypes.c_int
    lib.mx_last_hip_error.argtypes = []
    lib.mx_dispatch_capacity.restype = i64
    lib.mx_dispatch_capacity.argtypes = [i64, i32, i32, i32]
    lib.mx_prepare_workspace_size.restype = sz
    lib.mx_prepare_workspace_size.argtypes = [i64, i32, i32]
    lib.mx_prepare_moe_input.restype = ctypes.c_int
    lib.mx_prepare_moe_input.argtypes = [
        vp, i32, i64, i32, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, i64, vp, vp, i32, vp, sz, vp]
    lib.mx_prepare_moe_input_timed.restype = ctypes.c_int
    lib.mx_prepare_moe_input_timed.argtypes = [
        vp, i32, i64, i32, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, i64, vp, vp, i32, vp, sz, vp, vp, vp]
    lib.mx_prepare_moe_input_noalloc.restype = ctypes.c_int
    lib.mx_prepare_moe_input_noalloc.argtypes = [
        vp, i32, i64, i32, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, i64, vp, vp, i32, vp]
    lib.mx_prepare_dispatch.restype = ctypes.c_int
    lib.mx_prepare_dispatch.argtypes = [
        vp, i32, i64, i32, i32, i32, i32, i32, i32, i32,
        vp, vp, vp, vp, i64, vp, vp, i32, vp, sz,
        vp, i64, vp, i64, vp, i64, vp, vp]
    lib.mx_shuffle_rows.restype = ctypes.c_int
    lib.mx_shuffle_rows.argtypes = [vp, i64, i64, vp, i64, vp, vp]
    lib.mx_dispatch_rows.restype = ctypes.c_int
    lib.mx_dispatch_rows.argtypes = [vp, i64, i32, i64, vp, vp, i64, vp, i64, vp, vp]
    lib.mx_apply_shuffle_mul_sum.restype = ctypes.c_int
    lib.mx_apply_shuffle_mul_sum.argtypes = [vp, i32, i64, i64, vp, vp, i32, i64, i32, vp, i32, vp]
    lib.mx_dispatch_rows_timed.restype = ctypes.c_int
    lib.mx_dispatch_rows_timed.argtypes = [vp, i64, i32, i64, vp, vp, i64, vp, i64, vp, vp, vp, vp]
    lib.mx_apply_shuffle_mul_sum_timed.restype = ctypes.c_int
    lib.mx_apply_shuffle_mul_sum_timed.argtypes = [vp, i32, i64, i64, vp, vp, i32, i64, i32, vp,
                                                   i32, vp, vp, vp]
    lib.mx_moe_output_memset.restype = ctypes.c_int
    lib.mx_moe_output_memset.argtypes = [vp, i64, i32, i64, vp, vp]
    lib.mx_zero_padding_rows.restype = ctypes.c_int
    lib.mx_zero_padding_rows.argtypes = [vp, i64, i64, vp, vp, i32, vp]
    lib.mx_dispatch_rows_fp8.restype = ctypes.c_int
    lib.mx_dispatch_rows_fp8.argtypes = [vp, i32, i64, i32, i64, vp, vp, vp, i64, vp]
    lib.mx_moe_sort.restype = ctypes.c_int
    lib.mx_moe_sort.argtypes = [vp, i32, i64, i32, i32, i32, i32, i32, vp, vp, i64, vp, vp, i64,
                                vp, vp, vp, vp, sz, vp]
    lib.mx_bounds_checked.restype = i32
    lib.mx_bounds_checked.argtypes = []
    lib.mx_bounds_report.restype = ctypes.c_int
    lib.mx_bounds_report.argtypes = [ctypes.POINTER(ctypes.c_uint64), i32]
    lib.mx_bounds_shrink_outputs.restype = ctypes.c_int
    lib.mx_bounds_shrink_outputs.argtypes = [i64]
    return lib


def bounds_checked() -> bool:
    """Whether the loaded library is the bounds-checked one."""
    return bool(load_library().mx_bounds_checked())


def bounds_report(clear: bool = True) -> dict:
    """Out-of-bounds accesses the checked library's kernels counted since the
    last clear: loads, stores, and the address (or on-chip index) and site
    code of the first one (all zero with libmxmoe.so)."""
    r = (ctypes.c_uint64 * 4)()
    _call(load_library().mx_bounds_report(r, 1 if clear else 0), "bounds_report")
    return {"loads": int(r[0]), "stores": int(r[1]), "first_address": int(r[2]),
            "first_site": int(r[3])}


def bounds_shrink_outputs(nbytes: int) -> None:
    """Checked library: describe every output array to the kernels as
    ``nbytes`` shorter than it is, from the next call on (0 restores)."""
    _call(load_library().mx_bounds_shrink_outputs(int(nbytes)), "bounds_shrink_outputs")


def _ptr(t: torch.Tensor | None):
    if t is None or t.numel() == 0:
        return None
    return t.data_ptr()


def _check_dev(name: str, t: torch.Tensor, device: torch.device | None = None):
    # is_cuda / get_device() are the cheap forms of the device checks (a call
    # is host-bound at small batch sizes).
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU (got {t.device})")
    if device is not None and t.get_device() != device.index:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_i32(name: str, t: torch.Tensor, numel: int | None = None):
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32 (got {t.dtype})")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements (got {t.numel()})")


def _row_bytes(t: torch.Tensor) -> int:
    return math.prod(t.shape[1:]) * t.element_size()


# The current stream's raw handle: torch's private accessor skips building a
# Stream object (about 0.1 us against 1.9 us per call on MI355X hosts, which
# matters at small batch sizes where a call is host-bound); the public API is
# the fallback.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device: torch.device):
    if _raw_stream is not None and device.index is not None:
        return _raw_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _on(device: torch.device, fn, *args):
    """Call the C entry point ``fn(*args, stream)`` with the tensors' device
    current: HIP launches on the current device, so a call on tensors of
    another device switches to it for the launch (and back)."""
    if device.index is not None and device.index != torch.cuda.current_device():
        with torch.cuda.device(device):
            return fn(*args, _stream(device))
    return fn(*args, _stream(device))


def _call(status: int, what: str):
    if status != 0:
        raise MxError(status, what)


class BoundCall:
    """One call of a C entry point whose arguments were checked and marshalled
    once (see ``bind``).  Calling it enqueues the same work on the tensors'
    device's current stream.  It holds the tensors it points to, so they stay
    allocated while it lives; it does not see later changes to them (resizing
    or replacing a tensor needs a new bind).

    ``result`` is what the plain call returns (e.g. the output tensor).
    ``bound(kernel_events=(start, stop))`` uses the timed entry point, where
    the call has one."""

    __slots__ = ("_fn", "_timed", "_args", "_dev", "_what", "result", "_keep")

    def __init__(self, name: str, timed: str | None, args: tuple, dev: torch.device, what: str,
                 result, keep: tuple):
        lib = load_library()
        fn = getattr(lib, name)
        # pre-built ctypes objects pass through the argument conversion as they are
        self._args = tuple(t(a) if not isinstance(a, t) else a
                           for t, a in zip(fn.argtypes, args))
        self._fn = fn
        self._timed = getattr(lib, timed) if timed else None
        self._dev = dev
        self._what = what
        self.result = result
        self._keep = keep

    def __call__(self, kernel_events=None):
        dev = self._dev
        if kernel_events is None:
            st = _on(dev, self._fn, *self._args)
        else:
            if self._timed is None:
                raise ValueError(f"{self._what} has no timed form")
            st = _on(dev, self._timed, *self._args, *_event_handles(kernel_events))
        if st != 0:
            raise MxError(st, self._what)
        return self.result


def bind(fn, *args, **kwargs) -> BoundCall:
    """Check and marshal ``fn(*args, **kwargs)`` (one of this module's calls)
    once and return a ``BoundCall`` that repeats it without the checks."""
    bindable = (prepare_moe_input, shuffle_rows, dispatch_rows, apply_shuffle_mul_sum,
                moe_output_memset, zero_padding_rows, dispatch_rows_fp8, prepare_dispatch)
    if fn not in bindable:
        raise TypeError(f"cannot bind {getattr(fn, '__name__', fn)!r}")
    return fn(*args, _bind=True, **kwargs)


def _finish(dev: torch.device, name: str, args: tuple, what: str, bind_: bool, result=None,
            keep: tuple = (), timed: str | None = None, kernel_events=None):
    """Run (or, with bind_, bind) the entry point ``name`` on checked args."""
    if bind_:
        return BoundCall(name, timed, args, dev, what, result, keep)
    lib = load_library()
    if kernel_events is None:
        _call(_on(dev, getattr(lib, name), *args), what)
    else:
        _call(_on(dev, getattr(lib, timed), *args, *_event_handles(kernel_events)), what)
    return result


def _event_handles(kernel_events):
    """Raw hipEvent_t handles of a (start, stop) pair of torch.cuda.Event
    (created with enable_timing=True), for the timed entry points.  torch
    creates an event's HIP handle at its first record, so each event must have
    been recorded once before."""
    start, stop = kernel_events
    hs = []
    for e in (start, stop):
        if not isinstance(e, torch.cuda.Event):
            raise TypeError("kernel_events must be two torch.cuda.Event")
        if not e.cuda_event:
            raise ValueError("record each kernel event once before passing it (torch creates "
                             "the HIP event at its first record)")
        hs.append(e.cuda_event)
    return hs


def dispatch_capacity(num_tokens: int, topk: int, num_experts: int, row_align: int = 1) -> int:
    """Rows a dispatched buffer needs for any routing (T*k + E*(row_align-1))."""
    cap = load_library().mx_dispatch_capacity(num_tokens, topk, num_experts, row_align)
    if cap < 0:
        raise ValueError("dispatch capacity out of range")
    return cap


def prepare_workspace_size(num_tokens: int, topk: int, num_experts: int) -> int:
    return load_library().mx_prepare_workspace_size(num_tokens, topk, num_experts)


def empty_routing(num_tokens: int, topk: int, num_experts: int, device, row_align: int = 1,
                  blockscale: bool = False) -> dict:
    """Output and workspace tensors for prepare_moe_input (torch.empty)."""
    cap = dispatch_capacity(num_tokens, topk, num_experts, row_align)
    E = num_experts
    out = {
        "expert_offsets": torch.empty(E + 1, dtype=torch.int32, device=device),
        "problem_sizes1": torch.empty(E, 3, dtype=torch.int32, device=device),
        "problem_sizes2": torch.empty(E, 3, dtype=torch.int32, device=device),
        "input_permutation": torch.empty(cap, dtype=torch.int32, device=device),
        "output_permutation": torch.empty(num_tokens * topk, dtype=torch.int32, device=device),
        "blockscale_offsets": (torch.empty(E + 1, dtype=torch.int32, device=device)
                               if blockscale else None),
        "workspace": torch.empty(max(prepare_workspace_size(num_tokens, topk, E), 4),
                                 dtype=torch.uint8, device=device),
    }
    return out


def _prepare_args(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
                  output_permutation, num_experts, n, k, blockscale_offsets, row_align,
                  blockscale_align, workspace):
    """Checked ctypes arguments of mx_prepare_moe_input (without the stream),
    the device and the tensors they point to."""
    lib = load_library()
    _check_dev("topk_ids", topk_ids)
    dev = topk_ids.device
    if topk_ids.dim() != 2 or topk_ids.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_ids must be a 2-D int32 or int64 tensor")
    T, topk = topk_ids.shape
    E = int(num_experts)
    for name, t, numel in [("expert_offsets", expert_offsets, E + 1),
                           ("output_permutation", output_permutation, T * topk),
                           ("input_permutation", input_permutation, None),
                           ("problem_sizes1", problem_sizes1, 3 * E),
                           ("problem_sizes2", problem_sizes2, 3 * E),
                           ("blockscale_offsets", blockscale_offsets, E + 1)]:
        if t is None:
            if name in ("expert_offsets", "output_permutation", "input_permutation"):
                raise ValueError(f"{name} is required")
            continue
        _check_dev(name, t, dev)
        _check_i32(name, t, numel)
    if workspace is None:
        workspace = torch.empty(max(lib.mx_prepare_workspace_size(T, topk, E), 4),
                                dtype=torch.uint8, device=dev)
    _check_dev("workspace", workspace, dev)
    args = (_ptr(topk_ids), MX_I64 if topk_ids.dtype == torch.int64 else MX_I32, T, topk, E,
            2 * n, k, k, n, row_align,
            _ptr(expert_offsets), _ptr(problem_sizes1), _ptr(problem_sizes2),
            _ptr(input_permutation), input_permutation.numel(), _ptr(output_permutation),
            _ptr(blockscale_offsets), blockscale_align,
            _ptr(workspace), workspace.numel() * workspace.element_size())
    keep = (topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
            output_permutation, blockscale_offsets, workspace)
    return dev, args, keep


def prepare_moe_input(topk_ids: torch.Tensor, expert_offsets: torch.Tensor,
                      problem_sizes1: torch.Tensor | None, problem_sizes2: torch.Tensor | None,
                      input_permutation: torch.Tensor, output_permutation: torch.Tensor,
                      num_experts: int, n: int, k: int,
                      blockscale_offsets: torch.Tensor | None = None, *,
                      row_align: int = 1, blockscale_align: int = 128,
                      workspace: torch.Tensor | None = None, kernel_events=None,
                      _bind: bool = False):
    """Routing metadata for ``topk_ids`` [T, topk] (int32 or int64), in place.

    ``n`` and ``k`` are the expert MLP's intermediate and hidden sizes; the
    problem sizes are (count, 2n, k) for the gate+up GEMM and (count, k, n)
    for the down GEMM.  ``input_permutation`` must hold at least
    ``dispatch_capacity(T, topk, num_experts, row_align)`` entries.

    kernel_events: optional (start, stop) torch.cuda.Event pair, recorded with
    the begin and end of the routing kernels themselves
    (mx_prepare_moe_input_timed).
    """
    dev, args, keep = _prepare_args(topk_ids, expert_offsets, problem_sizes1, problem_sizes2,
                                    input_permutation, output_permutation, num_experts, n, k,
                                    blockscale_offsets, row_align, blockscale_align, workspace)
    return _finish(dev, "mx_prepare_moe_input", args, "prepare_moe_input", _bind, None, keep,
                   "mx_prepare_moe_input_timed", kernel_events)


def prepare_moe_input_noalloc(topk_ids: torch.Tensor, expert_offsets: torch.Tensor,
                              problem_sizes1: torch.Tensor | None,
                              problem_sizes2: torch.Tensor | None,
                              input_permutation: torch.Tensor, output_permutation: torch.Tensor,
                              num_experts: int, n: int, k: int,
                              blockscale_offsets: torch.Tensor | None = None, *,
                              row_align: int = 1, blockscale_align: int = 128) -> None:
    """prepare_moe_input without a workspace (mx_prepare_moe_input_noalloc):
    the routing scratch is the library's own per-GPU array, so the call
    allocates nothing.  Calls that overlap on one GPU share that array and
    race; calls ordered on one stream are safe."""
    lib = load_library()
    _check_dev("topk_ids", topk_ids)
    dev = topk_ids.device
    if topk_ids.dim() != 2 or topk_ids.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_ids must be a 2-D int32 or int64 tensor")
    T, topk = topk_ids.shape
    E = int(num_experts)
    for name, t, numel in [("expert_offsets", expert_offsets, E + 1),
                           ("output_permutation", output_permutation, T * topk),
                           ("input_permutation", input_permutation, None),
                           ("problem_sizes1", problem_sizes1, 3 * E),
                           ("problem_sizes2", problem_sizes2, 3 * E),
                           ("blockscale_offsets", blockscale_offsets, E + 1)]:
        if t is None:
            if name in ("expert_offsets", "output_permutation", "input_permutation"):
                raise ValueError(f"{name} is required")
            continue
        _check_dev(name, t, dev)
        _check_i32(name, t, numel)
    _call(_on(dev, lib.mx_prepare_moe_input_noalloc,
              _ptr(topk_ids), MX_I64 if topk_ids.dtype == torch.int64 else MX_I32, T, topk, E,
              2 * n, k, k, n, row_align,
              _ptr(expert_offsets), _ptr(problem_sizes1), _ptr(problem_sizes2),
              _ptr(input_permutation), input_permutation.numel(), _ptr(output_permutation),
              _ptr(blockscale_offsets), blockscale_align), "prepare_moe_input_noalloc")


def shuffle_rows(input: torch.Tensor, dst2src_map: torch.Tensor,
                 output: torch.Tensor | tuple | None = None, _bind: bool = False) -> torch.Tensor:
    """output[r] = input[dst2src_map[r]] byte for byte (rows with an index out
    of range keep their contents).  Any dtype; row = everything past dim 0.
    ``output`` is the tensor to write, or its shape (as sglang's shuffle_rows
    takes it), or None; either of the latter two allocates it."""
    lib = load_library()
    _check_dev("input", input)
    dev = input.device
    _check_dev("dst2src_map", dst2src_map, dev)
    _check_i32("dst2src_map", dst2src_map)
    n_dst = dst2src_map.numel()
    if output is None:
        output = torch.empty((n_dst,) + tuple(input.shape[1:]), dtype=input.dtype, device=dev)
    elif not isinstance(output, torch.Tensor):
        output = torch.empty(tuple(output), dtype=input.dtype, device=dev)
    _check_dev("output", output, dev)
    if output.dtype != input.dtype or output.shape[1:] != input.shape[1:] or len(output) != n_dst:
        raise ValueError("output must be [len(dst2src_map), *input.shape[1:]] of input's dtype")
    row_bytes = _row_bytes(input)
    if not n_dst and not _bind:
        return output
    args = (_ptr(input), input.shape[0], row_bytes, _ptr(dst2src_map), n_dst, _ptr(output))
    return _finish(dev, "mx_shuffle_rows", args, "shuffle_rows", _bind, output,
                   (input, dst2src_map, output))


def _dispatch_args(input, output_permutation, topk, output, side_input, side_output):
    """Checked ctypes arguments of mx_dispatch_rows (without the stream) and
    the device."""
    _check_dev("input", input)
    dev = input.device
    _check_dev("output_permutation", output_permutation, dev)
    _check_i32("output_permutation", output_permutation, input.shape[0] * topk)
    _check_dev("output", output, dev)
    if output.dtype != input.dtype or output.shape[1:] != input.shape[1:]:
        raise ValueError("output must have input's dtype and row shape")
    side_rb = 0
    if side_input is not None or side_output is not None:
        if side_input is None or side_output is None:
            raise ValueError("side_input and side_output go together")
        _check_dev("side_input", side_input, dev)
        _check_dev("side_output", side_output, dev)
        if side_input.shape[0] != input.shape[0] or side_output.shape[0] != output.shape[0] or \
                side_output.shape[1:] != side_input.shape[1:] or side_output.dtype != side_input.dtype:
            raise ValueError("side rows must match the main rows' counts and each other's shape")
        side_rb = _row_bytes(side_input)
    T = input.shape[0]
    args = (_ptr(input), T, topk, _row_bytes(input), _ptr(output_permutation), _ptr(output),
            output.shape[0], _ptr(side_input), side_rb, _ptr(side_output))
    return dev, args


def dispatch_rows(input: torch.Tensor, output_permutation: torch.Tensor, topk: int,
                  output: torch.Tensor, side_input: torch.Tensor | None = None,
                  side_output: torch.Tensor | None = None,
                  kernel_events=None, _bind: bool = False) -> torch.Tensor:
    """output[output_permutation[t*topk + j]] = input[t] for every token t and
    pick j (destinations out of range are skipped); optionally the same for
    a side row per token (e.g. FP8 block scales).

    kernel_events: optional (start, stop) torch.cuda.Event pair, recorded with
    the begin and end of the dispatch kernels themselves (mx_dispatch_rows_timed)."""
    dev, args = _dispatch_args(input, output_permutation, topk, output, side_input, side_output)
    if not (args[1] and args[6]) and not _bind:
        return output
    return _finish(dev, "mx_dispatch_rows", args, "dispatch_rows", _bind, output,
                   (input, output_permutation, output, side_input, side_output),
                   "mx_dispatch_rows_timed", kernel_events)


def prepare_dispatch(topk_ids: torch.Tensor, expert_offsets: torch.Tensor,
                     problem_sizes1: torch.Tensor | None, problem_sizes2: torch.Tensor | None,
                     input_permutation: torch.Tensor, output_permutation: torch.Tensor,
                     num_experts: int, n: int, k: int, input: torch.Tensor,
                     output: torch.Tensor, blockscale_offsets: torch.Tensor | None = None, *,
                     side_input: torch.Tensor | None = None,
                     side_output: torch.Tensor | None = None, row_align: int = 1,
                     blockscale_align: int = 128, workspace: torch.Tensor | None = None,
                     _bind: bool = False) -> torch.Tensor:
    """prepare_moe_input(...) and then dispatch_rows(input, output_permutation,
    topk, output, side_input, side_output) in one call (mx_prepare_dispatch),
    with the same results.  At decode-sized batches the library runs both in
    one launch.  Returns ``output``."""
    dev, pargs, pkeep = _prepare_args(topk_ids, expert_offsets, problem_sizes1, problem_sizes2,
                                      input_permutation, output_permutation, num_experts, n, k,
                                      blockscale_offsets, row_align, blockscale_align, workspace)
    if input.shape[0] != topk_ids.shape[0]:
        raise ValueError("input must have one row per token of topk_ids")
    ddev, dargs = _dispatch_args(input, output_permutation, topk_ids.shape[1], output,
                                 side_input, side_output)
    if ddev != dev:
        raise ValueError("input is on another device than topk_ids")
    # mx_dispatch_rows args: src, T, topk, row_bytes, perm, dst, n_dst, side_src, side_rb, side_dst
    args = pargs + (dargs[0], dargs[3], dargs[5], dargs[6], dargs[7], dargs[8], dargs[9])
    return _finish(dev, "mx_prepare_dispatch", args, "prepare_dispatch", _bind, output,
                   pkeep + (input, output, side_input, side_output))


def apply_shuffle_mul_sum(input: torch.Tensor, output: torch.Tensor,
                          permutation: torch.Tensor, factors: torch.Tensor | None = None,
                          kernel_events=None, _bind: bool = False):
    """output[t] = round(sum_j factors[t, j] * input[permutation[t*k + j]]) with
    fp32 accumulation (k = permutation.numel() // output.shape[0]); in place.

    kernel_events: optional (start, stop) torch.cuda.Event pair, recorded with
    the begin and end of the combine kernels themselves
    (mx_apply_shuffle_mul_sum_timed)."""
    lib = load_library()
    _check_dev("input", input)
    dev = input.device
    _check_dev("output", output, dev)
    _check_dev("permutation", permutation, dev)
    _check_i32("permutation", permutation)
    if input.dtype not in _FLOAT_CODES or output.dtype not in _FLOAT_CODES:
        raise TypeError("input and output must be float32, float16 or bfloat16")
    if input.dim() != 2 or output.dim() != 2 or input.shape[1] != output.shape[1]:
        raise ValueError("input [rows, hidden] and output [tokens, hidden] must share hidden")
    T, H = output.shape
    if T == 0 and not _bind:
        return None
    if T and permutation.numel() % T:
        raise ValueError("permutation length must be a multiple of the token count")
    topk = permutation.numel() // T if T else 1
    fcode = 0
    if factors is not None:
        _check_dev("factors", factors, dev)
        if factors.dtype not in _FLOAT_CODES or factors.numel() != T * topk:
            raise ValueError("factors must be [tokens, topk] float32 / float16 / bfloat16")
        fcode = _FLOAT_CODES[factors.dtype]
    args = (_ptr(input), _FLOAT_CODES[input.dtype], input.shape[0], H, _ptr(permutation),
            _ptr(factors), fcode, T, topk, _ptr(output), _FLOAT_CODES[output.dtype])
    return _finish(dev, "mx_apply_shuffle_mul_sum", args, "apply_shuffle_mul_sum", _bind, None,
                   (input, output, permutation, factors), "mx_apply_shuffle_mul_sum_timed",
                   kernel_events)


def moe_output_memset(output: torch.Tensor, output_permutation: torch.Tensor, topk: int,
                      _bind: bool = False):
    """In place: output row t becomes zeros iff one of its picks has a
    permuted index >= 0; the other rows are left untouched."""
    lib = load_library()
    _check_dev("output", output)
    dev = output.device
    T = output.shape[0]
    _check_dev("output_permutation", output_permutation, dev)
    _check_i32("output_permutation", output_permutation, T * topk)
    if not T and not _bind:
        return None
    args = (_ptr(output), T, topk, _row_bytes(output), _ptr(output_permutation))
    return _finish(dev, "mx_moe_output_memset", args, "moe_output_memset", _bind, None,
                   (output, output_permutation))


def zero_padding_rows(rows: torch.Tensor, input_permutation: torch.Tensor,
                      expert_offsets: torch.Tensor | None = None, _bind: bool = False):
    """In place: dispatched rows below the padded total (expert_offsets[-1],
    read on the device) whose source index is negative become zeros."""
    lib = load_library()
    _check_dev("rows", rows)
    dev = rows.device
    n = rows.shape[0]
    _check_dev("input_permutation", input_permutation, dev)
    _check_i32("input_permutation", input_permutation)
    if input_permutation.numel() < n:
        raise ValueError("input_permutation must cover every row")
    E = 0
    if expert_offsets is not None:
        _check_dev("expert_offsets", expert_offsets, dev)
        _check_i32("expert_offsets", expert_offsets)
        E = expert_offsets.numel() - 1
    if not n and not _bind:
        return None
    args = (_ptr(rows), n, _row_bytes(rows), _ptr(input_permutation), _ptr(expert_offsets), E)
    return _finish(dev, "mx_zero_padding_rows", args, "zero_padding_rows", _bind, None,
                   (rows, input_permutation, expert_offsets))


def moe_sort(topk_ids: torch.Tensor, num_experts: int, local_expert_offset: int,
             num_local_experts: int, tile_size: int, out: dict | None = None,
             workspace: torch.Tensor | None = None) -> dict:
    """Tile-padded sort metadata for the experts [local_expert_offset,
    local_expert_offset + num_local_experts) (see mx_moe_sort).  Returns a dict
    of int32 tensors: expanded_idx_to_permuted_idx [T*k],
    permuted_idx_to_expanded_idx [capacity], tile_idx_to_group_idx and
    tile_idx_to_mn_limit [max_tiles], total_num_padded_tokens [1],
    num_non_exiting_tiles [1], expert_offsets [num_local_experts + 1];
    ``out`` may supply any of them (already allocated, written in place)."""
    lib = load_library()
    _check_dev("topk_ids", topk_ids)
    dev = topk_ids.device
    if topk_ids.dim() != 2 or topk_ids.dtype not in (torch.int32, torch.int64):
        raise TypeError("topk_ids must be a 2-D int32 or int64 tensor")
    T, topk = topk_ids.shape
    cap = dispatch_capacity(T, topk, num_local_experts, tile_size)
    max_tiles = -(-cap // tile_size)
    sizes = {"expanded_idx_to_permuted_idx": T * topk, "permuted_idx_to_expanded_idx": cap,
             "tile_idx_to_group_idx": max_tiles, "tile_idx_to_mn_limit": max_tiles,
             "total_num_padded_tokens": 1, "num_non_exiting_tiles": 1,
             "expert_offsets": num_local_experts + 1}
    res = dict(out or {})
    for name, numel in sizes.items():
        if name not in res or res[name] is None:
            res[name] = torch.empty(numel, dtype=torch.int32, device=dev)
        _check_dev(name, res[name], dev)
        _check_i32(name, res[name])
        if name not in ("permuted_idx_to_expanded_idx", "tile_idx_to_group_idx",
                        "tile_idx_to_mn_limit") and res[name].numel() != numel:
            raise ValueError(f"{name} must have {numel} elements")
    if workspace is None:
        workspace = torch.empty(max(lib.mx_prepare_workspace_size(T, topk, num_local_experts), 4),
                                dtype=torch.uint8, device=dev)
    _check_dev("workspace", workspace, dev)
    nt = min(res["tile_idx_to_group_idx"].numel(), res["tile_idx_to_mn_limit"].numel())
    _call(_on(
        dev, lib.mx_moe_sort,
        _ptr(topk_ids), MX_I64 if topk_ids.dtype == torch.int64 else MX_I32, T, topk, num_experts,
        local_expert_offset, num_local_experts, tile_size,
        _ptr(res["expanded_idx_to_permuted_idx"]), _ptr(res["permuted_idx_to_expanded_idx"]),
        res["permuted_idx_to_expanded_idx"].numel(), _ptr(res["tile_idx_to_group_idx"]),
        _ptr(res["tile_idx_to_mn_limit"]), nt, _ptr(res["total_num_padded_tokens"]),
        _ptr(res["num_non_exiting_tiles"]), _ptr(res["expert_offsets"]),
        _ptr(workspace), workspace.numel() * workspace.element_size()), "moe_sort")
    return res


def dispatch_rows_fp8(input: torch.Tensor, output_permutation: torch.Tensor, topk: int,
                      output: torch.Tensor, output_scales: torch.Tensor, _bind: bool = False):
    """Quantize bf16 token rows to e4m3fn in 1x128 groups (scale = amax / 448)
    and write codes and scales to each token's k dispatched rows, in place.
    output: [rows, hidden] torch.float8_e4m3fn (or uint8); output_scales:
    [rows, hidden / 128] float32."""
    lib = load_library()
    _check_dev("input", input)
    dev = input.device
    if input.dtype != torch.bfloat16 or input.dim() != 2:
        raise TypeError("input must be a 2-D bfloat16 tensor")
    T, H = input.shape
    _check_dev("output_permutation", output_permutation, dev)
    _check_i32("output_permutation", output_permutation, T * topk)
    _check_dev("output", output, dev)
    _check_dev("output_scales", output_scales, dev)
    if output.element_size() != 1 or output.dim() != 2 or output.shape[1] != H:
        raise ValueError("output must be [rows, hidden] of a 1-byte dtype")
    if output_scales.dtype != torch.float32 or tuple(output_scales.shape) != (output.shape[0], H // 128):
        raise ValueError("output_scales must be float32 [rows, hidden / 128]")
    args = (_ptr(input), MX_BF16, T, topk, H, _ptr(output_permutation), _ptr(output),
            _ptr(output_scales), output.shape[0])
    return _finish(dev, "mx_dispatch_rows_fp8", args, "dispatch_rows_fp8", _bind, None,
                   (input, output_permutation, output, output_scales))

