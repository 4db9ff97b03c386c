"""The library's calls as PyTorch custom operators: ``torch.ops.mxmoe.*``.

The sglang page "[jit_kernel] Add prepare_moe_input JIT kernels" registers
its three calls as custom operators whose output arguments are mutated in
place ("Changes").  Importing this module does the same for every call of
this package: each operator declares the tensors it writes in
``mutates_args`` and runs the binding's call, so the library's kernels do the
work; its fake implementation only states that nothing is returned, so
``torch.compile`` traces through the calls without graph breaks.

    import combine_topk_ids_expert_amd.ops
    torch.ops.mxmoe.prepare_moe_input(ids, eo, ps1, ps2, inp, outp, E, n, k, bso, 1, 128, ws)

Outputs and workspaces are caller-allocated, as in the binding
(``empty_routing``, ``dispatch_capacity``, ``prepare_workspace_size``).
"""

from __future__ import annotations

from typing import Optional

import torch
from torch import Tensor

from . import (apply_shuffle_mul_sum as _combine, dispatch_rows as _dispatch,
               dispatch_rows_fp8 as _dispatch_fp8, moe_output_memset as _memset,
               moe_sort as _moe_sort, prepare_dispatch as _prepare_dispatch,
               prepare_moe_input as _prepare, shuffle_rows as _shuffle,
               zero_padding_rows as _zero_padding)

__all__ = ["OPS"]

_META = ("expert_offsets", "problem_sizes1", "problem_sizes2", "input_permutation",
         "output_permutation", "blockscale_offsets", "workspace")


@torch.library.custom_op("mxmoe::prepare_moe_input", mutates_args=_META, device_types="cuda")
def prepare_moe_input(topk_ids: Tensor, expert_offsets: Tensor, problem_sizes1: Optional[Tensor],
                      problem_sizes2: Optional[Tensor], input_permutation: Tensor,
                      output_permutation: Tensor, num_experts: int, n: int, k: int,
                      blockscale_offsets: Optional[Tensor], row_align: int,
                      blockscale_align: int, workspace: Tensor) -> None:
    _prepare(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
             output_permutation, num_experts, n, k, blockscale_offsets, row_align=row_align,
             blockscale_align=blockscale_align, workspace=workspace)


@torch.library.custom_op("mxmoe::prepare_dispatch", mutates_args=_META + ("output", "side_output"),
                         device_types="cuda")
def prepare_dispatch(topk_ids: Tensor, expert_offsets: Tensor, problem_sizes1: Optional[Tensor],
                     problem_sizes2: Optional[Tensor], input_permutation: Tensor,
                     output_permutation: Tensor, num_experts: int, n: int, k: int, input: Tensor,
                     output: Tensor, blockscale_offsets: Optional[Tensor],
                     side_input: Optional[Tensor], side_output: Optional[Tensor], row_align: int,
                     blockscale_align: int, workspace: Tensor) -> None:
    _prepare_dispatch(topk_ids, expert_offsets, problem_sizes1, problem_sizes2,
                      input_permutation, output_permutation, num_experts, n, k, input, output,
                      blockscale_offsets, side_input=side_input, side_output=side_output,
                      row_align=row_align, blockscale_align=blockscale_align,
                      workspace=workspace)


@torch.library.custom_op("mxmoe::shuffle_rows", mutates_args=("output",), device_types="cuda")
def shuffle_rows(input: Tensor, dst2src_map: Tensor, output: Tensor) -> None:
    _shuffle(input, dst2src_map, output)


@torch.library.custom_op("mxmoe::dispatch_rows", mutates_args=("output", "side_output"),
                         device_types="cuda")
def dispatch_rows(input: Tensor, output_permutation: Tensor, topk: int, output: Tensor,
                  side_input: Optional[Tensor], side_output: Optional[Tensor]) -> None:
    _dispatch(input, output_permutation, topk, output, side_input, side_output)


@torch.library.custom_op("mxmoe::apply_shuffle_mul_sum", mutates_args=("output",),
                         device_types="cuda")
def apply_shuffle_mul_sum(input: Tensor, output: Tensor, permutation: Tensor,
                          factors: Optional[Tensor]) -> None:
    _combine(input, output, permutation, factors)


@torch.library.custom_op("mxmoe::moe_output_memset", mutates_args=("output",),
                         device_types="cuda")
def moe_output_memset(output: Tensor, output_permutation: Tensor, topk: int) -> None:
    _memset(output, output_permutation, topk)


@torch.library.custom_op("mxmoe::zero_padding_rows", mutates_args=("rows",),
                         device_types="cuda")
def zero_padding_rows(rows: Tensor, input_permutation: Tensor,
                      expert_offsets: Optional[Tensor]) -> None:
    _zero_padding(rows, input_permutation, expert_offsets)


@torch.library.custom_op("mxmoe::dispatch_rows_fp8", mutates_args=("output", "output_scales"),
                         device_types="cuda")
def dispatch_rows_fp8(input: Tensor, output_permutation: Tensor, topk: int, output: Tensor,
                      output_scales: Tensor) -> None:
    _dispatch_fp8(input, output_permutation, topk, output, output_scales)


_SORT_OUT = ("expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
             "tile_idx_to_group_idx", "tile_idx_to_mn_limit", "total_num_padded_tokens",
             "num_non_exiting_tiles", "expert_offsets")


@torch.library.custom_op("mxmoe::moe_sort", mutates_args=_SORT_OUT + ("workspace",),
                         device_types="cuda")
def moe_sort(topk_ids: Tensor, num_experts: int, local_expert_offset: int,
             num_local_experts: int, tile_size: int, expanded_idx_to_permuted_idx: Tensor,
             permuted_idx_to_expanded_idx: Tensor, tile_idx_to_group_idx: Tensor,
             tile_idx_to_mn_limit: Tensor, total_num_padded_tokens: Tensor,
             num_non_exiting_tiles: Tensor, expert_offsets: Tensor, workspace: Tensor) -> None:
    out = dict(zip(_SORT_OUT, (expanded_idx_to_permuted_idx, permuted_idx_to_expanded_idx,
                               tile_idx_to_group_idx, tile_idx_to_mn_limit,
                               total_num_padded_tokens, num_non_exiting_tiles, expert_offsets)))
    _moe_sort(topk_ids, num_experts, local_expert_offset, num_local_experts, tile_size, out=out,
              workspace=workspace)


OPS = (prepare_moe_input, prepare_dispatch, shuffle_rows, dispatch_rows, apply_shuffle_mul_sum,
       moe_output_memset, zero_padding_rows, dispatch_rows_fp8, moe_sort)


def _returns_nothing(*args, **kwargs) -> None:
    return None


for _op in OPS:
    _op.register_fake(_returns_nothing)
