"""The custom-operator registration (combine_topk_ids_expert_amd.ops) on the
host: every call is a torch.ops.mxmoe operator whose schema marks exactly its
outputs as mutated, and CPU tensors are refused (the operators have a GPU
implementation only)."""

import pytest
import torch

import combine_topk_ids_expert_amd.ops  # noqa: F401  (registers torch.ops.mxmoe)

MUTATED = {
    "prepare_moe_input": {"expert_offsets", "problem_sizes1", "problem_sizes2",
                          "input_permutation", "output_permutation", "blockscale_offsets",
                          "workspace"},
    "prepare_dispatch": {"expert_offsets", "problem_sizes1", "problem_sizes2",
                         "input_permutation", "output_permutation", "blockscale_offsets",
                         "workspace", "output", "side_output"},
    "shuffle_rows": {"output"},
    "dispatch_rows": {"output", "side_output"},
    "apply_shuffle_mul_sum": {"output"},
    "moe_output_memset": {"output"},
    "zero_padding_rows": {"rows"},
    "dispatch_rows_fp8": {"output", "output_scales"},
    "moe_sort": {"expanded_idx_to_permuted_idx", "permuted_idx_to_expanded_idx",
                 "tile_idx_to_group_idx", "tile_idx_to_mn_limit", "total_num_padded_tokens",
                 "num_non_exiting_tiles", "expert_offsets", "workspace"},
}


@pytest.mark.parametrize("name", sorted(MUTATED))
def test_schema_marks_the_outputs_mutated(name):
    schema = getattr(torch.ops.mxmoe, name).default._schema
    written = {a.name for a in schema.arguments
               if a.alias_info is not None and a.alias_info.is_write}
    assert written == MUTATED[name]
    assert len(schema.returns) == 0


def test_cpu_tensors_are_refused():
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    perm = torch.zeros(4, dtype=torch.int32)
    out = torch.empty_like(x)
    with pytest.raises((NotImplementedError, RuntimeError)):
        torch.ops.mxmoe.shuffle_rows(x, perm, out)
