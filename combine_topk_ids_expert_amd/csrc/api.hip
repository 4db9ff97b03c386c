// C ABI of mxmoe: argument checks on the host, then the kernel launchers.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing; after the launches the HIP launch status is reported.
#include <hip/hip_runtime.h>

#include "../../include/mxmoe.h"
#include "launch.h"

namespace {

constexpr int64_t kMax31 = (int64_t)0x7fffffff;
// Longest row accepted: just under 64 MiB, so that a row's byte offsets, its
// buffer descriptors' extents and its column-chunk counts stay 32-bit.
constexpr int64_t kMaxRowBytes = (int64_t)65535 * 1024;
thread_local int g_last_hip_error = 0;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

mx_status hip_status(hipError_t e) {
    if (e == hipSuccess) return MX_OK;
    g_last_hip_error = (int)e;
    return MX_ERR_HIP;
}

int elem_bytes(int32_t dt) {
    switch (dt) {
    case MX_F32: return 4;
    case MX_F16: return 2;
    case MX_BF16: return 2;
    default: return 0;
    }
}

}  // namespace

namespace {

// The row dispatch and the combine with optional start / stop events (null
// for the plain entry points).
mx_status dispatch_rows(const void* src, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                        const int32_t* output_permutation, void* dst, int64_t num_dst_rows,
                        const void* side_src, int64_t side_row_bytes, void* side_dst,
                        void* start_event, void* stop_event, void* stream) {
    if (num_tokens < 0 || topk < 1 || row_bytes < 1 || row_bytes > kMaxRowBytes ||
        num_dst_rows < 0 || num_dst_rows > kMax31 || num_tokens > kMax31 / topk)
        return MX_ERR_INVALID_ARGUMENT;
    const bool side = side_src != nullptr || side_dst != nullptr;
    if (side && (side_src == nullptr || side_dst == nullptr || side_row_bytes < 1))
        return MX_ERR_INVALID_ARGUMENT;
    if (!side && side_row_bytes != 0) return MX_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && (src == nullptr || output_permutation == nullptr ||
                           (num_dst_rows > 0 && dst == nullptr)))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(output_permutation, 4)) return MX_ERR_MISALIGNED;
    if (num_tokens == 0 || num_dst_rows == 0) return MX_OK;
    return hip_status(mxmoe::launch_dispatch_rows(
        src, num_tokens, topk, row_bytes, output_permutation, dst, num_dst_rows,
        side ? side_src : nullptr, side ? side_row_bytes : 0, side ? side_dst : nullptr,
        static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(start_event),
        static_cast<hipEvent_t>(stop_event)));
}

mx_status apply_shuffle_mul_sum(const void* y, int32_t y_dtype, int64_t num_y_rows,
                                int64_t hidden, const int32_t* permutation,
                                const void* factors, int32_t factors_dtype,
                                int64_t num_tokens, int32_t topk, void* out, int32_t out_dtype,
                                void* start_event, void* stop_event, void* stream) {
    const int yb = elem_bytes(y_dtype), ob = elem_bytes(out_dtype);
    if (yb == 0 || ob == 0) return MX_ERR_UNSUPPORTED_DTYPE;
    if (factors != nullptr && elem_bytes(factors_dtype) == 0) return MX_ERR_UNSUPPORTED_DTYPE;
    if (num_y_rows < 0 || num_y_rows > kMax31 || hidden < 0 || num_tokens < 0 || topk < 1 ||
        num_tokens > kMax31 / topk || hidden > (int64_t)65535 * 1024 * 8)
        return MX_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && hidden > 0 &&
        (out == nullptr || permutation == nullptr || (num_y_rows > 0 && y == nullptr)))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(y, (size_t)yb) || !aligned(out, (size_t)ob) || !aligned(permutation, 4) ||
        (factors != nullptr && !aligned(factors, (size_t)elem_bytes(factors_dtype))))
        return MX_ERR_MISALIGNED;
    if (num_tokens == 0 || hidden == 0) return MX_OK;
    return hip_status(mxmoe::launch_combine(y, y_dtype, num_y_rows, hidden, permutation, factors,
                                            factors_dtype, num_tokens, topk, out, out_dtype,
                                            static_cast<hipStream_t>(stream),
                                            static_cast<hipEvent_t>(start_event),
                                            static_cast<hipEvent_t>(stop_event)));
}

}  // namespace

extern "C" {

const char* mx_status_string(mx_status s) {
    switch (s) {
    case MX_OK: return "success";
    case MX_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MX_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case MX_ERR_MISALIGNED: return "misaligned pointer";
    case MX_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MX_ERR_CAPACITY: return "input_permutation shorter than the dispatch capacity";
    case MX_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

int mx_last_hip_error(void) { return g_last_hip_error; }

int64_t mx_dispatch_capacity(int64_t num_tokens, int32_t topk, int32_t num_experts,
                             int32_t row_align) {
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || row_align < 1) return -1;
    if (num_tokens > kMax31 / topk) return -1;
    const int64_t cap = num_tokens * topk + (int64_t)num_experts * (row_align - 1);
    return cap > kMax31 ? -1 : cap;
}

size_t mx_prepare_workspace_size(int64_t num_tokens, int32_t topk, int32_t num_experts) {
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_experts > MX_MAX_EXPERTS)
        return 0;
    if (num_tokens > kMax31 / topk) return 0;
    return mxmoe::route_workspace_bytes(num_tokens * topk, num_experts);
}

mx_status mx_prepare_moe_input(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens,
                               int32_t topk, int32_t num_experts,
                               int32_t gemm1_n, int32_t gemm1_k, int32_t gemm2_n, int32_t gemm2_k,
                               int32_t row_align,
                               int32_t* expert_offsets, int32_t* problem_sizes1,
                               int32_t* problem_sizes2,
                               int32_t* input_permutation, int64_t input_permutation_len,
                               int32_t* output_permutation,
                               int32_t* blockscale_offsets, int32_t blockscale_align,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (ids_dtype != MX_I32 && ids_dtype != MX_I64) return MX_ERR_UNSUPPORTED_DTYPE;
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || num_experts > MX_MAX_EXPERTS ||
        row_align < 1)
        return MX_ERR_INVALID_ARGUMENT;
    const int64_t cap = mx_dispatch_capacity(num_tokens, topk, num_experts, row_align);
    if (cap < 0) return MX_ERR_INVALID_ARGUMENT;
    if (blockscale_offsets != nullptr) {
        if (blockscale_align < 1) return MX_ERR_INVALID_ARGUMENT;
        if (num_tokens * topk + (int64_t)num_experts * (blockscale_align - 1) > kMax31)
            return MX_ERR_INVALID_ARGUMENT;
    }
    const int64_t n = num_tokens * topk;
    if ((n > 0 && (topk_ids == nullptr || output_permutation == nullptr)) ||
        expert_offsets == nullptr || (input_permutation_len > 0 && input_permutation == nullptr))
        return MX_ERR_INVALID_ARGUMENT;
    if (input_permutation_len < cap) return MX_ERR_CAPACITY;
    if (input_permutation_len > kMax31) return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(topk_ids, ids_dtype == MX_I64 ? 8 : 4) || !aligned(expert_offsets, 4) ||
        !aligned(problem_sizes1, 4) || !aligned(problem_sizes2, 4) ||
        !aligned(input_permutation, 4) || !aligned(output_permutation, 4) ||
        !aligned(blockscale_offsets, 4) || !aligned(workspace, 4))
        return MX_ERR_MISALIGNED;
    const size_t need = mxmoe::route_workspace_bytes(n, num_experts);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return MX_ERR_WORKSPACE_TOO_SMALL;

    mxmoe::RouteArgs a{};
    a.ids = topk_ids;
    a.ids64 = ids_dtype == MX_I64;
    a.num_picks = n;
    a.topk = topk;
    a.num_experts = num_experts;
    a.row_align = row_align;
    a.bs_align = blockscale_offsets ? blockscale_align : 1;
    a.gemm[0] = gemm1_n;
    a.gemm[1] = gemm1_k;
    a.gemm[2] = gemm2_n;
    a.gemm[3] = gemm2_k;
    a.expert_offsets = expert_offsets;
    a.problem_sizes1 = problem_sizes1;
    a.problem_sizes2 = problem_sizes2;
    a.blockscale_offsets = blockscale_offsets;
    a.input_perm = input_permutation;
    a.input_perm_len = input_permutation_len;
    a.output_perm = output_permutation;
    a.workspace = static_cast<int32_t*>(workspace);
    return hip_status(mxmoe::launch_route(a, static_cast<hipStream_t>(stream)));
}

mx_status mx_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                          const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                          void* stream) {
    if (num_src_rows < 0 || num_dst_rows < 0 || row_bytes < 1 || row_bytes > kMaxRowBytes ||
        num_src_rows > kMax31 || num_dst_rows > kMax31)
        return MX_ERR_INVALID_ARGUMENT;
    if (num_dst_rows > 0 && (dst2src == nullptr || dst == nullptr ||
                             (num_src_rows > 0 && src == nullptr)))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(dst2src, 4)) return MX_ERR_MISALIGNED;
    if (num_dst_rows == 0) return MX_OK;
    return hip_status(mxmoe::launch_shuffle_rows(src, num_src_rows, row_bytes, dst2src,
                                                 num_dst_rows, dst,
                                                 static_cast<hipStream_t>(stream)));
}


mx_status mx_dispatch_rows(const void* src, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                           const int32_t* output_permutation, void* dst, int64_t num_dst_rows,
                           const void* side_src, int64_t side_row_bytes, void* side_dst,
                           void* stream) {
    return dispatch_rows(src, num_tokens, topk, row_bytes, output_permutation, dst, num_dst_rows,
                         side_src, side_row_bytes, side_dst, nullptr, nullptr, stream);
}

mx_status mx_dispatch_rows_timed(const void* src, int64_t num_tokens, int32_t topk,
                                 int64_t row_bytes, const int32_t* output_permutation, void* dst,
                                 int64_t num_dst_rows, const void* side_src,
                                 int64_t side_row_bytes, void* side_dst, void* start_event,
                                 void* stop_event, void* stream) {
    return dispatch_rows(src, num_tokens, topk, row_bytes, output_permutation, dst, num_dst_rows,
                         side_src, side_row_bytes, side_dst, start_event, stop_event, stream);
}

mx_status mx_apply_shuffle_mul_sum(const void* y, int32_t y_dtype, int64_t num_y_rows,
                                   int64_t hidden, const int32_t* permutation,
                                   const void* factors, int32_t factors_dtype,
                                   int64_t num_tokens, int32_t topk,
                                   void* out, int32_t out_dtype, void* stream) {
    return apply_shuffle_mul_sum(y, y_dtype, num_y_rows, hidden, permutation, factors,
                                 factors_dtype, num_tokens, topk, out, out_dtype, nullptr,
                                 nullptr, stream);
}

mx_status mx_apply_shuffle_mul_sum_timed(const void* y, int32_t y_dtype, int64_t num_y_rows,
                                         int64_t hidden, const int32_t* permutation,
                                         const void* factors, int32_t factors_dtype,
                                         int64_t num_tokens, int32_t topk, void* out,
                                         int32_t out_dtype, void* start_event, void* stop_event,
                                         void* stream) {
    return apply_shuffle_mul_sum(y, y_dtype, num_y_rows, hidden, permutation, factors,
                                 factors_dtype, num_tokens, topk, out, out_dtype, start_event,
                                 stop_event, stream);
}

mx_status mx_moe_output_memset(void* out, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                               const int32_t* output_permutation, void* stream) {
    if (num_tokens < 0 || topk < 1 || num_tokens > kMax31 / topk || row_bytes < 1 ||
        row_bytes > kMaxRowBytes)
        return MX_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && (out == nullptr || output_permutation == nullptr))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(output_permutation, 4)) return MX_ERR_MISALIGNED;
    if (num_tokens == 0) return MX_OK;
    return hip_status(mxmoe::launch_output_memset(out, num_tokens, topk, row_bytes,
                                                  output_permutation,
                                                  static_cast<hipStream_t>(stream)));
}

mx_status mx_zero_padding_rows(void* rows, int64_t num_rows, int64_t row_bytes,
                               const int32_t* input_permutation, const int32_t* expert_offsets,
                               int32_t num_experts, void* stream) {
    if (num_rows < 0 || num_rows > kMax31 || row_bytes < 1 || row_bytes > kMaxRowBytes)
        return MX_ERR_INVALID_ARGUMENT;
    if (expert_offsets != nullptr && (num_experts < 1 || num_experts > MX_MAX_EXPERTS))
        return MX_ERR_INVALID_ARGUMENT;
    if (num_rows > 0 && (rows == nullptr || input_permutation == nullptr))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(input_permutation, 4) || !aligned(expert_offsets, 4)) return MX_ERR_MISALIGNED;
    if (num_rows == 0) return MX_OK;
    return hip_status(mxmoe::launch_zero_padding(rows, num_rows, row_bytes, input_permutation,
                                                 expert_offsets, num_experts,
                                                 static_cast<hipStream_t>(stream)));
}

mx_status mx_moe_sort(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens, int32_t topk,
                      int32_t num_experts, int32_t local_expert_offset,
                      int32_t num_local_experts, int32_t tile_size,
                      int32_t* expanded_idx_to_permuted_idx,
                      int32_t* permuted_idx_to_expanded_idx, int64_t permuted_capacity,
                      int32_t* tile_idx_to_group_idx, int32_t* tile_idx_to_mn_limit,
                      int64_t max_tiles, int32_t* total_num_padded_tokens,
                      int32_t* num_non_exiting_tiles, int32_t* expert_offsets,
                      void* workspace, size_t workspace_bytes, void* stream) {
    if (ids_dtype != MX_I32 && ids_dtype != MX_I64) return MX_ERR_UNSUPPORTED_DTYPE;
    if (num_tokens < 0 || topk < 1 || num_experts < 1 || local_expert_offset < 0 ||
        num_local_experts < 1 || num_local_experts > MX_MAX_EXPERTS ||
        (int64_t)local_expert_offset + num_local_experts > num_experts || tile_size < 1)
        return MX_ERR_INVALID_ARGUMENT;
    const int64_t cap = mx_dispatch_capacity(num_tokens, topk, num_local_experts, tile_size);
    if (cap < 0) return MX_ERR_INVALID_ARGUMENT;
    const int64_t n = num_tokens * topk;
    if ((n > 0 && (topk_ids == nullptr || expanded_idx_to_permuted_idx == nullptr)) ||
        (permuted_capacity > 0 && permuted_idx_to_expanded_idx == nullptr) ||
        (max_tiles > 0 && (tile_idx_to_group_idx == nullptr || tile_idx_to_mn_limit == nullptr)) ||
        total_num_padded_tokens == nullptr || num_non_exiting_tiles == nullptr)
        return MX_ERR_INVALID_ARGUMENT;
    if (permuted_capacity < cap || max_tiles < (cap + tile_size - 1) / tile_size)
        return MX_ERR_CAPACITY;
    if (permuted_capacity > kMax31 || max_tiles > kMax31) return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(topk_ids, ids_dtype == MX_I64 ? 8 : 4) ||
        !aligned(expanded_idx_to_permuted_idx, 4) || !aligned(permuted_idx_to_expanded_idx, 4) ||
        !aligned(tile_idx_to_group_idx, 4) || !aligned(tile_idx_to_mn_limit, 4) ||
        !aligned(total_num_padded_tokens, 4) || !aligned(num_non_exiting_tiles, 4) ||
        !aligned(expert_offsets, 4) || !aligned(workspace, 4))
        return MX_ERR_MISALIGNED;
    const size_t need = mxmoe::route_workspace_bytes(n, num_local_experts);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return MX_ERR_WORKSPACE_TOO_SMALL;

    mxmoe::RouteArgs a{};
    a.ids = topk_ids;
    a.ids64 = ids_dtype == MX_I64;
    a.num_picks = n;
    a.topk = topk;
    a.num_experts = num_local_experts;
    a.row_align = tile_size;
    a.bs_align = 1;
    a.expert_offsets = expert_offsets;
    a.input_perm = permuted_idx_to_expanded_idx;
    a.input_perm_len = permuted_capacity;
    a.output_perm = expanded_idx_to_permuted_idx;
    a.workspace = static_cast<int32_t*>(workspace);
    a.id_offset = local_expert_offset;
    a.inp_expanded = true;
    a.tile_group = tile_idx_to_group_idx;
    a.tile_limit = tile_idx_to_mn_limit;
    a.max_tiles = max_tiles;
    a.padded_total = total_num_padded_tokens;
    a.tile_count = num_non_exiting_tiles;
    return hip_status(mxmoe::launch_route(a, static_cast<hipStream_t>(stream)));
}

mx_status mx_dispatch_rows_fp8(const void* src, int32_t src_dtype, int64_t num_tokens,
                               int32_t topk, int64_t hidden, const int32_t* output_permutation,
                               void* dst_q, float* dst_scales, int64_t num_dst_rows,
                               void* stream) {
    if (src_dtype != MX_BF16) return MX_ERR_UNSUPPORTED_DTYPE;
    if (num_tokens < 0 || topk < 1 || num_tokens > kMax31 / topk || hidden < 128 ||
        hidden % 128 != 0 || hidden > (int64_t)65535 * 1024 * 8 || num_dst_rows < 0 ||
        num_dst_rows > kMax31)
        return MX_ERR_INVALID_ARGUMENT;
    if (num_tokens > 0 && (src == nullptr || output_permutation == nullptr ||
                           (num_dst_rows > 0 && (dst_q == nullptr || dst_scales == nullptr))))
        return MX_ERR_INVALID_ARGUMENT;
    if (!aligned(src, 16) || !aligned(dst_q, 16) || !aligned(dst_scales, 4) ||
        !aligned(output_permutation, 4))
        return MX_ERR_MISALIGNED;
    if (num_tokens == 0 || num_dst_rows == 0) return MX_OK;
    return hip_status(mxmoe::launch_dispatch_quant_fp8(src, num_tokens, topk, hidden,
                                                       output_permutation, dst_q, dst_scales,
                                                       num_dst_rows,
                                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
