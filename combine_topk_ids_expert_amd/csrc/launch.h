// Internal launcher interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mxmoe {

struct RouteArgs {
    const void* ids;
    bool ids64;
    int64_t num_picks;        // T * k
    int32_t topk;
    int32_t num_experts;
    int32_t row_align;
    int32_t bs_align;
    int32_t gemm[4];          // gemm1_n, gemm1_k, gemm2_n, gemm2_k
    int32_t* expert_offsets;  // [E+1]
    int32_t* problem_sizes1;  // [E][3] or null
    int32_t* problem_sizes2;  // [E][3] or null
    int32_t* blockscale_offsets;  // [E+1] or null
    int32_t* input_perm;      // [input_perm_len]
    int64_t input_perm_len;
    int32_t* output_perm;     // [T*k]
    int32_t* workspace;
    // Local-expert window and tile metadata (zero / null for prepare_moe_input):
    int32_t id_offset;        // subtracted from every id; valid iff 0 <= id - offset < E
    bool inp_expanded;        // input_perm holds the pick index i instead of the token i / k
    int32_t* tile_group;      // [max_tiles] tile -> expert of its segment, -1 unused
    int32_t* tile_limit;      // [max_tiles] tile -> first row + count of its expert, -1 unused
    int64_t max_tiles;        // tiles are row_align rows
    int32_t* padded_total;    // [1] padded row total, or null
    int32_t* tile_count;      // [1] padded row total / row_align, or null
};

// Device workspace the routing kernels need for `num_picks` picks.
size_t route_workspace_bytes(int64_t num_picks, int32_t num_experts);
// Whether routing and the row dispatch of `num_tokens` rows of `row_bytes`
// can run as one launch (launch_route_dispatch): inputs the single-workgroup
// routing takes, 16-byte row widths and bases, a bounded grid.
bool route_dispatch_fusable(const RouteArgs& a, int64_t num_tokens, int64_t row_bytes,
                            const void* src, const void* dst);
// Routing metadata of `a` plus dst[output_perm[t*k+j]] = src[t] in one launch;
// only for arguments route_dispatch_fusable accepts.
hipError_t launch_route_dispatch(const RouteArgs& a, int64_t num_tokens, const void* src,
                                 int64_t row_bytes, void* dst, int64_t num_dst_rows,
                                 hipStream_t stream);
// start_event / stop_event (either may be null) are recorded with the begin
// of the first routing kernel and the end of the last one.
hipError_t launch_route(const RouteArgs& a, hipStream_t stream, hipEvent_t start_event = nullptr,
                        hipEvent_t stop_event = nullptr);

hipError_t launch_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                               const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                               hipStream_t stream);

// start_event / stop_event (either may be null) are recorded with the begin
// of the call's first kernel and the end of its last one.
hipError_t launch_dispatch_rows(const void* src, int64_t num_tokens, int32_t topk,
                                int64_t row_bytes, const int32_t* output_perm, void* dst,
                                int64_t num_dst_rows, const void* side_src,
                                int64_t side_row_bytes, void* side_dst, hipStream_t stream,
                                hipEvent_t start_event, hipEvent_t stop_event);

// dtype codes as in mxmoe.h (MX_F32 = 0, MX_F16 = 1, MX_BF16 = 2); factors_dtype
// is ignored when factors is null.
hipError_t launch_combine(const void* y, int y_dtype, int64_t num_y_rows, int64_t hidden,
                          const int32_t* perm, const void* factors, int factors_dtype,
                          int64_t num_tokens, int32_t topk, void* out, int out_dtype,
                          hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event);

hipError_t launch_zero_padding(void* rows, int64_t num_rows, int64_t row_bytes,
                               const int32_t* input_perm, const int32_t* expert_offsets,
                               int32_t num_experts, hipStream_t stream);

hipError_t launch_output_memset(void* out, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                                const int32_t* expanded_to_permuted, hipStream_t stream);

hipError_t launch_dispatch_quant_fp8(const void* src, int64_t num_tokens, int32_t topk,
                                     int64_t hidden, const int32_t* output_perm, void* dst_q,
                                     float* dst_scales, int64_t num_dst_rows,
                                     hipStream_t stream);

}  // namespace mxmoe
