/*
 * mxmoe -- MoE token dispatch and combine on one AMD MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels for the three host calls the sglang
 * page "[jit_kernel] Add prepare_moe_input JIT kernels" (section "Changes")
 * describes: prepare_moe_input builds routing metadata from top-k expert ids,
 * shuffle_rows gathers rows byte for byte, apply_shuffle_mul_sum gathers,
 * scales by the top-k weight and sums with fp32 accumulation.  A token-major
 * scatter form of the row gather (mx_dispatch_rows) is added because it
 * reads every token row once.
 *
 * Conventions shared by every call
 *   - Every array argument is a DEVICE pointer to memory the caller owns,
 *     laid out row-major and contiguous.  The library allocates and frees
 *     nothing, keeps no state between calls and never synchronises.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and launched on the current HIP device, which must own the stream and
 *     the arrays.  Outputs are written in place when the stream reaches the
 *     work.
 *   - Argument errors (null pointers, sizes out of range, unsupported dtypes,
 *     misaligned index arrays, short buffers) are detected on the host before
 *     any HIP call and returned as a status; nothing is enqueued then.  After
 *     each launch the HIP launch error is checked and reported as
 *     MX_ERR_HIP (mx_last_hip_error() gives the hipError_t value).
 *   - Index data is never trusted: ids outside [0, E) are dropped, row
 *     indices outside the given row counts are skipped.  No index value can
 *     make a kernel access memory outside the arrays described here.
 *   - Rows and picks are indexed with 32-bit integers: T*k, row capacities
 *     and row counts must stay below 2^31.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
    MX_OK = 0,
    MX_ERR_INVALID_ARGUMENT = 1,  /* null pointer, size out of range            */
    MX_ERR_UNSUPPORTED_DTYPE = 2, /* dtype not accepted by this call            */
    MX_ERR_MISALIGNED = 3,        /* pointer not aligned to its element size    */
    MX_ERR_WORKSPACE_TOO_SMALL = 4,
    MX_ERR_CAPACITY = 5,          /* input_permutation shorter than capacity    */
    MX_ERR_HIP = 6,               /* a HIP launch failed                        */
    MX_ERR_OUT_OF_BOUNDS = 7,     /* bounds-checked library only: a kernel
                                     access fell outside the call's arrays
                                     (see mx_bounds_checked)                   */
    /* widens the enum's value range to every non-negative 32-bit code, so
     * mx_status_string is defined for any code a caller passes */
    MX_STATUS_FORCE_INT32 = 0x7fffffff
} mx_status;

typedef enum mx_dtype {
    MX_F32 = 0,
    MX_F16 = 1,
    MX_BF16 = 2,
    MX_FP8_E4M3 = 3, /* OCP e4m3fn bytes; only as opaque row bytes          */
    MX_I32 = 4,
    MX_I64 = 5
} mx_dtype;

/* Largest expert count prepare_moe_input accepts. */
#define MX_MAX_EXPERTS 1024

/* Device scratch each GPU holds for mx_prepare_moe_input_noalloc: the
 * largest routing workspace any accepted size needs (at most 128 tiles x
 * MX_MAX_EXPERTS counts of 4 bytes). */
#define MX_NOALLOC_SCRATCH_BYTES (512 * 1024)

/* Text for a status code (static storage). */
const char* mx_status_string(mx_status status);

/* hipError_t of the last launch that returned MX_ERR_HIP on this thread. */
int mx_last_hip_error(void);

/*
 * Bounds-checked build.  The same sources built with MXMOE_CHECKED defined
 * give libmxmoe_checked.so, a debugging library with every entry point of
 * this header.  Each call there describes its arrays to its kernels (the
 * extents stated for each call below), and every global load and store of
 * the kernels is checked against them before it is made: an access that does
 * not lie wholly inside one array, or a store into an input, is counted and
 * skipped (a load yields zeros), so the kernel still ends normally, and the
 * call returns MX_ERR_OUT_OF_BOUNDS.  Indices into the kernels' on-chip
 * arrays that come from data are checked the same way.  Every call of the
 * checked library synchronises the device before and after its work and
 * serialises with other calls; under stream capture it returns MX_ERR_HIP
 * (hipErrorStreamCaptureUnsupported) and enqueues nothing.  libmxmoe.so
 * checks nothing and never returns MX_ERR_OUT_OF_BOUNDS.
 *
 * A second test build, libmxmoe_altgrid.so, has other tile sizes, path
 * limits and workgroup widths: the one-launch thresholds and workspace sizes
 * stated below are those of libmxmoe.so and differ there (ask
 * mx_prepare_workspace_size of the library in use), while every result is
 * the same bits.
 */

/* 1 in the bounds-checked library, 0 in libmxmoe.so. */
int32_t mx_bounds_checked(void);

/*
 * Out-of-bounds accesses counted since the last clear:
 *   report[0] loads, report[1] stores (and data-dependent on-chip indices),
 *   report[2] the byte address (or the index) of the first one counted,
 *   report[3] a code naming the access that made it (0: none), one of the
 *             CheckSite values of the library's sources.
 * report: host array of 4 (else MX_ERR_INVALID_ARGUMENT); clear != 0 resets
 * the counts after reading.  All zero in libmxmoe.so.
 */
mx_status mx_bounds_report(uint64_t* report, int32_t clear);

/*
 * Testing the checks themselves: from the next call on, every array a call
 * writes is described to its kernels as `bytes` shorter at its end than it
 * is (0 restores the true extents), so a kernel that writes the last bytes of
 * an output is caught and skipped while no access leaves the real arrays.
 * bytes >= 0 (else MX_ERR_INVALID_ARGUMENT).  libmxmoe.so accepts only 0.
 */
mx_status mx_bounds_shrink_outputs(int64_t bytes);

/*
 * Rows a dispatched buffer (and input_permutation) needs for ANY routing of
 * T tokens x k picks over E experts with segments padded to row_align:
 * T*k + E*(row_align - 1).  Returns -1 when an argument is out of range or
 * the result does not fit in 31 bits.  Host-only arithmetic.
 */
int64_t mx_dispatch_capacity(int64_t num_tokens, int32_t topk, int32_t num_experts,
                             int32_t row_align);

/* Bytes of device workspace mx_prepare_moe_input needs for these sizes
 * (0 when the arguments are out of range).  Host-only arithmetic. */
size_t mx_prepare_workspace_size(int64_t num_tokens, int32_t topk, int32_t num_experts);

/*
 * prepare_moe_input -- routing metadata (sglang prepare_moe_input page,
 * "Changes" item 1: compute_problem_sizes counts tokens per expert,
 * compute_expert_offsets takes the prefix sum, compute_expert_blockscale_
 * offsets gives the optional FP8 block-scale offsets, compute_arg_sorts
 * builds the input and output permutations).
 *
 * Picks are flattened i = t*k + j.  A pick is valid iff 0 <= id < E; with
 * count_e the number of valid picks of expert e:
 *
 *   expert_offsets[0] = 0,
 *   expert_offsets[e+1] = expert_offsets[e] + ceil(count_e / row_align) * row_align
 *   problem_sizes1[e] = {count_e, gemm1_n, gemm1_k}
 *   problem_sizes2[e] = {count_e, gemm2_n, gemm2_k}
 *   blockscale_offsets: the same running sum with blockscale_align in place
 *                       of row_align
 *   output_permutation[i] = dispatched row of pick i (-1 if the pick is dropped)
 *   input_permutation[r]  = source token (i / k) of dispatched row r, -1 for
 *                           padding rows and for rows past the last segment
 *
 * Rows of one expert hold its picks in ascending i (a stable counting sort),
 * so the result is deterministic and independent of launch shapes.
 *
 * topk_ids            [T, k] MX_I32 or MX_I64 (ids_dtype), 4- / 8-byte aligned
 * num_tokens (T) >= 0, topk (k) >= 1, 1 <= num_experts (E) <= MX_MAX_EXPERTS
 * row_align >= 1      1 = plain prefix sum; e.g. 128 pads each segment for a
 *                     grouped GEMM tile
 * expert_offsets      out [E+1] int32
 * problem_sizes1/2    out [E][3] int32, or NULL to skip
 * input_permutation   out [input_permutation_len] int32; every entry is
 *                     written.  input_permutation_len must be at least
 *                     mx_dispatch_capacity(T, k, E, row_align), else
 *                     MX_ERR_CAPACITY.
 * output_permutation  out [T*k] int32
 * blockscale_offsets  out [E+1] int32, or NULL to skip; blockscale_align >= 1
 *                     (128 for 1x128 FP8 block scales) when given
 * workspace           device scratch of at least
 *                     mx_prepare_workspace_size(T, k, E) bytes, 16-byte
 *                     aligned (else MX_ERR_MISALIGNED: the kernels read it
 *                     with 16-byte loads); contents on entry do not matter
 */
mx_status mx_prepare_moe_input(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens,
                               int32_t topk, int32_t num_experts,
                               int32_t gemm1_n, int32_t gemm1_k, int32_t gemm2_n, int32_t gemm2_k,
                               int32_t row_align,
                               int32_t* expert_offsets, int32_t* problem_sizes1,
                               int32_t* problem_sizes2,
                               int32_t* input_permutation, int64_t input_permutation_len,
                               int32_t* output_permutation,
                               int32_t* blockscale_offsets, int32_t blockscale_align,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * prepare_moe_input for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments, checks, work and results as
 * mx_prepare_moe_input, without the workspace.  The routing count table
 * lives in a device array of MX_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU until the process ends; its address is looked up at the first
 * call on a device (hipGetSymbolAddress, with that device current).  The
 * call allocates and frees nothing.  Sizes whose workspace would exceed the
 * array return MX_ERR_WORKSPACE_TOO_SMALL (no size this call accepts does).
 * The kernels write the whole table before reading it, so nothing needs to
 * be cleared between calls.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams, or from different
 * threads without ordering) race and give undefined results; calls ordered
 * on one stream are safe.
 */
mx_status mx_prepare_moe_input_noalloc(const void* topk_ids, int32_t ids_dtype,
                                       int64_t num_tokens, int32_t topk, int32_t num_experts,
                                       int32_t gemm1_n, int32_t gemm1_k, int32_t gemm2_n,
                                       int32_t gemm2_k, int32_t row_align,
                                       int32_t* expert_offsets, int32_t* problem_sizes1,
                                       int32_t* problem_sizes2, int32_t* input_permutation,
                                       int64_t input_permutation_len,
                                       int32_t* output_permutation, int32_t* blockscale_offsets,
                                       int32_t blockscale_align, void* stream);

/*
 * Timed form of mx_prepare_moe_input: the same arguments, checks, work and
 * results, plus start_event / stop_event (hipEvent_t created by the caller,
 * or NULL), recorded with the begin of the first routing kernel and the end
 * of the last one from the kernel dispatches' own timestamps (see the timed
 * forms of dispatch and combine below).
 */
mx_status mx_prepare_moe_input_timed(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens,
                                     int32_t topk, int32_t num_experts, int32_t gemm1_n,
                                     int32_t gemm1_k, int32_t gemm2_n, int32_t gemm2_k,
                                     int32_t row_align, int32_t* expert_offsets,
                                     int32_t* problem_sizes1, int32_t* problem_sizes2,
                                     int32_t* input_permutation, int64_t input_permutation_len,
                                     int32_t* output_permutation, int32_t* blockscale_offsets,
                                     int32_t blockscale_align, void* workspace,
                                     size_t workspace_bytes, void* start_event, void* stop_event,
                                     void* stream);

/*
 * prepare_dispatch -- prepare_moe_input followed by dispatch_rows (below) on
 * the same stream, in one call: the routing of the sglang page's "Changes"
 * item 1 and the rows of its item 2 (dst[output_permutation[t*k+j]] = src[t]).
 * The first twenty arguments are those of mx_prepare_moe_input, with the
 * same meaning, layout and checks; src, row_bytes, dst, num_dst_rows,
 * side_src, side_row_bytes and side_dst are those of mx_dispatch_rows.  The
 * results are bit-identical to the two calls.  Every argument of both is
 * checked before anything is launched, so an error status means nothing
 * was enqueued.
 *
 * Inputs that prepare_moe_input routes in one workgroup (up to 1024 picks,
 * or 2048 when input_permutation_len <= 2*T*k), with row_bytes and both row
 * bases multiples of 16, no side rows and at most 512 workgroups of 512
 * 16-byte vectors, run as one launch: every workgroup routes all picks
 * itself and copies its chunk of one token row, and the first also writes
 * the metadata.  This saves a launch and a dependent trip through memory at
 * decode-sized batches.  Other inputs run the kernels of the two calls.
 * Caller-owned memory as in both calls; nothing is allocated or freed.
 */
mx_status mx_prepare_dispatch(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens,
                              int32_t topk, int32_t num_experts, int32_t gemm1_n,
                              int32_t gemm1_k, int32_t gemm2_n, int32_t gemm2_k,
                              int32_t row_align, int32_t* expert_offsets,
                              int32_t* problem_sizes1, int32_t* problem_sizes2,
                              int32_t* input_permutation, int64_t input_permutation_len,
                              int32_t* output_permutation, int32_t* blockscale_offsets,
                              int32_t blockscale_align, void* workspace, size_t workspace_bytes,
                              const void* src, int64_t row_bytes, void* dst,
                              int64_t num_dst_rows, const void* side_src,
                              int64_t side_row_bytes, void* side_dst, void* stream);

/*
 * shuffle_rows -- dtype-agnostic row gather (sglang page, "Changes" item 2):
 *
 *   dst[r] = src[dst2src[r]]   (row_bytes bytes) for r < num_dst_rows
 *
 * Rows with dst2src[r] outside [0, num_src_rows) are left untouched.
 * src [num_src_rows, row_bytes], dst [num_dst_rows, row_bytes], any element
 * type; dst2src [num_dst_rows] int32 (e.g. input_permutation).
 * 1 <= row_bytes <= 65535 * 1024.
 * Copies use 16-byte accesses when row_bytes and both base pointers are
 * multiples of 16, else the widest width that divides all three.
 */
mx_status mx_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                          const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                          void* stream);

/*
 * dispatch_rows -- the same rows as shuffle_rows(src, input_permutation),
 * produced token by token so each source row is read once:
 *
 *   dst[output_permutation[t*k + j]] = src[t]   for t < T, j < k
 *
 * Destinations outside [0, num_dst_rows) are skipped.  Optionally a second
 * "side" row per token (e.g. the fp32 1x128 block scales of an FP8 row) is
 * copied the same way: side_dst[output_permutation[t*k+j]] = side_src[t]
 * (pass side_src = side_dst = NULL and side_row_bytes = 0 to skip).
 * src [T, row_bytes], dst [num_dst_rows, row_bytes], side arrays
 * [*, side_row_bytes]; output_permutation [T*k] int32;
 * 1 <= row_bytes <= 65535 * 1024.
 */
mx_status mx_dispatch_rows(const void* src, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                           const int32_t* output_permutation, void* dst, int64_t num_dst_rows,
                           const void* side_src, int64_t side_row_bytes, void* side_dst,
                           void* stream);

/*
 * dispatch_rows_fp8 -- dispatch with FP8 quantization fused in: every token
 * row is quantized in 1 x 128 groups to OCP e4m3fn codes with one fp32 scale
 * per group (the input quantization the TensorRT-LLM page "Enable CuteDSL
 * MoE with Large EP" performs before its MoE; the 1 x 128 block scales of
 * the sglang page's FP8 path), and the codes and scales go to the token's k
 * dispatched rows:
 *
 *   per group G of 128 elements of src[t]:
 *     amax  = max |x|,  scale = amax / 448 (1 when amax == 0)
 *     code  = e4m3fn(x / scale), round to nearest even, saturate at 448
 *   dst_q[output_permutation[t*k+j]][h]      = code(src[t][h])
 *   dst_scales[output_permutation[t*k+j]][G] = scale(G)
 *
 * fp32 arithmetic with IEEE division.  Non-finite inputs: amax skips NaN
 * and a NaN codes to 0x7f; an infinity makes its group's scale infinite, so
 * the group's finite values code to signed zero and its infinities to 0x7f.
 * Destinations outside [0, num_dst_rows) are skipped.  src [T, hidden]
 * MX_BF16, 16-byte aligned; dst_q [num_dst_rows, hidden] bytes, 16-byte
 * aligned; dst_scales [num_dst_rows, hidden / 128] fp32; hidden a multiple
 * of 128.
 */
mx_status mx_dispatch_rows_fp8(const void* src, int32_t src_dtype, int64_t num_tokens,
                               int32_t topk, int64_t hidden, const int32_t* output_permutation,
                               void* dst_q, float* dst_scales, int64_t num_dst_rows,
                               void* stream);

/*
 * apply_shuffle_mul_sum -- gather, scale, reduce (sglang page, "Changes"
 * item 3: FP32 accumulation, fp16 / bf16 / fp32):
 *
 *   out[t][h] = round_out( sum_{j=0..k-1} f[t][j] * y[permutation[t*k+j]][h] )
 *
 * The sum runs in fp32 in ascending j, each step one fused multiply-add
 * starting from +0; round_out rounds to nearest even (identity for fp32).
 * Picks whose row is outside [0, num_y_rows) contribute nothing.
 *
 * y           [num_y_rows, hidden], y_dtype MX_F32 / MX_F16 / MX_BF16
 * permutation [T*k] int32 (output_permutation of prepare_moe_input)
 * factors     [T, k] in MX_F32, MX_F16 or MX_BF16 (factors_dtype), or NULL
 *             for unit weights
 * out         [T, hidden], out_dtype MX_F32 / MX_F16 / MX_BF16
 * Pointers must be aligned to their element size.
 */
mx_status mx_apply_shuffle_mul_sum(const void* y, int32_t y_dtype, int64_t num_y_rows,
                                   int64_t hidden, const int32_t* permutation,
                                   const void* factors, int32_t factors_dtype,
                                   int64_t num_tokens, int32_t topk,
                                   void* out, int32_t out_dtype, void* stream);

/*
 * Timed forms of mx_dispatch_rows and mx_apply_shuffle_mul_sum, for
 * measuring the two row kernels with the backend's own timing (the benchmark
 * page "[RFC]: Comprehensive MoE / EP Kernel Benchmark Under Incast
 * Traffic", section "Timing Method", puts backend-specific timing behind
 * helpers).  Same arguments, checks, work and results as the plain calls,
 * plus two events:
 *
 * start_event, stop_event   hipEvent_t handles created by the caller (for
 *                           example with hipEventCreate), or NULL.  The call
 *                           records start_event with the begin of its first
 *                           kernel and stop_event with the end of its last,
 *                           from the kernel dispatch's own timestamps
 *                           (hipExtLaunchKernel), so hipEventElapsedTime
 *                           between them is the kernels' execution time
 *                           without the gap an event record queued on the
 *                           stream between launches adds.  A call that
 *                           launches nothing (no tokens, or no rows)
 *                           records neither event.
 */
mx_status mx_dispatch_rows_timed(const void* src, int64_t num_tokens, int32_t topk,
                                 int64_t row_bytes, const int32_t* output_permutation, void* dst,
                                 int64_t num_dst_rows, const void* side_src,
                                 int64_t side_row_bytes, void* side_dst, void* start_event,
                                 void* stop_event, void* stream);

mx_status mx_apply_shuffle_mul_sum_timed(const void* y, int32_t y_dtype, int64_t num_y_rows,
                                         int64_t hidden, const int32_t* permutation,
                                         const void* factors, int32_t factors_dtype,
                                         int64_t num_tokens, int32_t topk, void* out,
                                         int32_t out_dtype, void* start_event, void* stop_event,
                                         void* stream);

/*
 * moe_sort -- tile-padded sort metadata for one rank's window of experts
 * (the TensorRT-LLM page "Enable CuteDSL MoE with Large EP": the sort that
 * returns tile_idx_to_group_idx, tile_idx_to_mn_limit,
 * expanded_idx_to_permuted_idx, permuted_idx_to_expanded_idx,
 * total_num_padded_tokens and num_non_exiting_tiles for a grouped GEMM over
 * num_local_experts experts starting at local_expert_offset, in tiles of
 * tile_size rows).
 *
 * Pick i = t*k + j is local iff local_expert_offset <= id <
 * local_expert_offset + num_local_experts; its group is g = id -
 * local_expert_offset.  Local picks are sorted stably by group (ascending i
 * within a group); group g takes ceil(count_g / tile_size) whole tiles,
 * groups in order from row 0.
 *
 *   expanded_idx_to_permuted_idx[i] = row of pick i, -1 if not local
 *   permuted_idx_to_expanded_idx[r] = pick i held by row r, -1 for padding
 *                                     rows and rows past the last group
 *   tile_idx_to_group_idx[q]        = group of tile q, -1 past the last group
 *   tile_idx_to_mn_limit[q]         = first row of that group + count_g (end of
 *                                     the group's valid rows), -1 past the last
 *   total_num_padded_tokens[0]      = sum_g ceil(count_g / tile_size) * tile_size
 *   num_non_exiting_tiles[0]        = total_num_padded_tokens / tile_size
 *   expert_offsets[g] (optional)    = first row of group g, [num_local_experts+1]
 *
 * permuted_capacity >= mx_dispatch_capacity(T, k, num_local_experts,
 * tile_size) and max_tiles >= ceil(that capacity / tile_size), else
 * MX_ERR_CAPACITY; every entry of both arrays is written.  0 <=
 * local_expert_offset, local_expert_offset + num_local_experts <=
 * num_experts, num_local_experts <= MX_MAX_EXPERTS, tile_size >= 1.
 * workspace: mx_prepare_workspace_size(T, k, num_local_experts) bytes,
 * 16-byte aligned.
 */
mx_status mx_moe_sort(const void* topk_ids, int32_t ids_dtype, int64_t num_tokens, int32_t topk,
                      int32_t num_experts, int32_t local_expert_offset,
                      int32_t num_local_experts, int32_t tile_size,
                      int32_t* expanded_idx_to_permuted_idx,
                      int32_t* permuted_idx_to_expanded_idx, int64_t permuted_capacity,
                      int32_t* tile_idx_to_group_idx, int32_t* tile_idx_to_mn_limit,
                      int64_t max_tiles, int32_t* total_num_padded_tokens,
                      int32_t* num_non_exiting_tiles, int32_t* expert_offsets,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_output_memset -- zero in place the output rows of the tokens that
 * receive expert results (the TensorRT-LLM page "Enable CuteDSL MoE with
 * Large EP", walkthrough and its in-place memset test: rows whose token has
 * a permuted index >= 0 become zero, the others are left untouched):
 *
 *   out[t] = 0 (row_bytes zero bytes)  iff  exists j: output_permutation[t*k+j] >= 0
 *
 * out [T, row_bytes] any element type; output_permutation [T*k] int32.
 * 1 <= row_bytes <= 65535 * 1024.
 */
mx_status mx_moe_output_memset(void* out, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                               const int32_t* output_permutation, void* stream);

/*
 * zero_padding_rows -- zero-fill the padding rows of a dispatched buffer, so
 * a grouped GEMM that reads whole row_align tiles reads zeros there:
 *
 *   rows[r] = 0  iff  r < limit and input_permutation[r] < 0
 *
 * limit = expert_offsets[num_experts] (the padded total, read on the device)
 * when expert_offsets is given, else num_rows; rows at or past it (unused
 * capacity) are left untouched.  With expert_offsets (the offsets
 * prepare_moe_input wrote: monotone, starting at 0) the work is spread per
 * expert segment; segment bounds are clipped to [0, num_rows), so other
 * offset values cannot cause accesses outside the arrays.  rows [num_rows,
 * row_bytes]; input_permutation [num_rows] int32 (from prepare_moe_input).
 * 1 <= row_bytes <= 65535 * 1024.
 */
mx_status mx_zero_padding_rows(void* rows, int64_t num_rows, int64_t row_bytes,
                               const int32_t* input_permutation, const int32_t* expert_offsets,
                               int32_t num_experts, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
