// Zeroing rows in place: the MoE output memset (the TensorRT-LLM page
// "Enable CuteDSL MoE with Large EP", walkthrough: zero the output row of
// every token that has a valid permuted index, leave the others) and the
// zero-fill of the padding rows of a dispatched buffer, for grouped GEMMs
// that read whole tiles.
//
// The memset has the shape of the row copies: a workgroup per row and column
// chunk, one 16-byte (or narrower) non-temporal store per thread; whether a
// row is zeroed is decided once per workgroup from the index data.  The
// padding fill works per expert segment (see zero_padding_expert_kernel).
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

#ifndef MXMOE_ZERO_THREADS
#define MXMOE_ZERO_THREADS 128
#endif
constexpr int kZeroThreads = MXMOE_ZERO_THREADS;   // workgroup width (longer rows are cut into column chunks)
static_assert(kZeroThreads % kWave == 0 && kZeroThreads <= 1024, "whole waves, at most 1024");

// LDS reserved per workgroup of the per-segment padding fill: at most 10 of
// its two-wave workgroups per CU instead of 16.  At T = 4096 (event times on
// MI355X) it filled the padding in 35.5 us, against 37.9 us uncapped, 36.0 us
// at 8 per CU, 35.8 at 12 and 37.8 at 16.  The output memset keeps no cap:
// capped at 8 or 6 per CU it was slower (15.1 and 20.1 us against 12.4).
constexpr size_t kZeroPaddingLds = 16 * 1024;


template <int V> struct ZVec;
template <> struct ZVec<16> { using T = u32x4; };
template <> struct ZVec<8> { using T = u32x2; };
template <> struct ZVec<4> { using T = uint32_t; };
template <> struct ZVec<2> { using T = uint16_t; };
template <> struct ZVec<1> { using T = uint8_t; };

template <int V>
__device__ __forceinline__ void zero_vector(uint8_t* row, int64_t c, int64_t nvec) {
    using T = typename ZVec<V>::T;
    if (c < nvec && MX_CAN_STORE(reinterpret_cast<T*>(row) + c, sizeof(T), kSiteZeroRows))
        __builtin_nontemporal_store(T{}, reinterpret_cast<T*>(row) + c);
}

// Without expert offsets: row r is zeroed iff its source index is negative
// (every row of the buffer is considered); one workgroup per row and column
// chunk.
template <int V>
__global__ __launch_bounds__(kZeroThreads) void zero_padding_kernel(
    uint8_t* __restrict__ rows, int64_t row_bytes, const int32_t* __restrict__ input_perm,
    int32_t chunks) {
    int64_t chunk;
    const int64_t r = chunk_row(chunks, chunk);
    if (!MX_CAN_LOAD(input_perm + r, 4, kSiteZeroIndex) || input_perm[r] >= 0) return;
    zero_vector<V>(rows + r * row_bytes, chunk * blockDim.x + threadIdx.x, row_bytes / V);
}

// With expert offsets only the rows inside the expert segments are
// considered: workgroup (e, s, c) takes every kSlices-th row of segment e
// [expert_offsets[e], expert_offsets[e+1]) from row seg0 + s, reads 64 of
// their source indices per ballot, and zeroes column chunk c of exactly the
// rows whose index is negative.  A segment holds at most row_align - 1
// padding rows, so the grid is E x kSlices x chunks workgroups instead of
// one per row of capacity.  Segment bounds are clipped to [0, num_rows).
// 32 slices with 128-thread chunks measured best on MI355X: at T = 4096,
// H = 7168 with 128-row padding 39.7 us against 46.5 us for 16 slices of
// whole-row workgroups; 64 slices took 36.6 us there, but 29.7 us instead of
// 17.2 us for a call with nothing to zero, where every workgroup only scans.
#ifndef MXMOE_ZERO_SLICES
#define MXMOE_ZERO_SLICES 32
#endif
constexpr int kSlices = MXMOE_ZERO_SLICES;

// es0: index of the launch's first (expert, slice) pair, e * kSlices + s.
template <int V>
__global__ __launch_bounds__(kZeroThreads) void zero_padding_expert_kernel(
    uint8_t* __restrict__ rows, int64_t num_rows, int64_t row_bytes,
    const int32_t* __restrict__ input_perm, const int32_t* __restrict__ expert_offsets,
    int64_t es0, int32_t chunks) {
    int64_t chunk;
    const int64_t es = es0 + chunk_row(chunks, chunk);
    const int e = (int)(es / kSlices);
    const int slice = (int)(es - (int64_t)e * kSlices);
    const int lane = threadIdx.x & (kWave - 1);
    const bool seg_ok = MX_CAN_LOAD(expert_offsets + e, 8, kSiteZeroIndex);
    int64_t seg0 = seg_ok ? expert_offsets[e] : 0;
    int64_t seg1 = seg_ok ? expert_offsets[e + 1] : 0;
    if (seg0 < 0) seg0 = 0;
    if (seg1 > num_rows) seg1 = num_rows;
    const int64_t nvec = row_bytes / V;
    const int64_t c = chunk * blockDim.x + threadIdx.x;
    for (int64_t base = seg0 + slice; base < seg1; base += (int64_t)kSlices * kWave) {
        const int64_t r = base + (int64_t)lane * kSlices;
        const bool pad =
            r < seg1 && MX_CAN_LOAD(input_perm + r, 4, kSiteZeroIndex) && input_perm[r] < 0;
        uint64_t m = __ballot(pad);                    // wave-uniform from here on
        while (m != 0ull) {
            const int l = __builtin_ctzll(m);
            m &= m - 1;
            zero_vector<V>(rows + (base + (int64_t)l * kSlices) * row_bytes, c, nvec);
        }
    }
}

// Output row t is zeroed iff one of its topk picks has a permuted index
// >= 0; one workgroup per row and column chunk.
template <int V>
__global__ __launch_bounds__(kZeroThreads) void output_memset_kernel(
    uint8_t* __restrict__ out, int64_t row_bytes, int32_t topk,
    const int32_t* __restrict__ expanded_to_permuted, int32_t chunks) {
    int64_t chunk;
    const int64_t t = chunk_row(chunks, chunk);
    const int lane = threadIdx.x & (kWave - 1);
    bool any = false;
    for (int j0 = 0; j0 < topk; j0 += kWave) {       // wave-uniform
        const int j = j0 + lane;
        const bool valid = j < topk &&
                           MX_CAN_LOAD(expanded_to_permuted + t * topk + j, 4, kSiteZeroIndex) &&
                           expanded_to_permuted[t * topk + j] >= 0;
        any = any || __ballot(valid) != 0ull;
    }
    if (!any) return;
    zero_vector<V>(out + t * row_bytes, chunk * blockDim.x + threadIdx.x, row_bytes / V);
}

int zvec_width(int64_t row_bytes, const void* p) {
    const uint64_t bits = (uint64_t)row_bytes | (uint64_t)(uintptr_t)p;
    for (int v = 16; v > 1; v >>= 1)
        if ((bits & (uint64_t)(v - 1)) == 0) return v;
    return 1;
}


}  // namespace

hipError_t launch_zero_padding(void* rows, int64_t num_rows, int64_t row_bytes,
                               const int32_t* input_perm, const int32_t* expert_offsets,
                               int32_t num_experts, hipStream_t stream) {
    if (num_rows == 0) return hipSuccess;
    const int v = zvec_width(row_bytes, rows);
    uint8_t* p = static_cast<uint8_t*>(rows);
    const RowShape sh = row_shape(row_bytes / v, kZeroThreads);
    if (expert_offsets != nullptr) {
        // (expert, slice) pairs take the place of rows in the launch shape.
        const int64_t pairs = (int64_t)num_experts * kSlices;
        const int32_t* eo = expert_offsets;
        return for_row_batches(pairs, sh, [&](int64_t es0, int64_t, dim3 grid, dim3 block,
                                              hipEvent_t e0, hipEvent_t e1) {
            switch (v) {
            case 16: launch_kernel(zero_padding_expert_kernel<16>, grid, block, kZeroPaddingLds, stream, e0, e1, p, num_rows, row_bytes, input_perm, eo, es0, sh.chunks); break;
            case 8: launch_kernel(zero_padding_expert_kernel<8>, grid, block, kZeroPaddingLds, stream, e0, e1, p, num_rows, row_bytes, input_perm, eo, es0, sh.chunks); break;
            case 4: launch_kernel(zero_padding_expert_kernel<4>, grid, block, kZeroPaddingLds, stream, e0, e1, p, num_rows, row_bytes, input_perm, eo, es0, sh.chunks); break;
            case 2: launch_kernel(zero_padding_expert_kernel<2>, grid, block, kZeroPaddingLds, stream, e0, e1, p, num_rows, row_bytes, input_perm, eo, es0, sh.chunks); break;
            default: launch_kernel(zero_padding_expert_kernel<1>, grid, block, kZeroPaddingLds, stream, e0, e1, p, num_rows, row_bytes, input_perm, eo, es0, sh.chunks); break;
            }
        });
    }
    return for_row_batches(num_rows, sh, [&](int64_t r0, int64_t, dim3 grid, dim3 block,
                                             hipEvent_t e0, hipEvent_t e1) {
        uint8_t* pr = p + r0 * row_bytes;
        const int32_t* m = input_perm + r0;
        switch (v) {
        case 16: launch_kernel(zero_padding_kernel<16>, grid, block, 0, stream, e0, e1, pr, row_bytes, m, sh.chunks); break;
        case 8: launch_kernel(zero_padding_kernel<8>, grid, block, 0, stream, e0, e1, pr, row_bytes, m, sh.chunks); break;
        case 4: launch_kernel(zero_padding_kernel<4>, grid, block, 0, stream, e0, e1, pr, row_bytes, m, sh.chunks); break;
        case 2: launch_kernel(zero_padding_kernel<2>, grid, block, 0, stream, e0, e1, pr, row_bytes, m, sh.chunks); break;
        default: launch_kernel(zero_padding_kernel<1>, grid, block, 0, stream, e0, e1, pr, row_bytes, m, sh.chunks); break;
        }
    });
}

hipError_t launch_output_memset(void* out, int64_t num_tokens, int32_t topk, int64_t row_bytes,
                                const int32_t* expanded_to_permuted, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int v = zvec_width(row_bytes, out);
    const RowShape sh = row_shape(row_bytes / v, kZeroThreads);
    uint8_t* p = static_cast<uint8_t*>(out);
    return for_row_batches(num_tokens, sh, [&](int64_t t0, int64_t, dim3 grid, dim3 block,
                                               hipEvent_t e0, hipEvent_t e1) {
        uint8_t* pt = p + t0 * row_bytes;
        const int32_t* e = expanded_to_permuted + t0 * topk;
        switch (v) {
        case 16: launch_kernel(output_memset_kernel<16>, grid, block, 0, stream, e0, e1, pt, row_bytes, topk, e, sh.chunks); break;
        case 8: launch_kernel(output_memset_kernel<8>, grid, block, 0, stream, e0, e1, pt, row_bytes, topk, e, sh.chunks); break;
        case 4: launch_kernel(output_memset_kernel<4>, grid, block, 0, stream, e0, e1, pt, row_bytes, topk, e, sh.chunks); break;
        case 2: launch_kernel(output_memset_kernel<2>, grid, block, 0, stream, e0, e1, pt, row_bytes, topk, e, sh.chunks); break;
        default: launch_kernel(output_memset_kernel<1>, grid, block, 0, stream, e0, e1, pt, row_bytes, topk, e, sh.chunks); break;
        }
    });
}

}  // namespace mxmoe
