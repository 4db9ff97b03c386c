// Combine for MoE: gather each token's k expert-output rows, scale each by its
// top-k weight and sum in fp32, then round once to the output type (the
// apply_shuffle_mul_sum call of the sglang page "[jit_kernel] Add
// prepare_moe_input JIT kernels", section "Changes", item 3: FP32
// accumulation, fp16 / bf16 / fp32).
//
// out[t][h] = round( fma(y[r_{k-1}][h], w_{k-1}, ... fma(y[r_0][h], w_0, +0)) )
// with r_j = permutation[t*k + j]; picks whose row is out of range are
// skipped.  The ascending-j chain of fused multiply-adds is the only order
// used, so the result does not depend on launch shapes.
//
// One workgroup per token and column chunk of one wave (the chunks of a token
// are neighbours in the grid), 12 to 16 per CU (see below).  A thread owns 8
// columns and issues the loads of up to 8 picks before the first
// multiply-add, so each wave keeps 8 KiB (16-bit y) of reads in flight; the
// row indices and weights are loaded one per lane and broadcast with
// readlane.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kGroup = 8;      // columns per thread in the vector path
constexpr int kPickBatch = 8;  // picks whose loads are issued together
#ifndef MXMOE_COMBINE_THREADS
#define MXMOE_COMBINE_THREADS 64
#endif
constexpr int kCombineThreads = MXMOE_COMBINE_THREADS;   // workgroup width; longer rows are cut into chunks
static_assert(kCombineThreads % kWave == 0 && kCombineThreads <= 1024, "whole waves, at most 1024");

// LDS reserved per workgroup of the vector path, which caps the one-wave
// workgroups per CU (32 without a cap): fewer gathers in flight per CU ran
// faster on MI355X.  The best cap depends on the output store policy
// (combine_store_policy below).
//   Streaming stores: 12 per CU.  Against two-wave chunks capped at 7 per CU
//     it took 1580 -> 1535 us at T = 65536 with fp32 output; 13 per CU ran
//     1522 against 1515 us, 14 and more or 11 and fewer were slower still.
//     (Uncapped, one-wave chunks had been slower than two-wave ones.)
//   Allocating stores: 13 per CU.  Against 12: 85.4 -> 84.1 us at T = 4096,
//     159.9 -> 157.3 us at K-hot T = 8192, 185.3 -> 184.3 us on the Zipf
//     workload; 11 and fewer slower everywhere.
//   Allocating stores, at most 4096 tokens: 16 per CU.  Combine alone was
//     1-7% faster than at 13 per CU from 1024 to 4096 tokens under uniform,
//     K-hot and Zipf routing, and the T = 4096, H = 7168 step 186.7-187.0 ->
//     184.4-185.2 us warm; at K-hot T = 8192 and the Zipf workload (16384
//     tokens) 16 per CU lost 3-5 us within the step.
constexpr size_t kCombineLdsStream = 13 * 1024;  // 12 per CU
constexpr size_t kCombineLdsKeep = 12 * 1024;    // 13 per CU
constexpr size_t kCombineLdsKeepSmall = 10 * 1024;  // 16 per CU
constexpr int64_t kSmallCombineTokens = 4096;


// N consecutive elements of a row, moved with one 8- or 16-byte access.
// Expert output rows are read exactly once, so the loads carry the
// non-temporal hint.  The 16-byte stores of the output rows go through
// store16 with the policy combine_store_policy picks, the 8-byte ones are
// non-temporal.
template <typename TY, int N>
struct Cols {
    static constexpr int kBytes = N * (int)sizeof(typename TY::storage);
    static_assert(kBytes == 8 || kBytes == 16, "one 8- or 16-byte access per set");
    uint32_t w[kBytes / 4];
    __device__ float at(int e) const {
        if constexpr (sizeof(typename TY::storage) == 4) {
            return __uint_as_float(w[e]);
        } else {
            const uint32_t x = w[e >> 1];
            return to_f32(TY{}, (uint16_t)((e & 1) ? (x >> 16) : (x & 0xffffu)));
        }
    }
};

template <typename TY, int N>
__device__ __forceinline__ Cols<TY, N> load_cols(const typename TY::storage* p) {
    Cols<TY, N> v;
    if (!MX_CAN_LOAD(p, (Cols<TY, N>::kBytes), kSiteCombineY)) return Cols<TY, N>{};
    if constexpr (Cols<TY, N>::kBytes == 16) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
        for (int i = 0; i < 4; ++i) v.w[i] = q[i];
    } else {
        const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        v.w[0] = q[0];
        v.w[1] = q[1];
    }
    return v;
}

// Stores columns [col, col + N) of the output row that starts at `row`
// (wave-uniform) and holds `hidden` elements.
template <typename TO, int N, int P>
__device__ __forceinline__ void store_cols(typename TO::storage* row, int64_t hidden, int64_t col,
                                           const float* acc) {
    using SO = typename TO::storage;
    constexpr int kBytes = N * (int)sizeof(SO);
    static_assert(kBytes == 8 || kBytes == 16, "one 8- or 16-byte access per set");
    uint32_t w[kBytes / 4];
    if constexpr (sizeof(SO) == 2) {
#pragma unroll
        for (int i = 0; i < kBytes / 4; ++i)
            w[i] = (uint32_t)from_f32(TO{}, acc[2 * i]) |
                   ((uint32_t)from_f32(TO{}, acc[2 * i + 1]) << 16);
    } else {
#pragma unroll
        for (int i = 0; i < kBytes / 4; ++i) w[i] = __float_as_uint(acc[i]);
    }
    if constexpr (kBytes == 16) {
        const u32x4 q = {w[0], w[1], w[2], w[3]};
        store16<P>(q, reinterpret_cast<uint8_t*>(row), hidden * (int64_t)sizeof(SO),
                   col * (int64_t)sizeof(SO), kSiteCombineOut);
    } else {
        const u32x2 q = {w[0], w[1]};
        if (MX_CAN_STORE(row + col, 8, kSiteCombineOut))
            __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(row + col));
    }
}

// Cache policy of the output stores.  While the whole output fits in the 256
// MB Infinity Cache the stores allocate (kKeep) and the lines are written
// back after the kernel, during whatever runs next; a larger output streams
// (kStream).  On MI355X, under the occupancy cap, allocating stores took
// combine from 90.2 to 88.3 us at T = 4096 (58.7 MB of output), 165.1 ->
// 161.0 us at K-hot T = 8192 and 189.7 -> 185.5 us for the Zipf workload,
// with the whole step shorter by as much; the 1.88 GB fp32 output at T =
// 65536 ran 1572 us allocating against 1522 us streaming and 1528 us with
// plain non-temporal stores.
inline StorePolicy combine_store_policy(int64_t out_bytes) {
    return out_bytes > kCacheResidentBytes ? kStream : kKeep;
}

// Weight of pick (t, j) in fp32.  FDT: -1 unit weights, else the dtype code
// (0 fp32, 1 fp16, 2 bf16).
template <int FDT>
__device__ __forceinline__ float load_factor(const void* f, int64_t idx) {
    if constexpr (FDT < 0) {
        return 1.0f;
    } else if constexpr (FDT == 0) {
        const float* q = static_cast<const float*>(f) + idx;
        return MX_CAN_LOAD(q, 4, kSiteCombineFactor) ? *q : 0.0f;
    } else {
        const uint16_t* q = static_cast<const uint16_t*>(f) + idx;
        const uint16_t h = MX_CAN_LOAD(q, 2, kSiteCombineFactor) ? *q : (uint16_t)0;
        if constexpr (FDT == 1) return to_f32(F16{}, h);
        else return to_f32(BF16{}, h);
    }
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Vector path: hidden % 8 == 0 and y / out 16-byte aligned.  A thread owns 8
// columns.  With 16-bit y and out they are 8 consecutive columns (16-byte
// loads and stores).  When y or out is fp32 they are two sets of 4, at
// lane*4 and 256 + lane*4 within the wave's 512 columns, so that every
// 16-byte access of a wave covers 1 KiB of one row: 8 consecutive fp32
// columns per lane would leave every other 16 bytes of each load or store
// instruction to the next one.  Measured on MI355X at T = 65536 (bf16 y, fp32
// out): 16-byte loads of 8 consecutive columns with two such half-filled
// 16-byte stores ran 2703 us against 1528 us for this layout, same bits.  Each wave loads the token's row indices and
// weights one per lane (one vector load each) and broadcasts them with
// readlane; every loop around a readlane is uniform, so threads past the row
// end stay in the loops and only skip their memory accesses.
template <typename TY, typename TO, int FDT, int P>
__global__ __launch_bounds__(kCombineThreads) void combine_vec_kernel(
    const typename TY::storage* __restrict__ y, int64_t num_y_rows, int64_t hidden,
    const int32_t* __restrict__ perm, const void* __restrict__ factors, int32_t topk,
    typename TO::storage* __restrict__ out, int32_t chunks) {
    constexpr int kSets =
        (sizeof(typename TY::storage) == 4 || sizeof(typename TO::storage) == 4) ? 2 : 1;
    constexpr int kCols = kGroup / kSets;
    int64_t chunk;
    const int64_t t = chunk_row(chunks, chunk);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave_col = (chunk * blockDim.x + (threadIdx.x - lane)) * kGroup;
    int64_t col[kSets];
    bool active[kSets];
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
        col[s] = wave_col + (int64_t)(s * kWave + lane) * kCols;
        active[s] = col[s] < hidden;
    }
    const int32_t* rows = perm + t * topk;
    float acc[kSets][kCols];
#pragma unroll
    for (int s = 0; s < kSets; ++s)
#pragma unroll
        for (int e = 0; e < kCols; ++e) acc[s][e] = 0.0f;
    for (int j0 = 0; j0 < topk; j0 += kWave) {
        const int nj = topk - j0 < kWave ? topk - j0 : kWave;
        int my_r = -1;
        float my_w = 0.0f;
        if (lane < nj) {
            my_r = MX_CAN_LOAD(rows + j0 + lane, 4, kSiteCombineIndex) ? rows[j0 + lane] : -1;
            if (my_r >= num_y_rows) my_r = -1;
            my_w = load_factor<FDT>(factors, t * topk + j0 + lane);
        }
        for (int jb = 0; jb < nj; jb += kPickBatch) {
            int32_t r[kPickBatch];
            float w[kPickBatch];
            Cols<TY, kCols> v[kPickBatch][kSets];
#pragma unroll
            for (int jj = 0; jj < kPickBatch; ++jj) {
                r[jj] = jb + jj < nj ? __builtin_amdgcn_readlane(my_r, jb + jj) : -1;
                w[jj] = readlane_f(my_w, jb + jj);
            }
            if constexpr (FDT == 0) {
                // fp32 weights: the wait for the weights comes before the
                // batch, so the row loads below go out together as they are
                // (checked in the assembly by the combine ISA test), and
                // this form measured about 1% faster than the one below.
#pragma unroll
                for (int jj = 0; jj < kPickBatch; ++jj)
#pragma unroll
                    for (int s = 0; s < kSets; ++s)
                        if (r[jj] >= 0 && active[s])
                            v[jj][s] = load_cols<TY, kCols>(y + (int64_t)r[jj] * hidden + col[s]);
#pragma unroll
                for (int jj = 0; jj < kPickBatch; ++jj) {
                    if (r[jj] < 0) continue;
#pragma unroll
                    for (int s = 0; s < kSets; ++s)
#pragma unroll
                        for (int e = 0; e < kCols; ++e)
                            acc[s][e] = __builtin_fmaf(v[jj][s].at(e), w[jj], acc[s][e]);
                }
            } else {
                // Every multiply-add runs whether or not its row was loaded:
                // a skipped row is zeros with weight zero, which leaves acc as
                // it is (acc starts at +0 and a sum is -0 only if both terms
                // are, so acc is never -0 and acc + 0 == acc).  Under the same
                // test as the loads, the compiler could not pair loads with
                // their uses in these forms and waited for every load before
                // issuing the next, at half the bandwidth.
#pragma unroll
                for (int jj = 0; jj < kPickBatch; ++jj)
#pragma unroll
                    for (int s = 0; s < kSets; ++s) {
                        v[jj][s] = Cols<TY, kCols>{};
                        if (r[jj] >= 0 && active[s])
                            v[jj][s] = load_cols<TY, kCols>(y + (int64_t)r[jj] * hidden + col[s]);
                    }
#pragma unroll
                for (int jj = 0; jj < kPickBatch; ++jj) {
                    const float wj = r[jj] >= 0 ? w[jj] : 0.0f;
#pragma unroll
                    for (int s = 0; s < kSets; ++s)
#pragma unroll
                        for (int e = 0; e < kCols; ++e)
                            acc[s][e] = __builtin_fmaf(v[jj][s].at(e), wj, acc[s][e]);
                }
            }
        }
    }
#pragma unroll
    for (int s = 0; s < kSets; ++s)
        if (active[s]) store_cols<TO, kCols, P>(out + t * hidden, hidden, col[s], acc[s]);
}

// Scalar path for any hidden size and element-aligned pointers.
template <typename TY, typename TO, int FDT>
__global__ __launch_bounds__(kCombineThreads) void combine_scalar_kernel(
    const typename TY::storage* __restrict__ y, int64_t num_y_rows, int64_t hidden,
    const int32_t* __restrict__ perm, const void* __restrict__ factors, int32_t topk,
    typename TO::storage* __restrict__ out, int32_t chunks) {
    int64_t chunk;
    const int64_t t = chunk_row(chunks, chunk);
    const int64_t h = chunk * blockDim.x + threadIdx.x;
    if (h >= hidden) return;
    const int32_t* rows = perm + t * topk;
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j) {
        const int32_t r = MX_CAN_LOAD(rows + j, 4, kSiteCombineIndex) ? rows[j] : -1;
        if (r < 0 || r >= num_y_rows) continue;
        const float w = load_factor<FDT>(factors, t * topk + j);
        const typename TY::storage* q = y + (int64_t)r * hidden + h;
        const typename TY::storage x =
            MX_CAN_LOAD(q, sizeof(*q), kSiteCombineY) ? *q : typename TY::storage{};
        acc = __builtin_fmaf(to_f32(TY{}, x), w, acc);
    }
    if (MX_CAN_STORE(out + t * hidden + h, sizeof(*out), kSiteCombineOut))
        out[t * hidden + h] = from_f32(TO{}, acc);
}

template <typename TY, typename TO, int FDT>
hipError_t launch_typed(const void* y, int64_t num_y_rows, int64_t hidden, const int32_t* perm,
                        const void* factors, int64_t T, int32_t topk, void* out,
                        hipStream_t stream, hipEvent_t start, hipEvent_t stop) {
    using SY = typename TY::storage;
    using SO = typename TO::storage;
    const bool vec = hidden % kGroup == 0 && ((uintptr_t)y % 16) == 0 && ((uintptr_t)out % 16) == 0;
    const RowShape sh = row_shape(vec ? hidden / kGroup : hidden, kCombineThreads);
    const int64_t factor_bytes = FDT == 0 ? 4 : 2;
    const bool keep = combine_store_policy(T * hidden * (int64_t)sizeof(SO)) == kKeep;
    const size_t keep_lds = T <= kSmallCombineTokens ? kCombineLdsKeepSmall : kCombineLdsKeep;
    return for_row_batches(T, sh, [&](int64_t t0, int64_t, dim3 grid, dim3 block,
                                      hipEvent_t e0, hipEvent_t e1) {
        const int32_t* p = perm + t0 * topk;
        const void* f = factors ? static_cast<const char*>(factors) + t0 * topk * factor_bytes
                                : nullptr;
        SO* o = static_cast<SO*>(out) + t0 * hidden;
        if (vec && keep)
            launch_kernel(combine_vec_kernel<TY, TO, FDT, kKeep>, grid, block, keep_lds, stream,
                          e0, e1, static_cast<const SY*>(y), num_y_rows, hidden, p, f, topk, o,
                          sh.chunks);
        else if (vec)
            launch_kernel(combine_vec_kernel<TY, TO, FDT, kStream>, grid, block, kCombineLdsStream, stream,
                          e0, e1, static_cast<const SY*>(y), num_y_rows, hidden, p, f, topk, o,
                          sh.chunks);
        else
            launch_kernel(combine_scalar_kernel<TY, TO, FDT>, grid, block, 0, stream, e0, e1,
                          static_cast<const SY*>(y), num_y_rows, hidden, p, f, topk, o, sh.chunks);
    }, start, stop);
}

template <typename TY, typename TO>
hipError_t launch_factor(int fdt, const void* y, int64_t num_y_rows, int64_t hidden,
                         const int32_t* perm, const void* factors, int64_t T, int32_t topk,
                         void* out, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    switch (fdt) {
    case -1: return launch_typed<TY, TO, -1>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    case 0: return launch_typed<TY, TO, 0>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    case 1: return launch_typed<TY, TO, 1>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    default: return launch_typed<TY, TO, 2>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    }
}

template <typename TY>
hipError_t launch_out(int out_dtype, const void* y, int64_t num_y_rows, int64_t hidden,
                      const int32_t* perm, const void* factors, int fdt, int64_t T,
                      int32_t topk, void* out, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    switch (out_dtype) {
    case 0: return launch_factor<TY, F32>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    case 1: return launch_factor<TY, F16>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    default: return launch_factor<TY, BF16>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream, e0, e1);
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, int64_t num_y_rows, int64_t hidden,
                          const int32_t* perm, const void* factors, int factors_dtype,
                          int64_t num_tokens, int32_t topk, void* out, int out_dtype,
                          hipStream_t stream, hipEvent_t start_event, hipEvent_t stop_event) {
    if (num_tokens == 0 || hidden == 0) return hipSuccess;
    const int fdt = factors ? factors_dtype : -1;
    hipEvent_t e0 = start_event, e1 = stop_event;
    switch (y_dtype) {
    case 0: return launch_out<F32>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream, e0, e1);
    case 1: return launch_out<F16>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream, e0, e1);
    default: return launch_out<BF16>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream, e0, e1);
    }
}

}  // namespace mxmoe
