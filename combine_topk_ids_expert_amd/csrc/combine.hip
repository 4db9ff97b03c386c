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
// One workgroup per token (and column chunk).  A thread owns 8 consecutive
// columns and issues the 16-byte loads of up to 8 picks before the first
// multiply-add, so each wave keeps 8 KiB (16-bit y) of reads in flight; the
// row indices and weights are loaded one per lane and broadcast with
// readlane.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kGroup = 8;      // columns per thread in the vector path
constexpr int kPickBatch = 8;  // picks whose loads are issued together
constexpr int kMaxThreads = 1024;


// 8 consecutive elements of a row, moved with 16-byte accesses.  Expert
// output rows are read exactly once, so the loads carry the non-temporal
// hint; so do the stores of the write-once output rows.
template <typename TY> struct Pack;
template <> struct Pack<BF16> { u32x4 q; __device__ float at(int e) const { const uint32_t w = q[e >> 1]; return to_f32(BF16{}, (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu))); } };
template <> struct Pack<F16> { u32x4 q; __device__ float at(int e) const { const uint32_t w = q[e >> 1]; return to_f32(F16{}, (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu))); } };
template <> struct Pack<F32> { u32x4 q[2]; __device__ float at(int e) const { return __uint_as_float(q[e >> 2][e & 3]); } };

template <typename TY>
__device__ __forceinline__ Pack<TY> load_pack(const typename TY::storage* p) {
    Pack<TY> v;
    const u32x4* q = reinterpret_cast<const u32x4*>(p);
    if constexpr (sizeof(typename TY::storage) == 2) {
        v.q = __builtin_nontemporal_load(q);
    } else {
        v.q[0] = __builtin_nontemporal_load(q);
        v.q[1] = __builtin_nontemporal_load(q + 1);
    }
    return v;
}

template <typename TO>
__device__ __forceinline__ void store_pack(typename TO::storage* p, const float* acc) {
    u32x4* o = reinterpret_cast<u32x4*>(p);
    if constexpr (sizeof(typename TO::storage) == 2) {
        u32x4 q;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            q[i] = (uint32_t)from_f32(TO{}, acc[2 * i]) |
                   ((uint32_t)from_f32(TO{}, acc[2 * i + 1]) << 16);
        __builtin_nontemporal_store(q, o);
    } else {
        const u32x4 q0 = {__float_as_uint(acc[0]), __float_as_uint(acc[1]),
                          __float_as_uint(acc[2]), __float_as_uint(acc[3])};
        const u32x4 q1 = {__float_as_uint(acc[4]), __float_as_uint(acc[5]),
                          __float_as_uint(acc[6]), __float_as_uint(acc[7])};
        __builtin_nontemporal_store(q0, o);
        __builtin_nontemporal_store(q1, o + 1);
    }
}

// Weight of pick (t, j) in fp32.  FDT: -1 unit weights, else the dtype code
// (0 fp32, 1 fp16, 2 bf16).
template <int FDT>
__device__ __forceinline__ float load_factor(const void* f, int64_t idx) {
    if constexpr (FDT < 0) {
        return 1.0f;
    } else if constexpr (FDT == 0) {
        return static_cast<const float*>(f)[idx];
    } else {
        const uint16_t h = static_cast<const uint16_t*>(f)[idx];
        if constexpr (FDT == 1) return to_f32(F16{}, h);
        else return to_f32(BF16{}, h);
    }
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Vector path: hidden % 8 == 0 and y / out 16-byte aligned.  Each wave loads
// the token's row indices and weights one per lane (one vector load each) and
// broadcasts them with readlane; every loop around a readlane is uniform, so
// threads past the row end stay in the loops and only skip their memory
// accesses.
template <typename TY, typename TO, int FDT>
__global__ __launch_bounds__(kMaxThreads) void combine_vec_kernel(
    const typename TY::storage* __restrict__ y, int64_t num_y_rows, int64_t hidden,
    const int32_t* __restrict__ perm, const void* __restrict__ factors, int32_t topk,
    typename TO::storage* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t col = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * kGroup;
    const bool active = col < hidden;
    const int32_t* rows = perm + t * topk;
    float acc[kGroup];
#pragma unroll
    for (int e = 0; e < kGroup; ++e) acc[e] = 0.0f;
    for (int j0 = 0; j0 < topk; j0 += kWave) {
        const int nj = topk - j0 < kWave ? topk - j0 : kWave;
        int my_r = -1;
        float my_w = 0.0f;
        if (lane < nj) {
            my_r = rows[j0 + lane];
            if (my_r >= num_y_rows) my_r = -1;
            my_w = load_factor<FDT>(factors, t * topk + j0 + lane);
        }
        for (int jb = 0; jb < nj; jb += kPickBatch) {
            int32_t r[kPickBatch];
            float w[kPickBatch];
            Pack<TY> v[kPickBatch];
#pragma unroll
            for (int jj = 0; jj < kPickBatch; ++jj) {
                r[jj] = jb + jj < nj ? __builtin_amdgcn_readlane(my_r, jb + jj) : -1;
                w[jj] = readlane_f(my_w, jb + jj);
            }
#pragma unroll
            for (int jj = 0; jj < kPickBatch; ++jj)
                if (r[jj] >= 0 && active) v[jj] = load_pack<TY>(y + (int64_t)r[jj] * hidden + col);
#pragma unroll
            for (int jj = 0; jj < kPickBatch; ++jj) {
                if (r[jj] < 0) continue;
#pragma unroll
                for (int e = 0; e < kGroup; ++e)
                    acc[e] = __builtin_fmaf(v[jj].at(e), w[jj], acc[e]);
            }
        }
    }
    if (active) store_pack<TO>(out + t * hidden + col, acc);
}

// Scalar path for any hidden size and element-aligned pointers.
template <typename TY, typename TO, int FDT>
__global__ __launch_bounds__(kMaxThreads) void combine_scalar_kernel(
    const typename TY::storage* __restrict__ y, int64_t num_y_rows, int64_t hidden,
    const int32_t* __restrict__ perm, const void* __restrict__ factors, int32_t topk,
    typename TO::storage* __restrict__ out) {
    const int64_t t = blockIdx.x;
    const int64_t h = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    if (h >= hidden) return;
    const int32_t* rows = perm + t * topk;
    float acc = 0.0f;
    for (int j = 0; j < topk; ++j) {
        const int32_t r = rows[j];
        if (r < 0 || r >= num_y_rows) continue;
        const float w = load_factor<FDT>(factors, t * topk + j);
        acc = __builtin_fmaf(to_f32(TY{}, y[(int64_t)r * hidden + h]), w, acc);
    }
    out[t * hidden + h] = from_f32(TO{}, acc);
}

template <typename TY, typename TO, int FDT>
hipError_t launch_typed(const void* y, int64_t num_y_rows, int64_t hidden, const int32_t* perm,
                        const void* factors, int64_t T, int32_t topk, void* out,
                        hipStream_t stream) {
    using SY = typename TY::storage;
    using SO = typename TO::storage;
    const bool vec = hidden % kGroup == 0 && ((uintptr_t)y % 16) == 0 && ((uintptr_t)out % 16) == 0;
    const int64_t items = vec ? hidden / kGroup : hidden;
    int64_t threads = (items + kWave - 1) / kWave * kWave;
    if (threads > kMaxThreads) threads = kMaxThreads;
    const int64_t chunks = (items + threads - 1) / threads;
    const dim3 grid((unsigned)T, (unsigned)chunks, 1);
    if (vec)
        combine_vec_kernel<TY, TO, FDT><<<grid, (unsigned)threads, 0, stream>>>(
            static_cast<const SY*>(y), num_y_rows, hidden, perm, factors, topk,
            static_cast<SO*>(out));
    else
        combine_scalar_kernel<TY, TO, FDT><<<grid, (unsigned)threads, 0, stream>>>(
            static_cast<const SY*>(y), num_y_rows, hidden, perm, factors, topk,
            static_cast<SO*>(out));
    return hipGetLastError();
}

template <typename TY, typename TO>
hipError_t launch_factor(int fdt, const void* y, int64_t num_y_rows, int64_t hidden,
                         const int32_t* perm, const void* factors, int64_t T, int32_t topk,
                         void* out, hipStream_t stream) {
    switch (fdt) {
    case -1: return launch_typed<TY, TO, -1>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    case 0: return launch_typed<TY, TO, 0>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    case 1: return launch_typed<TY, TO, 1>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    default: return launch_typed<TY, TO, 2>(y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    }
}

template <typename TY>
hipError_t launch_out(int out_dtype, const void* y, int64_t num_y_rows, int64_t hidden,
                      const int32_t* perm, const void* factors, int fdt, int64_t T,
                      int32_t topk, void* out, hipStream_t stream) {
    switch (out_dtype) {
    case 0: return launch_factor<TY, F32>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    case 1: return launch_factor<TY, F16>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    default: return launch_factor<TY, BF16>(fdt, y, num_y_rows, hidden, perm, factors, T, topk, out, stream);
    }
}

}  // namespace

hipError_t launch_combine(const void* y, int y_dtype, int64_t num_y_rows, int64_t hidden,
                          const int32_t* perm, const void* factors, int factors_dtype,
                          int64_t num_tokens, int32_t topk, void* out, int out_dtype,
                          hipStream_t stream) {
    if (num_tokens == 0 || hidden == 0) return hipSuccess;
    const int fdt = factors ? factors_dtype : -1;
    switch (y_dtype) {
    case 0: return launch_out<F32>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream);
    case 1: return launch_out<F16>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream);
    default: return launch_out<BF16>(out_dtype, y, num_y_rows, hidden, perm, factors, fdt, num_tokens, topk, out, stream);
    }
}

}  // namespace mxmoe
