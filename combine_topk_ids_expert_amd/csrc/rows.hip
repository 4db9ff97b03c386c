// Row movement for MoE dispatch: the dtype-agnostic row gather (shuffle_rows,
// sglang page "[jit_kernel] Add prepare_moe_input JIT kernels", section
// "Changes", item 2, which copies rows with 16-byte vector accesses) and its
// token-major scatter form, which reads every token row once and writes it to
// each of its k dispatched rows.
//
// Both are HBM-bound byte copies.  A workgroup owns one row (or a column
// chunk of at most 1024 vectors of one row) and each thread moves exactly one
// 16-byte vector: one load, then one store per destination.  Short-lived
// workgroups with one access per thread sustained the highest write rate on
// MI355X (several accesses per thread, or looping workgroups, wrote slower).
// The write-once destination rows are stored non-temporal and system-coherent
// (store16_stream), the source rows are loaded with the default policy: both
// measured fastest of the cache policies tried.  Rows whose byte width or base
// pointers are not multiples of 16 fall back to the widest access width that
// divides them.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kMaxRowThreads = 1024;


template <int V> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

// Copies vector c of one row (vectors of T) to each destination row
// rows[0..n) that lies in [0, num_dst_rows); with rows == nullptr the only
// destination is `single_row`.  Threads past the row end (c >= nvec) take
// part in the wave-uniform destination loop but access nothing.  The
// destination indices sit one per lane and are broadcast with readlane;
// destination rows are written once and not read again by this pass, so the
// stores carry the non-temporal hint (16-byte ones through store16_stream,
// which adds the system-coherent bits).
template <typename T>
__device__ __forceinline__ void copy_vector_to(const T* __restrict__ in, int64_t c, int64_t nvec,
                                               uint8_t* __restrict__ dst, int64_t row_bytes,
                                               const int32_t* __restrict__ rows, int n,
                                               int64_t num_dst_rows, int32_t single_row = -1) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool live = c < nvec;
    T v{};
    if (live) v = in[c];
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int nj = n - j0 < kWave ? n - j0 : kWave;
        int my_r = lane < nj ? (rows ? rows[j0 + lane] : single_row) : -1;
        if (my_r >= num_dst_rows) my_r = -1;
        for (int j = 0; j < nj; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(my_r, j);
            if (r < 0 || !live) continue;
            uint8_t* row = dst + (int64_t)r * row_bytes;
            if constexpr (sizeof(T) == 16)
                store16_stream(v, row, row_bytes, c * 16);
            else
                __builtin_nontemporal_store(v, reinterpret_cast<T*>(row) + c);
        }
    }
}

// dst[r] = src[dst2src[r]]: workgroup (blockIdx.x = r, blockIdx.y = column
// chunk), one vector per thread.
template <int V>
__global__ __launch_bounds__(kMaxRowThreads) void shuffle_rows_kernel(
    const uint8_t* __restrict__ src, int64_t num_src_rows, int64_t row_bytes,
    const int32_t* __restrict__ dst2src, uint8_t* __restrict__ dst) {
    using T = typename Vec<V>::T;
    const int32_t r = (int32_t)blockIdx.x;
    const int32_t s = dst2src[r];
    if (s < 0 || s >= num_src_rows) return;
    const int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    const T* in = reinterpret_cast<const T*>(src + (int64_t)s * row_bytes);
    copy_vector_to<T>(in, c, row_bytes / V, dst, row_bytes, nullptr, 1, (int64_t)r + 1, r);
}

// dst[output_perm[t*k + j]] = src[t] for every j: workgroup (blockIdx.x =
// token t, blockIdx.y = column chunk), one vector per thread; the side row
// (if any) goes with chunk 0.
template <int V, int SV>
__global__ __launch_bounds__(kMaxRowThreads) void dispatch_rows_kernel(
    const uint8_t* __restrict__ src, int64_t row_bytes, int32_t topk,
    const int32_t* __restrict__ output_perm, uint8_t* __restrict__ dst, int64_t num_dst_rows,
    const uint8_t* __restrict__ side_src, int64_t side_row_bytes,
    uint8_t* __restrict__ side_dst) {
    using T = typename Vec<V>::T;
    const int64_t t = blockIdx.x;
    const int32_t* rows = output_perm + t * topk;
    const int64_t c = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    copy_vector_to<T>(reinterpret_cast<const T*>(src + t * row_bytes), c, row_bytes / V, dst,
                      row_bytes, rows, topk, num_dst_rows);
    if constexpr (SV > 0) {
        using S = typename Vec<SV>::T;
        if (blockIdx.y == 0) {
            const int64_t ns = side_row_bytes / SV;
            for (int64_t c0 = 0; c0 < ns; c0 += blockDim.x)
                copy_vector_to<S>(reinterpret_cast<const S*>(side_src + t * side_row_bytes),
                                  c0 + threadIdx.x, ns, side_dst, side_row_bytes, rows, topk,
                                  num_dst_rows);
        }
    }
}

int vec_width(int64_t row_bytes, const void* a, const void* b) {
    const uint64_t bits = (uint64_t)row_bytes | (uint64_t)(uintptr_t)a | (uint64_t)(uintptr_t)b;
    for (int v = 16; v > 1; v >>= 1)
        if ((bits & (uint64_t)(v - 1)) == 0) return v;
    return 1;
}

// Launch shape: one vector per thread; a row of nvec vectors is cut into the
// fewest column chunks of at most kMaxRowThreads vectors, and the workgroup
// width is the chunk rounded up to whole waves.
void row_grid(int64_t rows, int64_t row_bytes, int v, dim3& grid, dim3& block) {
    const int64_t nvec = row_bytes / v;
    const int64_t chunks = (nvec + kMaxRowThreads - 1) / kMaxRowThreads;
    int64_t threads = (nvec + chunks - 1) / chunks;
    threads = (threads + kWave - 1) / kWave * kWave;
    grid = dim3((unsigned)rows, (unsigned)chunks, 1);
    block = dim3((unsigned)threads, 1, 1);
}

template <int V>
hipError_t launch_dispatch_v(dim3 grid, dim3 block, int side_vec, const uint8_t* s,
                             int64_t row_bytes, int32_t topk, const int32_t* output_perm,
                             uint8_t* d, int64_t num_dst_rows, const uint8_t* ss,
                             int64_t side_row_bytes, uint8_t* sd, hipStream_t stream) {
    switch (side_vec) {
    case 0: dispatch_rows_kernel<V, 0><<<grid, block, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd); break;
    case 16: dispatch_rows_kernel<V, 16><<<grid, block, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd); break;
    case 4: dispatch_rows_kernel<V, 4><<<grid, block, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd); break;
    default: dispatch_rows_kernel<V, 1><<<grid, block, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                               const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                               hipStream_t stream) {
    if (num_dst_rows == 0) return hipSuccess;
    const int v = vec_width(row_bytes, src, dst);
    dim3 grid, block;
    row_grid(num_dst_rows, row_bytes, v, grid, block);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    switch (v) {
    case 16: shuffle_rows_kernel<16><<<grid, block, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d); break;
    case 8: shuffle_rows_kernel<8><<<grid, block, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d); break;
    case 4: shuffle_rows_kernel<4><<<grid, block, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d); break;
    case 2: shuffle_rows_kernel<2><<<grid, block, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d); break;
    default: shuffle_rows_kernel<1><<<grid, block, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d); break;
    }
    return hipGetLastError();
}

hipError_t launch_dispatch_rows(const void* src, int64_t num_tokens, int32_t topk,
                                int64_t row_bytes, const int32_t* output_perm, void* dst,
                                int64_t num_dst_rows, const void* side_src,
                                int64_t side_row_bytes, void* side_dst, hipStream_t stream) {
    if (num_tokens == 0) return hipSuccess;
    const int v = vec_width(row_bytes, src, dst);
    int side_vec = 0;
    if (side_src != nullptr) {
        const int sv = vec_width(side_row_bytes, side_src, side_dst);
        side_vec = sv >= 16 ? 16 : sv >= 4 ? 4 : 1;
    }
    dim3 grid, block;
    row_grid(num_tokens, row_bytes, v, grid, block);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    const uint8_t* ss = static_cast<const uint8_t*>(side_src);
    uint8_t* sd = static_cast<uint8_t*>(side_dst);
    switch (v) {
    case 16: return launch_dispatch_v<16>(grid, block, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, stream);
    case 8: return launch_dispatch_v<8>(grid, block, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, stream);
    case 4: return launch_dispatch_v<4>(grid, block, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, stream);
    case 2: return launch_dispatch_v<2>(grid, block, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, stream);
    default: return launch_dispatch_v<1>(grid, block, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, stream);
    }
}

}  // namespace mxmoe
