// Row movement for MoE dispatch: the dtype-agnostic row gather (shuffle_rows,
// sglang page "[jit_kernel] Add prepare_moe_input JIT kernels", section
// "Changes", item 2, which copies rows with 16-byte vector accesses) and its
// token-major scatter form, which reads every token row once and writes it to
// each of its k dispatched rows.
//
// Both are HBM-bound byte copies.  A workgroup owns one row (or a column
// chunk of one row); each thread loads its kUnroll vectors of a round before
// storing any, so a wave keeps kUnroll KiB of 16-byte reads in flight, and
// the write-once destination rows are stored with the non-temporal hint.  Rows
// whose byte width or base pointers are not multiples of 16 fall back to the
// widest access width that divides them.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kRowThreads = 256;
constexpr int kUnroll = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int V> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

// Destination rows are written once and not read again by this pass, so
// stores carry the non-temporal hint (streamed past the caches instead of
// displacing data still to be read).
template <typename T>
__device__ __forceinline__ void put(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

// Copies columns [c0, c1) of one row (vectors of T) to each destination row
// rows[0..n) that lies in [0, num_dst_rows); with rows == nullptr the only
// destination is `single_row`.  The column rounds and the
// destination loop are uniform across the workgroup, so the destination
// indices sit one per lane and are broadcast with readlane.
template <typename T>
__device__ __forceinline__ void copy_row_to(const T* __restrict__ in, int64_t c0, int64_t c1,
                                            uint8_t* __restrict__ dst, int64_t row_bytes,
                                            const int32_t* __restrict__ rows, int n,
                                            int64_t num_dst_rows, int32_t single_row = -1) {
    const int lane = threadIdx.x & (kWave - 1);
    constexpr int64_t kStep = (int64_t)kRowThreads * kUnroll;
    for (int64_t b = c0; b < c1; b += kStep) {
        const int64_t c = b + threadIdx.x;
        const bool full = b + kStep <= c1;
        T v0{}, v1{}, v2{}, v3{};
        if (full) {
            v0 = in[c];
            v1 = in[c + kRowThreads];
            v2 = in[c + 2 * kRowThreads];
            v3 = in[c + 3 * kRowThreads];
        } else {
            if (c < c1) v0 = in[c];
            if (c + kRowThreads < c1) v1 = in[c + kRowThreads];
            if (c + 2 * kRowThreads < c1) v2 = in[c + 2 * kRowThreads];
            if (c + 3 * kRowThreads < c1) v3 = in[c + 3 * kRowThreads];
        }
        for (int j0 = 0; j0 < n; j0 += kWave) {
            const int nj = n - j0 < kWave ? n - j0 : kWave;
            int my_r = lane < nj ? (rows ? rows[j0 + lane] : single_row) : -1;
            if (my_r >= num_dst_rows) my_r = -1;
            for (int j = 0; j < nj; ++j) {
                const int32_t r = __builtin_amdgcn_readlane(my_r, j);
                if (r < 0) continue;
                T* out = reinterpret_cast<T*>(dst + (int64_t)r * row_bytes);
                if (full) {
                    put(out + c, v0);
                    put(out + c + kRowThreads, v1);
                    put(out + c + 2 * kRowThreads, v2);
                    put(out + c + 3 * kRowThreads, v3);
                } else {
                    if (c < c1) put(out + c, v0);
                    if (c + kRowThreads < c1) put(out + c + kRowThreads, v1);
                    if (c + 2 * kRowThreads < c1) put(out + c + 2 * kRowThreads, v2);
                    if (c + 3 * kRowThreads < c1) put(out + c + 3 * kRowThreads, v3);
                }
            }
        }
    }
}

// dst[r] = src[dst2src[r]] for the column chunk blockIdx.y of row blockIdx.x.
template <int V>
__global__ __launch_bounds__(kRowThreads) void shuffle_rows_kernel(
    const uint8_t* __restrict__ src, int64_t num_src_rows, int64_t row_bytes,
    const int32_t* __restrict__ dst2src, uint8_t* __restrict__ dst, int64_t chunk_vecs) {
    using T = typename Vec<V>::T;
    const int32_t r = (int32_t)blockIdx.x;
    const int32_t s = dst2src[r];
    if (s < 0 || s >= num_src_rows) return;
    const int64_t nvec = row_bytes / V;
    const int64_t c0 = (int64_t)blockIdx.y * chunk_vecs;
    const int64_t c1 = c0 + chunk_vecs < nvec ? c0 + chunk_vecs : nvec;
    const T* in = reinterpret_cast<const T*>(src + (int64_t)s * row_bytes);
    copy_row_to<T>(in, c0, c1, dst, row_bytes, nullptr, 1, (int64_t)r + 1, r);
}

// dst[output_perm[t*k + j]] = src[t] for the column chunk blockIdx.y of token
// blockIdx.x and every j; the side row (if any) goes with chunk 0.
template <int V, int SV>
__global__ __launch_bounds__(kRowThreads) void dispatch_rows_kernel(
    const uint8_t* __restrict__ src, int64_t row_bytes, int32_t topk,
    const int32_t* __restrict__ output_perm, uint8_t* __restrict__ dst, int64_t num_dst_rows,
    int64_t chunk_vecs, const uint8_t* __restrict__ side_src, int64_t side_row_bytes,
    uint8_t* __restrict__ side_dst) {
    using T = typename Vec<V>::T;
    const int64_t t = blockIdx.x;
    const int32_t* rows = output_perm + t * topk;
    const int64_t nvec = row_bytes / V;
    const int64_t c0 = (int64_t)blockIdx.y * chunk_vecs;
    const int64_t c1 = c0 + chunk_vecs < nvec ? c0 + chunk_vecs : nvec;
    copy_row_to<T>(reinterpret_cast<const T*>(src + t * row_bytes), c0, c1, dst, row_bytes, rows,
                   topk, num_dst_rows);
    if constexpr (SV > 0) {
        using S = typename Vec<SV>::T;
        if (blockIdx.y == 0)
            copy_row_to<S>(reinterpret_cast<const S*>(side_src + t * side_row_bytes), 0,
                           side_row_bytes / SV, side_dst, side_row_bytes, rows, topk,
                           num_dst_rows);
    }
}

int vec_width(int64_t row_bytes, const void* a, const void* b) {
    const uint64_t bits = (uint64_t)row_bytes | (uint64_t)(uintptr_t)a | (uint64_t)(uintptr_t)b;
    for (int v = 16; v > 1; v >>= 1)
        if ((bits & (uint64_t)(v - 1)) == 0) return v;
    return 1;
}

// Column chunking: a workgroup covers at most kRowThreads * kUnroll * 4
// vectors of a row; longer rows are split over gridDim.y.
void row_grid(int64_t rows, int64_t row_bytes, int v, dim3& grid, int64_t& chunk_vecs) {
    const int64_t nvec = row_bytes / v;
    const int64_t max_chunk = (int64_t)kRowThreads * kUnroll * 4;
    const int64_t chunks = (nvec + max_chunk - 1) / max_chunk;
    chunk_vecs = (nvec + chunks - 1) / chunks;
    grid = dim3((unsigned)rows, (unsigned)chunks, 1);
}

template <int V>
hipError_t launch_dispatch_v(dim3 grid, int side_vec, const uint8_t* s, int64_t row_bytes,
                             int32_t topk, const int32_t* output_perm, uint8_t* d,
                             int64_t num_dst_rows, int64_t chunk, const uint8_t* ss,
                             int64_t side_row_bytes, uint8_t* sd, hipStream_t stream) {
    switch (side_vec) {
    case 0: dispatch_rows_kernel<V, 0><<<grid, kRowThreads, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd); break;
    case 16: dispatch_rows_kernel<V, 16><<<grid, kRowThreads, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd); break;
    case 4: dispatch_rows_kernel<V, 4><<<grid, kRowThreads, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd); break;
    default: dispatch_rows_kernel<V, 1><<<grid, kRowThreads, 0, stream>>>(s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                               const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                               hipStream_t stream) {
    if (num_dst_rows == 0) return hipSuccess;
    const int v = vec_width(row_bytes, src, dst);
    dim3 grid;
    int64_t chunk;
    row_grid(num_dst_rows, row_bytes, v, grid, chunk);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    switch (v) {
    case 16: shuffle_rows_kernel<16><<<grid, kRowThreads, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d, chunk); break;
    case 8: shuffle_rows_kernel<8><<<grid, kRowThreads, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d, chunk); break;
    case 4: shuffle_rows_kernel<4><<<grid, kRowThreads, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d, chunk); break;
    case 2: shuffle_rows_kernel<2><<<grid, kRowThreads, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d, chunk); break;
    default: shuffle_rows_kernel<1><<<grid, kRowThreads, 0, stream>>>(s, num_src_rows, row_bytes, dst2src, d, chunk); break;
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
    dim3 grid;
    int64_t chunk;
    row_grid(num_tokens, row_bytes, v, grid, chunk);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    const uint8_t* ss = static_cast<const uint8_t*>(side_src);
    uint8_t* sd = static_cast<uint8_t*>(side_dst);
    switch (v) {
    case 16: return launch_dispatch_v<16>(grid, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd, stream);
    case 8: return launch_dispatch_v<8>(grid, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd, stream);
    case 4: return launch_dispatch_v<4>(grid, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd, stream);
    case 2: return launch_dispatch_v<2>(grid, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd, stream);
    default: return launch_dispatch_v<1>(grid, side_vec, s, row_bytes, topk, output_perm, d, num_dst_rows, chunk, ss, side_row_bytes, sd, stream);
    }
}

}  // namespace mxmoe
