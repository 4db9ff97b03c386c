// Row movement for MoE dispatch: the dtype-agnostic row gather (shuffle_rows,
// sglang page "[jit_kernel] Add prepare_moe_input JIT kernels", section
// "Changes", item 2, which copies rows with 16-byte vector accesses) and its
// token-major scatter form, which reads every token row once and writes it to
// each of its k dispatched rows.
//
// Both are HBM-bound byte copies.  A workgroup owns a column chunk of at most
// 128 vectors of one row (the chunks of a row are neighbours in the grid) and
// each thread moves exactly one 16-byte vector: one load, then one store per
// destination; the scatter form runs at most 6 or 8 workgroups per CU.
// Short-lived workgroups with one access per thread sustained the highest
// write rate on MI355X (several accesses per thread, or looping workgroups,
// wrote slower).  The write-once destination rows are stored
// system-coherent: non-temporal while the source rows fit in the Infinity
// Cache, allocating beyond that (store16, dispatch_store_policy).  The source
// rows are loaded with the default policy.  Each measured fastest of the
// cache policies tried.  Rows whose byte width or base pointers are not
// multiples of 16 fall back to the widest access width that divides them.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

// Workgroup width of the row copies: rows of more than 128 vectors are cut
// into column chunks.  Two-wave workgroups copied 1-2% faster than one
// workgroup per 14 KiB row (896 threads).
#ifndef MXMOE_ROW_THREADS
#define MXMOE_ROW_THREADS 128
#endif
constexpr int kRowThreads = MXMOE_ROW_THREADS;
static_assert(kRowThreads % kWave == 0 && kRowThreads <= 1024, "whole waves, at most 1024");

// LDS reserved per workgroup of the row dispatch: at most 8 of its
// workgroups per CU (16 waves) instead of 16.  Fewer scattered destination
// streams per CU wrote faster on MI355X: 1632 -> 1502 us at T = 65536 over
// 288 slots, 105.3 -> 98.7 us for the FP8 rows of the Zipf workload, 170 ->
// 167 us at K-hot T = 8192 and 94 -> 92.7 us at T = 4096.  18-20 KiB
// measured alike; from 16 KiB down, or 21 KiB up, some workload lost.
constexpr size_t kDispatchLds = 19 * 1024;
// While the source rows fit the Infinity Cache (streaming stores), rows of
// 8 KiB and more wrote faster at 6 workgroups per CU: T = 4096, H = 7168 cold
// 202.1 -> 199.3-199.9 us per step and warm 188.0-188.7 -> 187.6, K-hot T =
// 8192 warm 334.5-335.4 -> 331.5 (cold level).  The FP8 rows of the Zipf
// workload (4 KiB) lost 3-18 us at 6 per CU, and the 288-slot rows, whose
// source exceeds the cache, 80 us; 5 or 4 per CU lost up to 50 us cold.
constexpr size_t kDispatchLdsWide = 26 * 1024;
constexpr int64_t kWideRowBytes = 8192;


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
// narrow stores carry the non-temporal hint and the 16-byte ones go through
// store16 with cache policy P.
template <typename T, int P = kStream>
__device__ __forceinline__ void copy_vector_to(const T* __restrict__ in, int64_t c, int64_t nvec,
                                               uint8_t* __restrict__ dst, int64_t row_bytes,
                                               const int32_t* __restrict__ rows, int n,
                                               int64_t num_dst_rows, int32_t single_row = -1) {
    const int lane = threadIdx.x & (kWave - 1);
    const bool live = c < nvec;
    T v{};
    if (live && MX_CAN_LOAD(in + c, sizeof(T), kSiteRowSrc)) v = in[c];
    for (int j0 = 0; j0 < n; j0 += kWave) {
        const int nj = n - j0 < kWave ? n - j0 : kWave;
        int my_r = -1;
        if (lane < nj)
            my_r = rows ? (MX_CAN_LOAD(rows + j0 + lane, 4, kSiteRowIndex) ? rows[j0 + lane] : -1)
                        : single_row;
        if (my_r >= num_dst_rows) my_r = -1;
        for (int j = 0; j < nj; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(my_r, j);
            if (r < 0 || !live) continue;
            uint8_t* row = dst + (int64_t)r * row_bytes;
            if constexpr (sizeof(T) == 16)
                store16<P>(v, row, row_bytes, c * 16, kSiteRowDst);
            else if (MX_CAN_STORE(reinterpret_cast<T*>(row) + c, sizeof(T), kSiteRowDst))
                __builtin_nontemporal_store(v, reinterpret_cast<T*>(row) + c);
        }
    }
}

// dst[r] = src[dst2src[r]]: one workgroup per destination row r and column
// chunk, one vector per thread.
template <int V>
__global__ __launch_bounds__(kRowThreads) void shuffle_rows_kernel(
    const uint8_t* __restrict__ src, int64_t num_src_rows, int64_t row_bytes,
    const int32_t* __restrict__ dst2src, uint8_t* __restrict__ dst, int32_t chunks) {
    using T = typename Vec<V>::T;
    int64_t chunk;
    const int64_t r = chunk_row(chunks, chunk);
    const int32_t s = MX_CAN_LOAD(dst2src + r, 4, kSiteRowIndex) ? dst2src[r] : -1;
    if (s < 0 || s >= num_src_rows) return;
    const int64_t c = chunk * blockDim.x + threadIdx.x;
    const T* in = reinterpret_cast<const T*>(src + (int64_t)s * row_bytes);
    copy_vector_to<T>(in, c, row_bytes / V, dst, row_bytes, nullptr, 1, r + 1, (int32_t)r);
}

// Destination indices a side-row thread loads before its stores.
constexpr int kSideBatch = 8;

// Side rows (the block scales of FP8 rows) of tokens [t0, t0 + group) of
// n: thread i of the workgroup takes vector i % ns of token t0 + i / ns (ns
// vectors of S per side row), loads it and the token's destination indices
// kSideBatch at a time, then stores it to each destination row.
template <typename S, int P>
__device__ __forceinline__ void copy_side_rows(const uint8_t* __restrict__ side_src,
                                               int64_t side_row_bytes, int64_t ns, int64_t t0,
                                               int32_t group, int64_t n,
                                               const int32_t* __restrict__ output_perm,
                                               int32_t topk, uint8_t* __restrict__ side_dst,
                                               int64_t num_dst_rows) {
    for (int64_t c0 = 0; c0 < ns * group; c0 += blockDim.x) {
        const int64_t i = c0 + threadIdx.x;
        const int64_t u = i / ns;
        const int64_t p = i - u * ns;
        const int64_t t = t0 + u;
        const bool live = u < group && t < n;
        const S* in = reinterpret_cast<const S*>(side_src + t * side_row_bytes) + p;
        S v{};
        if (live && MX_CAN_LOAD(in, sizeof(S), kSiteRowSrc)) v = *in;
        for (int j0 = 0; j0 < topk; j0 += kSideBatch) {
            int32_t dr[kSideBatch];
#pragma unroll
            for (int jj = 0; jj < kSideBatch; ++jj) {
                const int32_t* q = output_perm + t * topk + j0 + jj;
                dr[jj] = live && j0 + jj < topk && MX_CAN_LOAD(q, 4, kSiteRowIndex) ? *q : -1;
            }
#pragma unroll
            for (int jj = 0; jj < kSideBatch; ++jj) {
                const int32_t r = dr[jj];
                if (r < 0 || r >= num_dst_rows) continue;
                uint8_t* row = side_dst + (int64_t)r * side_row_bytes;
                if constexpr (sizeof(S) == 16)
                    store16<P>(v, row, side_row_bytes, p * 16, kSiteRowDst);
                else if (MX_CAN_STORE(reinterpret_cast<S*>(row) + p, sizeof(S), kSiteRowDst))
                    __builtin_nontemporal_store(v, reinterpret_cast<S*>(row) + p);
            }
        }
    }
}

// dst[output_perm[t*k + j]] = src[t] for every j: one workgroup per token t
// and column chunk, one vector per thread.  P is the cache policy of the
// 16-byte stores.  With side rows (SV > 0) the n tokens of the launch are
// taken in groups of `group`: the group's group * chunks row workgroups,
// then one workgroup for the group's side rows (copy_side_rows).  Side rows
// copied by chunk 0 of each token after its row had cost the Zipf workload's
// FP8 dispatch (4 KiB rows, 128-byte scale rows) 140.5 us against 106 us
// without them, with the caches flushed before the call; the separate side
// workgroups took it to 113.5 us.  With the caches warm the separate form
// measured 105.6 us against 99.6 us: there the longer chunk-0 workgroups had
// thinned the scattered row writes in flight.
template <int V, int SV, int P>
__global__ __launch_bounds__(kRowThreads) void dispatch_rows_kernel(
    const uint8_t* __restrict__ src, int64_t row_bytes, int32_t topk,
    const int32_t* __restrict__ output_perm, uint8_t* __restrict__ dst, int64_t num_dst_rows,
    const uint8_t* __restrict__ side_src, int64_t side_row_bytes,
    uint8_t* __restrict__ side_dst, int32_t chunks, int64_t n, int32_t group) {
    using T = typename Vec<V>::T;
    int64_t t, chunk;
    if constexpr (SV > 0) {
        const uint32_t per = (uint32_t)group * (uint32_t)chunks + 1;
        const uint32_t g = blockIdx.x / per;
        const uint32_t w = blockIdx.x - g * per;
        if (w == per - 1) {
            copy_side_rows<typename Vec<SV>::T, P>(side_src, side_row_bytes, side_row_bytes / SV,
                                                   (int64_t)g * group, group, n, output_perm,
                                                   topk, side_dst, num_dst_rows);
            return;
        }
        t = (int64_t)g * group + w / (uint32_t)chunks;
        chunk = w % (uint32_t)chunks;
        if (t >= n) return;
    } else {
        t = chunk_row(chunks, chunk);
    }
    const int64_t c = chunk * blockDim.x + threadIdx.x;
    copy_vector_to<T, P>(reinterpret_cast<const T*>(src + t * row_bytes), c, row_bytes / V, dst,
                         row_bytes, output_perm + t * topk, topk, num_dst_rows);
}

int vec_width(int64_t row_bytes, const void* a, const void* b) {
    const uint64_t bits = (uint64_t)row_bytes | (uint64_t)(uintptr_t)a | (uint64_t)(uintptr_t)b;
    for (int v = 16; v > 1; v >>= 1)
        if ((bits & (uint64_t)(v - 1)) == 0) return v;
    return 1;
}

template <int V, int P>
void launch_dispatch_v(dim3 grid, dim3 block, size_t lds, int32_t chunks, int side_vec,
                       const uint8_t* s, int64_t row_bytes, int32_t topk,
                       const int32_t* output_perm, uint8_t* d, int64_t num_dst_rows,
                       const uint8_t* ss, int64_t side_row_bytes, uint8_t* sd, int64_t n,
                       int32_t group, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
    switch (side_vec) {
    case 0: launch_kernel(dispatch_rows_kernel<V, 0, P>, grid, block, lds, stream, e0, e1, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, chunks, n, group); break;
    case 16: launch_kernel(dispatch_rows_kernel<V, 16, P>, grid, block, lds, stream, e0, e1, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, chunks, n, group); break;
    case 4: launch_kernel(dispatch_rows_kernel<V, 4, P>, grid, block, lds, stream, e0, e1, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, chunks, n, group); break;
    default: launch_kernel(dispatch_rows_kernel<V, 1, P>, grid, block, lds, stream, e0, e1, s, row_bytes, topk, output_perm, d, num_dst_rows, ss, side_row_bytes, sd, chunks, n, group); break;
    }
}

}  // namespace

hipError_t launch_shuffle_rows(const void* src, int64_t num_src_rows, int64_t row_bytes,
                               const int32_t* dst2src, int64_t num_dst_rows, void* dst,
                               hipStream_t stream) {
    if (num_dst_rows == 0) return hipSuccess;
    const int v = vec_width(row_bytes, src, dst);
    const RowShape sh = row_shape(row_bytes / v, kRowThreads);
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    return for_row_batches(num_dst_rows, sh, [&](int64_t r0, int64_t, dim3 grid, dim3 block,
                                                 hipEvent_t e0, hipEvent_t e1) {
        const int32_t* m = dst2src + r0;
        uint8_t* dr = d + r0 * row_bytes;
        switch (v) {
        case 16: launch_kernel(shuffle_rows_kernel<16>, grid, block, 0, stream, e0, e1, s, num_src_rows, row_bytes, m, dr, sh.chunks); break;
        case 8: launch_kernel(shuffle_rows_kernel<8>, grid, block, 0, stream, e0, e1, s, num_src_rows, row_bytes, m, dr, sh.chunks); break;
        case 4: launch_kernel(shuffle_rows_kernel<4>, grid, block, 0, stream, e0, e1, s, num_src_rows, row_bytes, m, dr, sh.chunks); break;
        case 2: launch_kernel(shuffle_rows_kernel<2>, grid, block, 0, stream, e0, e1, s, num_src_rows, row_bytes, m, dr, sh.chunks); break;
        default: launch_kernel(shuffle_rows_kernel<1>, grid, block, 0, stream, e0, e1, s, num_src_rows, row_bytes, m, dr, sh.chunks); break;
        }
    });
}

hipError_t launch_dispatch_rows(const void* src, int64_t num_tokens, int32_t topk,
                                int64_t row_bytes, const int32_t* output_perm, void* dst,
                                int64_t num_dst_rows, const void* side_src,
                                int64_t side_row_bytes, void* side_dst, hipStream_t stream,
                                hipEvent_t start_event, hipEvent_t stop_event) {
    if (num_tokens == 0) return hipSuccess;
    const int v = vec_width(row_bytes, src, dst);
    int side_vec = 0;
    if (side_src != nullptr) {
        const int sv = vec_width(side_row_bytes, side_src, side_dst);
        side_vec = sv >= 16 ? 16 : sv >= 4 ? 4 : 1;
    }
    RowShape sh = row_shape(row_bytes / v, kRowThreads);
    // Side rows: `group` tokens share one side workgroup (as many whole side
    // rows as it has threads, at least one).  A launch of n tokens then has
    // ceil(n / group) * (group * chunks + 1) workgroups, at most
    // n * (chunks + 1) when n is a multiple of group, which every batch but
    // the last is.
    int32_t group = 1;
    if (side_vec != 0) {
        const int64_t ns = side_row_bytes / side_vec;
        group = ns <= sh.threads ? (int32_t)(sh.threads / ns) : 1;
        int64_t rows = ((int64_t)1 << 31) / ((int64_t)(sh.chunks + 1) * sh.threads);
        if (rows < 1) rows = 1;
        if (group > rows) group = (int32_t)rows;
        sh.rows_per_launch = rows - rows % group;
    }
    const bool keep = dispatch_store_policy(num_tokens * (row_bytes + side_row_bytes)) == kKeep;
    const size_t lds = !keep && row_bytes >= kWideRowBytes ? kDispatchLdsWide : kDispatchLds;
    const uint8_t* s = static_cast<const uint8_t*>(src);
    uint8_t* d = static_cast<uint8_t*>(dst);
    const uint8_t* ss = static_cast<const uint8_t*>(side_src);
    uint8_t* sd = static_cast<uint8_t*>(side_dst);
    return for_row_batches(num_tokens, sh, [&](int64_t t0, int64_t n, dim3 grid, dim3 block,
                                               hipEvent_t e0, hipEvent_t e1) {
        if (side_vec != 0)
            grid.x = (unsigned)((n + group - 1) / group * ((int64_t)group * sh.chunks + 1));
        const uint8_t* st = s + t0 * row_bytes;
        const int32_t* pt = output_perm + t0 * topk;
        const uint8_t* sst = ss ? ss + t0 * side_row_bytes : nullptr;
        switch (v) {
        case 16:
            if (keep) launch_dispatch_v<16, kKeep>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1);
            else launch_dispatch_v<16, kStream>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1);
            break;
        case 8: launch_dispatch_v<8, kStream>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1); break;
        case 4: launch_dispatch_v<4, kStream>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1); break;
        case 2: launch_dispatch_v<2, kStream>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1); break;
        default: launch_dispatch_v<1, kStream>(grid, block, lds, sh.chunks, side_vec, st, row_bytes, topk, pt, d, num_dst_rows, sst, side_row_bytes, sd, n, group, stream, e0, e1); break;
        }
    }, start_event, stop_event);
}

}  // namespace mxmoe
