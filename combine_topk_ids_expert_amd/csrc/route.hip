// Routing metadata for MoE dispatch: tokens per expert, padded expert offsets,
// block-scale offsets, and the stable input / output permutations (the
// prepare_moe_input call of the sglang page "[jit_kernel] Add
// prepare_moe_input JIT kernels", section "Changes", item 1).
//
// The permutations are a stable counting sort of the flat picks i = t*k + j
// by expert id.  The picks are cut into tiles; each tile is one workgroup of
// 8 waves, and each wave owns a contiguous stretch of the tile.  A wave
// counts its picks per expert into its private LDS row with an LDS atomic
// per pick.  To place them, 64 picks at a time, lanes holding the same
// expert find each other with one ballot per id bit (match_key); every
// lane's rank among equal ids is the popcount of matching lanes below it,
// and the lowest such lane advances the wave's cursor for the expert.  Since
// the wave stretches, the 64-pick groups and the lanes are each walked in
// ascending pick order, base(wave, expert) + rank is the stable position.
//
//   small inputs (up to 1024 picks, or 2048 with little padding, where it
//                measured faster): one workgroup counts, scans and scatters
//                (one launch);
//   medium inputs (up to 8192 picks): one launch of one workgroup per tile;
//                every workgroup counts every pick itself (totals, and the
//                picks before its tile), then places its tile's picks;
//   larger inputs, two launches:
//     count   -- one workgroup per tile writes the tile's count of every
//                expert to the workspace, expert-major ([E][tiles]);
//     scatter -- every workgroup requests its tile's ids, then the whole
//                count table (a few lanes per expert row, 16-byte loads
//                issued together), recounts its tile per wave while the
//                table is in flight, adds each row's partial sums with DPP,
//                scans the padded totals over experts itself, takes its
//                tile's base per expert and writes both permutations;
//                workgroup 0 writes the offsets and sizes.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kBatch = 8;                 // 64-pick groups loaded per round
constexpr int kMaxE = 1024;
constexpr int kTableBatch = 8;            // 16-byte count-table loads in flight per lane

#ifndef MXMOE_FUSED_MAX
#define MXMOE_FUSED_MAX 2048
#endif
#ifndef MXMOE_FUSED_ALWAYS
#define MXMOE_FUSED_ALWAYS 1024
#endif
#ifndef MXMOE_MAX_TILES
#define MXMOE_MAX_TILES 128
#endif
// Single-launch path: always up to kFusedAlways picks; up to kFusedMax when
// input_permutation is at most twice the picks (little padding), since the
// one workgroup also writes every padding and unused entry.
constexpr int64_t kFusedMax = MXMOE_FUSED_MAX;
constexpr int64_t kFusedAlways = MXMOE_FUSED_ALWAYS < MXMOE_FUSED_MAX ? MXMOE_FUSED_ALWAYS : MXMOE_FUSED_MAX;
constexpr int64_t kMaxTiles = MXMOE_MAX_TILES;  // tiles of the two-launch path (at most)
static_assert(kMaxTiles >= 1 && kMaxTiles <= 128,
              "the count-table read covers rows of at most 32 16-byte vectors");
constexpr int64_t kTileQuantum = kRouteThreads; // tile sizes are multiples of this

// Every scatter workgroup reads the whole count table (tiles x E entries),
// while its own work grows with the picks of its tile.  Measured on MI355X:
// about 0.16 us per 1000 table entries, and about 1.6 us per 1024 picks of a
// tile once a wave's stretch needs more than one round.  So with many experts
// the tile count is capped near kTableBudget / E, but never so low that a
// tile passes kOneRoundTile picks (E = 1000, 32768 picks: 16 tiles, 13.7 us
// where 64 took 19.0 us).
#ifndef MXMOE_TABLE_BUDGET
#define MXMOE_TABLE_BUDGET 16384
#endif
constexpr int64_t kTableBudget = MXMOE_TABLE_BUDGET;
constexpr int64_t kOneRoundTile = (int64_t)kBatch * kWave * kRouteWaves;  // 4096

// Tile size of the two-launch path: the smallest multiple of kTileQuantum
// that covers n picks in at most max_tiles(n, E) tiles.
__host__ __device__ inline int64_t max_tiles(int64_t n, int E) {
    int64_t mt = E > 0 && kTableBudget / E < kMaxTiles ? kTableBudget / E : kMaxTiles;
    const int64_t floor_tiles = (n + kOneRoundTile - 1) / kOneRoundTile;
    if (mt < floor_tiles) mt = floor_tiles;
    if (mt > kMaxTiles) mt = kMaxTiles;
    return mt < 1 ? 1 : mt;
}

__host__ __device__ inline int64_t tile_picks(int64_t n, int E) {
    const int64_t mt = max_tiles(n, E);
    int64_t per = (n + mt - 1) / mt;
    per = (per + kTileQuantum - 1) / kTileQuantum * kTileQuantum;
    return per < kTileQuantum ? kTileQuantum : per;
}

struct Shape {
    int64_t n;        // picks
    int E, nbits, k;
    int32_t id_offset;
    bool expanded;    // input_perm holds i instead of i / k
};

__device__ __forceinline__ int round_up_i(int v, int a) { return (v + a - 1) / a * a; }

// This wave's stretch [w0, w1) of the tile [t0, t1): equal stretches of a
// multiple of 64 picks, in wave order.
__device__ __forceinline__ void wave_stretch(int64_t t0, int64_t t1, int wave, int64_t& w0,
                                             int64_t& w1) {
    const int64_t per = ((t1 - t0 + kRouteWaves * kWave - 1) / (kRouteWaves * kWave)) * kWave;
    w0 = t0 + per * wave;
    w1 = w0 + per < t1 ? w0 + per : t1;
    if (w0 > t1) w0 = t1;
}

// One round of up to kBatch 64-pick groups starting at g0, keys loaded.
// Groups wholly past w1 are skipped (a wave-uniform test).  Inside a group,
// lanes past w1 load the stretch's last id instead of branching around the
// load, so all loads are issued before the first wait (a load under a
// per-lane branch gets its own wait and the round would cost kBatch
// latencies); their keys are then set to -1.
//
// Split in two so a caller can issue the loads early and convert later:
// load_raw issues the loads, raw_to_keys turns the ids into keys (a key is
// the id minus id_offset, or -1 past w1 and outside [0, E)).
template <typename IdT>
__device__ __forceinline__ void load_raw(const IdT* ids, int64_t g0, int64_t w1,
                                         IdT (&v)[kBatch]) {
    const int lane = lane_id();
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        const int64_t i = g0 + b * kWave + lane;
        const IdT* p = ids + (i < w1 ? i : w1 - 1);
        v[b] = g0 + b * kWave < w1 && MX_CAN_LOAD(p, sizeof(IdT), kSiteIds) ? *p : IdT(0);
    }
}

template <typename IdT>
__device__ __forceinline__ void raw_to_keys(const IdT (&v)[kBatch], int64_t g0, int64_t w1, int E,
                                            int32_t id_offset, int (&key)[kBatch]) {
    const int lane = lane_id();
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        const int64_t i = g0 + b * kWave + lane;
        const int64_t x = (int64_t)v[b] - id_offset;
        key[b] = (i < w1 && x >= 0 && x < E) ? (int)x : -1;
    }
}

template <typename IdT>
__device__ __forceinline__ void load_keys(const IdT* ids, int64_t g0, int64_t w1, int E,
                                          int32_t id_offset, int (&key)[kBatch]) {
    IdT v[kBatch];
    load_raw(ids, g0, w1, v);
    raw_to_keys(v, g0, w1, E, id_offset, key);
}

// Count a round of keys per expert into this wave's LDS row.  Counting
// needs no ranks, so every lane adds 1 with an LDS atomic (the row is the
// wave's own; the atomic only resolves lanes of one instruction that hold
// the same key): one instruction per 64 picks where matching needs a
// ballot per id bit.  Groups wholly past w1 hold no keys and are skipped.
__device__ __forceinline__ void count_keys(const int (&key)[kBatch], int64_t g0, int64_t w1,
                                           const Shape& s, int* row) {
    (void)s;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        if (g0 + b * kWave >= w1) break;                // wave-uniform
        if (key[b] >= 0 && MX_IN_RANGE(key[b], s.E, kSiteLocal)) atomicAdd(&row[key[b]], 1);
    }
}

// Place a round of keys: row[e] holds the next free dispatched row of expert
// e for this wave on entry and is advanced as picks are placed (groups past
// w1 skipped as in count_keys).
// kLocal: outp is the workgroup's LDS copy of the output permutation (a
// workgroup that routes for itself only), and inp is not written.
template <bool kLocal = false>
__device__ __forceinline__ void scatter_keys(const int (&key)[kBatch], int64_t g0, int64_t w1,
                                             const Shape& s, int* row, int32_t* outp,
                                             int32_t* inp, int64_t inp_len) {
    const int lane = lane_id();
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
        if (g0 + b * kWave >= w1) break;                // wave-uniform
        const int64_t i = g0 + b * kWave + lane;
        const uint64_t m = match_key(key[b], s.nbits);
        const int rank = lanes_below(m);
        const bool key_ok = key[b] >= 0 && MX_IN_RANGE(key[b], s.E, kSiteLocal);
        if (key_ok) {
            const int r = row[key[b]] + rank;   // every lane reads before the update below
            if (kLocal ? MX_IN_RANGE(i, kFusedMax, kSiteLocal)
                       : MX_CAN_STORE(outp + i, 4, kSiteOutPerm))
                outp[i] = r;
            if (!kLocal && r < inp_len && MX_CAN_STORE(inp + r, 4, kSiteInPerm))
                inp[r] = s.expanded ? (int32_t)i : (int32_t)((uint32_t)i / (uint32_t)s.k);
        } else if (i < w1 && (kLocal ? MX_IN_RANGE(i, kFusedMax, kSiteLocal)
                                     : MX_CAN_STORE(outp + i, 4, kSiteOutPerm))) {
            outp[i] = -1;
        }
        if (key_ok && rank == 0) row[key[b]] += __popcll(m);
    }
}

// Count the valid picks of [w0, w1) per expert into this wave's LDS row.
template <typename IdT>
__device__ void count_stretch(const IdT* ids, int64_t w0, int64_t w1, const Shape& s,
                              int* row) {
    for (int64_t g0 = w0; g0 < w1; g0 += kBatch * kWave) {
        int key[kBatch];
        load_keys(ids, g0, w1, s.E, s.id_offset, key);
        count_keys(key, g0, w1, s, row);
    }
}

// Scatter the picks of [w0, w1) (see scatter_keys).
template <typename IdT>
__device__ void scatter_stretch(const IdT* ids, int64_t w0, int64_t w1, const Shape& s,
                                int* row, int32_t* outp, int32_t* inp, int64_t inp_len) {
    for (int64_t g0 = w0; g0 < w1; g0 += kBatch * kWave) {
        int key[kBatch];
        load_keys(ids, g0, w1, s.E, s.id_offset, key);
        scatter_keys(key, g0, w1, s, row, outp, inp, inp_len);
    }
}

// Exclusive scan over experts of the padded counts (row_align and
// blockscale_align) in one workgroup; writes expert_offsets, problem sizes
// and block-scale offsets, and leaves each segment start in off[e].
// Returns the padded row total R.
__device__ int scan_experts(const RouteArgs& a, const int* cnt, int* off, int* tmp,
                            bool write_meta) {
    const int E = a.num_experts;
    const int nt = blockDim.x, tid = threadIdx.x;
    const int per = (E + nt - 1) / nt;
    const int e0 = tid * per < E ? tid * per : E;
    const int e1 = e0 + per < E ? e0 + per : E;
    int sr = 0, sb = 0;
    for (int e = e0; e < e1; ++e) {
        sr += round_up_i(cnt[e], a.row_align);
        sb += round_up_i(cnt[e], a.bs_align);
    }
    const int ir = wave_inclusive_sum(sr), ib = wave_inclusive_sum(sb);
    const int wave = tid / kWave, nw = nt / kWave;
    if ((tid & (kWave - 1)) == kWave - 1) { tmp[wave] = ir; tmp[32 + wave] = ib; }
    __syncthreads();
    if (tid < kWave) {
        const int vr = tid < nw ? tmp[tid] : 0, vb = tid < nw ? tmp[32 + tid] : 0;
        const int cr = wave_inclusive_sum(vr), cb = wave_inclusive_sum(vb);
        if (tid < nw) { tmp[64 + tid] = cr - vr; tmp[96 + tid] = cb - vb; }
        if (tid == nw - 1) { tmp[128] = cr; }
    }
    __syncthreads();
    int xr = tmp[64 + wave] + ir - sr, xb = tmp[96 + wave] + ib - sb;
    if (!write_meta) {
        for (int e = e0; e < e1; ++e) {
            off[e] = xr;
            xr += round_up_i(cnt[e], a.row_align);
        }
        return tmp[128];
    }
    if (tid == 0) {
        if (a.expert_offsets && MX_CAN_STORE(a.expert_offsets, 4, kSiteMeta))
            a.expert_offsets[0] = 0;
        if (a.blockscale_offsets && MX_CAN_STORE(a.blockscale_offsets, 4, kSiteMeta))
            a.blockscale_offsets[0] = 0;
    }
    for (int e = e0; e < e1; ++e) {
        const int c = cnt[e];
        off[e] = xr;
        xr += round_up_i(c, a.row_align);
        xb += round_up_i(c, a.bs_align);
        if (a.expert_offsets && MX_CAN_STORE(a.expert_offsets + e + 1, 4, kSiteMeta))
            a.expert_offsets[e + 1] = xr;
        if (a.blockscale_offsets && MX_CAN_STORE(a.blockscale_offsets + e + 1, 4, kSiteMeta))
            a.blockscale_offsets[e + 1] = xb;
        if (a.problem_sizes1 && MX_CAN_STORE(a.problem_sizes1 + 3 * e, 12, kSiteMeta)) {
            a.problem_sizes1[3 * e] = c;
            a.problem_sizes1[3 * e + 1] = a.gemm[0];
            a.problem_sizes1[3 * e + 2] = a.gemm[1];
        }
        if (a.problem_sizes2 && MX_CAN_STORE(a.problem_sizes2 + 3 * e, 12, kSiteMeta)) {
            a.problem_sizes2[3 * e] = c;
            a.problem_sizes2[3 * e + 1] = a.gemm[2];
            a.problem_sizes2[3 * e + 2] = a.gemm[3];
        }
    }
    return tmp[128];
}

// -1 into the padding rows of every expert handled by this wave and into
// the rows past the last segment, [R, inp_len), strided over all threads.
// The wave's experts are first_wave, first_wave + wave_stride, ...; 64 of
// them at a time go one per lane (one LDS read covers them all, where a
// loop with a dependent LDS read per expert cost microseconds), and the
// padding rows of those that have any are written 64 rows per store.
__device__ void fill_unused_rows(const RouteArgs& a, const int* cnt, const int* off, int R,
                                 int first_wave, int wave_stride, int64_t first_thread,
                                 int64_t thread_stride) {
    const int lane = lane_id();
    for (int j0 = 0; first_wave + j0 * wave_stride < a.num_experts; j0 += kWave) {
        const int e = first_wave + (j0 + lane) * wave_stride;
        int r0 = 0, n = 0;
        if (e < a.num_experts) {
            const int c = cnt[e];
            r0 = off[e] + c;
            n = round_up_i(c, a.row_align) - c;
        }
        uint64_t todo = __ballot(n > 0);
        while (todo != 0ull) {                               // wave-uniform
            const int l = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int p0 = __builtin_amdgcn_readlane(r0, l), pn = __builtin_amdgcn_readlane(n, l);
            for (int q = lane; q < pn; q += kWave)
                if (MX_CAN_STORE(a.input_perm + (int64_t)p0 + q, 4, kSiteInPerm))
                    a.input_perm[(int64_t)p0 + q] = -1;
        }
    }
    for (int64_t r = R + first_thread; r < a.input_perm_len; r += thread_stride)
        if (MX_CAN_STORE(a.input_perm + r, 4, kSiteInPerm)) a.input_perm[r] = -1;
}

// Tile maps of the tile-padded sort: the tiles [off[e], off[e] + padded
// count) / row_align of every expert handled by this wave get the expert and
// its row limit off[e] + cnt[e]; tiles past R / row_align get -1; the first
// thread of the grid writes the totals.  A wave's experts are taken 64 at a
// time, one per lane, as in fill_unused_rows.
__device__ void fill_tiles(const RouteArgs& a, const int* cnt, const int* off, int R,
                           int first_wave, int wave_stride, int64_t first_thread,
                           int64_t thread_stride) {
    if (a.tile_group == nullptr) return;
    const int lane = lane_id();
    const int S = a.row_align;
    for (int j0 = 0; first_wave + j0 * wave_stride < a.num_experts; j0 += kWave) {
        const int e = first_wave + (j0 + lane) * wave_stride;
        int q0 = 0, nq = 0, lim = 0;
        if (e < a.num_experts) {
            const int c = cnt[e];
            q0 = off[e] / S;
            nq = (c + S - 1) / S;
            lim = off[e] + c;
        }
        uint64_t todo = __ballot(nq > 0);
        while (todo != 0ull) {                               // wave-uniform
            const int l = __builtin_ctzll(todo);
            todo &= todo - 1;
            const int p0 = __builtin_amdgcn_readlane(q0, l), pn = __builtin_amdgcn_readlane(nq, l);
            const int pl = __builtin_amdgcn_readlane(lim, l);
            const int pe = first_wave + (j0 + l) * wave_stride;
            for (int q = lane; q < pn; q += kWave) {
                if (MX_CAN_STORE(a.tile_group + (int64_t)p0 + q, 4, kSiteTiles))
                    a.tile_group[(int64_t)p0 + q] = pe;
                if (MX_CAN_STORE(a.tile_limit + (int64_t)p0 + q, 4, kSiteTiles))
                    a.tile_limit[(int64_t)p0 + q] = pl;
            }
        }
    }
    for (int64_t q = R / S + first_thread; q < a.max_tiles; q += thread_stride) {
        if (MX_CAN_STORE(a.tile_group + q, 4, kSiteTiles)) a.tile_group[q] = -1;
        if (MX_CAN_STORE(a.tile_limit + q, 4, kSiteTiles)) a.tile_limit[q] = -1;
    }
    if (first_thread == 0) {
        if (a.padded_total && MX_CAN_STORE(a.padded_total, 4, kSiteTiles)) a.padded_total[0] = R;
        if (a.tile_count && MX_CAN_STORE(a.tile_count, 4, kSiteTiles)) a.tile_count[0] = R / S;
    }
}

// ---- single workgroup: count, scan and scatter in one launch -----------------

// A wave's stretch is at most kFusedRounds rounds of picks, so its ids are
// loaded once, all at the start, and kept in registers for both passes.
constexpr int64_t kRoundPicks = (int64_t)kBatch * kWave;
constexpr int kFusedRounds =
    kFusedMax > kRoundPicks * kRouteWaves
        ? (int)((kFusedMax + kRoundPicks * kRouteWaves - 1) / (kRoundPicks * kRouteWaves))
        : 1;
static_assert(kFusedMax <= kFusedRounds * kRoundPicks * kRouteWaves,
              "single-launch routing keeps at most kFusedRounds rounds per wave");

// The single-workgroup routing.  kLocal: the workgroup routes only for
// itself and leaves the output permutation in lperm (LDS); otherwise it
// writes every metadata array.
template <typename IdT, bool kLocal>
__device__ __forceinline__ void fused_route(const RouteArgs& a, const Shape& s,
                                            int (&rows)[kRouteWaves][kMaxE], int* cnt, int* off,
                                            int* tmp, int* lperm) {
    const int tid = threadIdx.x, wave = tid / kWave;
    const IdT* ids = static_cast<const IdT*>(a.ids);
    int64_t w0, w1;
    wave_stretch(0, s.n, wave, w0, w1);
    IdT raw[kFusedRounds][kBatch];
#pragma unroll
    for (int r = 0; r < kFusedRounds; ++r) load_raw(ids, w0 + r * kRoundPicks, w1, raw[r]);

    for (int e = tid; e < s.E; e += kRouteThreads)
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] = 0;
    __syncthreads();
    int key[kFusedRounds][kBatch];
#pragma unroll
    for (int r = 0; r < kFusedRounds; ++r) {
        raw_to_keys(raw[r], w0 + r * kRoundPicks, w1, s.E, s.id_offset, key[r]);
        count_keys(key[r], w0 + r * kRoundPicks, w1, s, rows[wave]);
    }
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            const int c = rows[w][e];
            rows[w][e] = run;
            run += c;
        }
        cnt[e] = run;
    }
    __syncthreads();
    const int R = scan_experts(a, cnt, off, tmp, !kLocal);
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads)
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] += off[e];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kFusedRounds; ++r)
        scatter_keys<kLocal>(key[r], w0 + r * kRoundPicks, w1, s, rows[wave],
                             kLocal ? lperm : a.output_perm, a.input_perm, a.input_perm_len);
    if (!kLocal) {
        fill_unused_rows(a, cnt, off, R, wave, kRouteWaves, tid, kRouteThreads);
        fill_tiles(a, cnt, off, R, wave, kRouteWaves, tid, kRouteThreads);
    }
}

template <typename IdT>
__global__ __launch_bounds__(kRouteThreads) void route_fused_kernel(RouteArgs a, Shape s) {
    __shared__ int rows[kRouteWaves][kMaxE];
    __shared__ int cnt[kMaxE];
    __shared__ int off[kMaxE];
    __shared__ int tmp[160];
    fused_route<IdT, false>(a, s, rows, cnt, off, tmp, nullptr);
}

// Routing and dispatch in one launch, for inputs the single-workgroup
// routing takes: one workgroup per token and chunk of 512 16-byte vectors of
// its row.  Each workgroup requests its vector of the token row first, then
// runs the whole routing itself (the ids are at most a few KB) with the
// output permutation kept in LDS, and stores the vector to the token's k
// rows; workgroup 0, the first to start, also writes every metadata array.
// This saves a launch and a dependent trip through memory between routing
// and dispatch at decode-sized batches.
template <typename IdT, int P>
__global__ __launch_bounds__(kRouteThreads) void route_dispatch_kernel(
    RouteArgs a, Shape s, const uint8_t* __restrict__ src, int64_t row_bytes,
    uint8_t* __restrict__ dst, int64_t num_dst_rows, int32_t chunks) {
    __shared__ int rows[kRouteWaves][kMaxE];
    __shared__ int cnt[kMaxE];
    __shared__ int off[kMaxE];
    __shared__ int tmp[160];
    __shared__ int lperm[kFusedMax];
    int64_t chunk;
    const int64_t t = chunk_row(chunks, chunk);
    const int64_t nvec = row_bytes / 16;
    const int64_t c = chunk * kRouteThreads + threadIdx.x;
    const bool live = c < nvec;
    u32x4 v{0u, 0u, 0u, 0u};
    if (live && MX_CAN_LOAD(src + t * row_bytes + c * 16, 16, kSiteRowSrc))
        v = reinterpret_cast<const u32x4*>(src + t * row_bytes)[c];
    if (blockIdx.x == 0) {
        fused_route<IdT, false>(a, s, rows, cnt, off, tmp, nullptr);
        // This workgroup's own rows: read back what it wrote to output_perm
        // (the same workgroup, ordered by the barrier).
        __syncthreads();
        for (int j = threadIdx.x; j < s.k; j += kRouteThreads)
            if (MX_IN_RANGE(t * s.k + j, kFusedMax, kSiteLocal))
                lperm[t * s.k + j] = MX_CAN_LOAD(a.output_perm + t * s.k + j, 4, kSiteOutPerm)
                                         ? a.output_perm[t * s.k + j]
                                         : -1;
    } else {
        fused_route<IdT, true>(a, s, rows, cnt, off, tmp, lperm);
    }
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    for (int j0 = 0; j0 < s.k; j0 += kWave) {
        const int nj = s.k - j0 < kWave ? s.k - j0 : kWave;
        int my_r = -1;
        if (lane < nj && MX_IN_RANGE(t * s.k + j0 + lane, kFusedMax, kSiteLocal))
            my_r = lperm[t * s.k + j0 + lane];
        if (my_r >= num_dst_rows) my_r = -1;
        for (int j = 0; j < nj; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(my_r, j);
            if (r < 0 || !live) continue;
            store16<P>(v, dst + (int64_t)r * row_bytes, row_bytes, c * 16, kSiteRowDst);
        }
    }
}

// ---- one launch, every workgroup counting every pick ------------------------

#ifndef MXMOE_SPREAD_MAX
#define MXMOE_SPREAD_MAX 8192
#endif
// Picks up to which the medium path below replaces the two launches.  Every
// workgroup counts every pick, so its cost grows with the picks: measured on
// MI355X it saves 16-35% up to 8192 picks under uniform, K-hot, Zipf and
// one-expert routing and 4% with 8 experts (5.4-7.6 against 7.6-10.9 us back
// to back), about breaks even at 16384 and loses at 32768.
constexpr int64_t kSpreadMax = MXMOE_SPREAD_MAX;
static_assert(kSpreadMax == 0 || kSpreadMax >= kFusedMax,
              "the medium path starts where the single-workgroup path ends");

// Medium inputs: tiles as in the two-launch path, but each workgroup counts
// every pick itself (totals per expert, and the picks before its tile), so
// no count table passes between launches.  The picks outside the tile are
// strided over all threads, kSpreadBatch loads per thread in flight, and
// counted with workgroup-wide LDS atomics; the tile's own picks are counted
// per wave, placed as in route_scatter_kernel.
constexpr int kSpreadBatch = 8;

template <typename IdT>
__global__ __launch_bounds__(kRouteThreads) void route_spread_kernel(RouteArgs a, Shape s,
                                                                     int64_t tile, int tiles) {
    __shared__ int rows[kRouteWaves][kMaxE];
    __shared__ int cnt[kMaxE];
    __shared__ int pre[kMaxE];
    __shared__ int off[kMaxE];
    __shared__ int tmp[160];
    const int tid = threadIdx.x, wave = tid / kWave;
    const int b = blockIdx.x;
    const IdT* ids = static_cast<const IdT*>(a.ids);
    const int64_t t0 = (int64_t)b * tile;
    const int64_t t1 = t0 + tile < s.n ? t0 + tile : s.n;
    int64_t w0, w1;
    wave_stretch(t0, t1, wave, w0, w1);
    const bool one_round = w1 - w0 <= kBatch * kWave;
    IdT raw[kBatch];
    if (one_round) load_raw(ids, w0, w1, raw);
    for (int e = tid; e < s.E; e += kRouteThreads) {
        cnt[e] = 0;
        pre[e] = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] = 0;
    }
    __syncthreads();
    // Picks outside [t0, t1): thread tid takes i = tid + j * kRouteThreads.
    // Indices past n (or inside the tile) load the last pick and drop it, so
    // every batch issues all its loads before the first use.
    const int64_t outside = s.n - (t1 - t0);
    for (int64_t j0 = 0; j0 * kRouteThreads < outside; j0 += kSpreadBatch) {
        IdT v[kSpreadBatch];
        int64_t idx[kSpreadBatch];
#pragma unroll
        for (int u = 0; u < kSpreadBatch; ++u) {
            const int64_t q = (j0 + u) * kRouteThreads + tid;      // q-th pick outside the tile
            idx[u] = q < t0 ? q : q + (t1 - t0);
            const IdT* p = ids + (q < outside ? idx[u] : s.n - 1);
            v[u] = MX_CAN_LOAD(p, sizeof(IdT), kSiteIds) ? *p : IdT(0);
        }
        int key8[kSpreadBatch];
        bool one = true;
#pragma unroll
        for (int u = 0; u < kSpreadBatch; ++u) {
            const int64_t q = (j0 + u) * kRouteThreads + tid;
            const int64_t x = (int64_t)v[u] - s.id_offset;
            key8[u] = q < outside && x >= 0 && x < s.E ? (int)x : -1;
        }
        // A batch whose valid picks all hold one expert is added with one
        // atomic per total: with every pick on one expert, per-lane atomics
        // on one address would serialize across the whole workgroup.
        const int k0 = __builtin_amdgcn_readfirstlane(key8[0]);
#pragma unroll
        for (int u = 0; u < kSpreadBatch; ++u) one = one && (key8[u] == k0 || key8[u] < 0);
        if (__ballot(!one) == 0ull) {                    // wave-uniform
            if (k0 >= 0) {
                int all = 0, before = 0;
#pragma unroll
                for (int u = 0; u < kSpreadBatch; ++u) {
                    all += __popcll(__ballot(key8[u] == k0));
                    before += __popcll(__ballot(key8[u] == k0 && idx[u] < t0));
                }
                if (lane_id() == 0) {
                    atomicAdd(&cnt[k0], all);
                    if (before) atomicAdd(&pre[k0], before);
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kSpreadBatch; ++u) {
                if (key8[u] < 0) continue;
                atomicAdd(&cnt[key8[u]], 1);
                if (idx[u] < t0) atomicAdd(&pre[key8[u]], 1);
            }
        }
    }
    int key[kBatch];
    if (one_round) {
        raw_to_keys(raw, w0, w1, s.E, s.id_offset, key);
        count_keys(key, w0, w1, s, rows[wave]);
    } else count_stretch<IdT>(ids, w0, w1, s, rows[wave]);
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads) {
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            const int c = rows[w][e];
            rows[w][e] = run;
            run += c;
        }
        cnt[e] += run;
    }
    __syncthreads();
    const int R = scan_experts(a, cnt, off, tmp, b == 0);
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads)
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] += off[e] + pre[e];
    __syncthreads();
    if (one_round)
        scatter_keys(key, w0, w1, s, rows[wave], a.output_perm, a.input_perm, a.input_perm_len);
    else
        scatter_stretch<IdT>(ids, w0, w1, s, rows[wave], a.output_perm, a.input_perm,
                             a.input_perm_len);
    fill_unused_rows(a, cnt, off, R, b * kRouteWaves + wave, tiles * kRouteWaves,
                     (int64_t)b * kRouteThreads + tid, (int64_t)tiles * kRouteThreads);
    fill_tiles(a, cnt, off, R, b * kRouteWaves + wave, tiles * kRouteWaves,
               (int64_t)b * kRouteThreads + tid, (int64_t)tiles * kRouteThreads);
}

// ---- two-launch path -------------------------------------------------------

// Tile counts per expert, expert-major: workspace[e * stride + tile] with the
// row stride rounded up to 4 tiles (16 bytes).
template <typename IdT>
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(RouteArgs a, Shape s,
                                                                   int64_t tile, int tiles) {
    __shared__ int rows[kRouteWaves][kMaxE];
    const int tid = threadIdx.x, wave = tid / kWave;
    for (int e = tid; e < s.E; e += kRouteThreads)
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * tile;
    const int64_t t1 = t0 + tile < s.n ? t0 + tile : s.n;
    int64_t w0, w1;
    wave_stretch(t0, t1, wave, w0, w1);
    count_stretch<IdT>(static_cast<const IdT*>(a.ids), w0, w1, s, rows[wave]);
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads) {
        int sum = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) sum += rows[w][e];
        int32_t* slot = a.workspace + (int64_t)e * round_up_i(tiles, 4) + blockIdx.x;
        if (MX_CAN_STORE(slot, 4, kSiteTableStore)) *slot = sum;
    }
}

// kTwo: rows of more than 16 vectors (more than 64 tiles), two vectors per
// lane.  A template parameter so that every table load of a batch is issued
// unconditionally: the wait for the ids, requested before the table, can then
// count the table loads still in flight instead of waiting for all of them.
template <typename IdT, bool kTwo>
__global__ __launch_bounds__(kRouteThreads) void route_scatter_kernel(RouteArgs a, Shape s,
                                                                      int64_t tile, int tiles) {
    __shared__ int rows[kRouteWaves][kMaxE];
    __shared__ int cnt[kMaxE];
    __shared__ int off[kMaxE];
    __shared__ int pre[kMaxE];
    __shared__ int tmp[160];
    const int tid = threadIdx.x, wave = tid / kWave;
    const int b = blockIdx.x;
    const IdT* ids = static_cast<const IdT*>(a.ids);
    const int64_t t0 = (int64_t)b * tile;
    const int64_t t1 = t0 + tile < s.n ? t0 + tile : s.n;
    int64_t w0, w1;
    wave_stretch(t0, t1, wave, w0, w1);
    // A stretch of at most one round keeps its keys in registers for both
    // passes; they are requested first so their latency overlaps the table.
    const bool one_round = w1 - w0 <= kBatch * kWave;
    IdT raw[kBatch];
    if (one_round) load_raw(ids, w0, w1, raw);
    for (int e = tid; e < s.E; e += kRouteThreads)
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) rows[w][e] = 0;

    // Expert totals over all tiles and this tile's prefix.  A row of the count
    // table is q = stride / 4 16-byte vectors (at most 32, since tiles <= 128).
    // L lanes share a row (q rounded up to a power of two, at most 16), each
    // taking vectors sub and sub + L, so one load instruction of a wave reads
    // whole cache lines of 64 / L consecutive rows, where a row per lane would
    // touch 64 lines per instruction.  The loads of a batch are issued
    // together; each row's L partial sums are then added with DPP.
    const int stride = round_up_i(tiles, 4);
    const int q = stride / 4;
    int L = 1;
    while (L < q && L < 16) L <<= 1;
    constexpr bool two = kTwo;                        // q > L
    const int rpi = kWave / L;                        // rows per wave instruction
    const int lane = tid & (kWave - 1), sub = lane & (L - 1), slot = lane / L;
    const int iters = (s.E + kRouteWaves * rpi - 1) / (kRouteWaves * rpi);
    const int sub0 = sub < q ? sub : q - 1, sub1 = sub + L < q ? sub + L : q - 1;
    constexpr int kRowBatch = two ? kTableBatch / 2 : kTableBatch;   // rows per batch
    // Entry c of this lane's vectors holds tile g_c; it adds to the expert's
    // total iff g_c < tiles (a row's padding columns are never written) and to
    // this tile's prefix iff g_c < b.  Both tests depend on the lane alone, so
    // they become masks once, outside the table loop, which then costs one
    // AND and one add per entry and total.
    int key[kBatch];
    int mtot[8], mpre[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int g = c < 4 ? sub * 4 + c : (sub + L) * 4 + c - 4;
        mtot[c] = g < tiles ? -1 : 0;
        mpre[c] = g < b ? -1 : 0;
    }
    using Batch = u32x4[kRowBatch];
    auto issue = [&](int it0, Batch& v0, Batch& v1) {
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            const int e = ((it0 + u) * kRouteWaves + wave) * rpi + slot;
            const u32x4* row = reinterpret_cast<const u32x4*>(
                a.workspace + (int64_t)(e < s.E ? e : s.E - 1) * stride);
            // Rows past the last are loaded from row E - 1 and then dropped,
            // so the number of loads in flight does not depend on the data.
            const bool live = it0 + u < iters;           // wave-uniform
            const u32x4 x0 = MX_CAN_LOAD(row + sub0, 16, kSiteTableLoad)
                                 ? row[sub0]
                                 : u32x4{0u, 0u, 0u, 0u};
            v0[u] = live ? x0 : u32x4{0u, 0u, 0u, 0u};
            if constexpr (two) {
                const u32x4 x1 = MX_CAN_LOAD(row + sub1, 16, kSiteTableLoad)
                                     ? row[sub1]
                                     : u32x4{0u, 0u, 0u, 0u};
                v1[u] = live ? x1 : u32x4{0u, 0u, 0u, 0u};
            } else {
                v1[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto fold = [&](int it0, const Batch& v0, const Batch& v1) {
#pragma unroll
        for (int u = 0; u < kRowBatch; ++u) {
            if (it0 + u >= iters) break;                 // wave-uniform
            const int e = ((it0 + u) * kRouteWaves + wave) * rpi + slot;
            int tot = 0, before = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int x = (int)v0[u][c];
                tot += x & mtot[c];
                before += x & mpre[c];
            }
            if constexpr (two) {
#pragma unroll
                for (int c = 4; c < 8; ++c) {
                    const int x = (int)v1[u][c - 4];
                    tot += x & mtot[c];
                    before += x & mpre[c];
                }
            }
            tot = group_sum(tot, L);
            before = group_sum(before, L);
            if (sub == 0 && e < s.E) {
                cnt[e] = tot;
                pre[e] = before;
            }
        }
    };
    Batch v0, v1;
    issue(0, v0, v1);
    // The tile's own count per wave needs only the ids, which were requested
    // before the table and arrive first: it runs while the first batch of the
    // table is still in flight.
    __syncthreads();
    if (one_round) {
        raw_to_keys(raw, w0, w1, s.E, s.id_offset, key);
        count_keys(key, w0, w1, s, rows[wave]);
    } else count_stretch<IdT>(ids, w0, w1, s, rows[wave]);
    fold(0, v0, v1);
    for (int it0 = kRowBatch; it0 < iters; it0 += kRowBatch) {
        issue(it0, v0, v1);
        fold(it0, v0, v1);
    }
    __syncthreads();
    const int R = scan_experts(a, cnt, off, tmp, b == 0);
    __syncthreads();
    for (int e = tid; e < s.E; e += kRouteThreads) {
        int run = off[e] + pre[e];
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            const int c = rows[w][e];
            rows[w][e] = run;
            run += c;
        }
    }
    __syncthreads();
    if (one_round)
        scatter_keys(key, w0, w1, s, rows[wave], a.output_perm, a.input_perm, a.input_perm_len);
    else
        scatter_stretch<IdT>(ids, w0, w1, s, rows[wave], a.output_perm, a.input_perm,
                             a.input_perm_len);
    fill_unused_rows(a, cnt, off, R, b * kRouteWaves + wave, tiles * kRouteWaves,
                     (int64_t)b * kRouteThreads + tid, (int64_t)tiles * kRouteThreads);
    fill_tiles(a, cnt, off, R, b * kRouteWaves + wave, tiles * kRouteWaves,
               (int64_t)b * kRouteThreads + tid, (int64_t)tiles * kRouteThreads);
}

int id_bits(int E) { return E <= 1 ? 0 : 32 - __builtin_clz((unsigned)(E - 1)); }

// Inputs the single-workgroup routing takes.
bool single_launch(const RouteArgs& a) {
    return a.num_picks <= kFusedAlways ||
           (a.num_picks <= kFusedMax && a.input_perm_len <= 2 * a.num_picks);
}

Shape shape_of(const RouteArgs& a) {
    return Shape{a.num_picks, a.num_experts, id_bits(a.num_experts), a.topk, a.id_offset,
                 a.inp_expanded};
}

// Workgroups of route_dispatch_kernel at most: each one routes all picks on
// its own, so past about two per CU the repeated routing costs more than the
// launch it saves.
constexpr int64_t kMaxRouteDispatchGroups = 512;

template <typename IdT>
hipError_t launch_typed(const RouteArgs& a, hipStream_t stream, hipEvent_t start,
                        hipEvent_t stop) {
    const Shape s = shape_of(a);
    if (single_launch(a)) {
        launch_kernel(route_fused_kernel<IdT>, dim3(1), dim3(kRouteThreads), 0, stream, start,
                      stop, a, s);
        return hipGetLastError();
    }
    const int64_t tile = tile_picks(a.num_picks, a.num_experts);
    const int tiles = (int)((a.num_picks + tile - 1) / tile);
    if (a.num_picks <= kSpreadMax) {
        launch_kernel(route_spread_kernel<IdT>, dim3(tiles), dim3(kRouteThreads), 0, stream,
                      start, stop, a, s, tile, tiles);
        return hipGetLastError();
    }
    launch_kernel(route_count_kernel<IdT>, dim3(tiles), dim3(kRouteThreads), 0, stream, start,
                  nullptr, a, s, tile, tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool two = (tiles + 3) / 4 > 16;            // table rows of more than 16 vectors
    launch_kernel(two ? route_scatter_kernel<IdT, true> : route_scatter_kernel<IdT, false>,
                  dim3(tiles), dim3(kRouteThreads), 0, stream, nullptr, stop, a, s, tile, tiles);
    return hipGetLastError();
}

}  // namespace

bool route_dispatch_fusable(const RouteArgs& a, int64_t num_tokens, int64_t row_bytes,
                            const void* src, const void* dst) {
    if (num_tokens < 1 || !single_launch(a) || a.inp_expanded || a.tile_group != nullptr)
        return false;
    if (row_bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0)
        return false;
    const int64_t chunks = (row_bytes / 16 + kRouteThreads - 1) / kRouteThreads;
    return num_tokens * chunks <= kMaxRouteDispatchGroups;
}

hipError_t launch_route_dispatch(const RouteArgs& a, int64_t num_tokens, const void* src,
                                 int64_t row_bytes, void* dst, int64_t num_dst_rows,
                                 hipStream_t stream) {
    const Shape s = shape_of(a);
    const int32_t chunks = (int32_t)((row_bytes / 16 + kRouteThreads - 1) / kRouteThreads);
    const dim3 grid((unsigned)(num_tokens * chunks)), block(kRouteThreads);
    const uint8_t* sp = static_cast<const uint8_t*>(src);
    uint8_t* dp = static_cast<uint8_t*>(dst);
    if (a.ids64)
        hipLaunchKernelGGL((route_dispatch_kernel<int64_t, kStream>), grid, block, 0, stream, a,
                           s, sp, row_bytes, dp, num_dst_rows, chunks);
    else
        hipLaunchKernelGGL((route_dispatch_kernel<int32_t, kStream>), grid, block, 0, stream, a,
                           s, sp, row_bytes, dp, num_dst_rows, chunks);
    return hipGetLastError();
}

size_t route_workspace_bytes(int64_t num_picks, int32_t num_experts) {
    if (num_picks <= kFusedAlways || num_picks <= kSpreadMax) return 0;
    const int64_t tile = tile_picks(num_picks, num_experts);
    const int64_t tiles = (num_picks + tile - 1) / tile;
    return (size_t)((tiles + 3) / 4 * 4 * (int64_t)num_experts * (int64_t)sizeof(int32_t));
}

hipError_t launch_route(const RouteArgs& a, hipStream_t stream, hipEvent_t start_event,
                        hipEvent_t stop_event) {
    return a.ids64 ? launch_typed<int64_t>(a, stream, start_event, stop_event)
                   : launch_typed<int32_t>(a, stream, start_event, stop_event);
}

}  // namespace mxmoe
