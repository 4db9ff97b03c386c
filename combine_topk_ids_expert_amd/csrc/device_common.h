// Device-side helpers shared by the mxmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Launch shape of the row kernels (dispatch, combine, row shuffle, zeroing,
// quantize-on-dispatch): one workgroup per (row, column chunk), flattened
// into blockIdx.x with the chunk varying fastest, so the chunks of one row run
// next to each other.  Workgroups are at most `max_threads` wide (whole
// waves); the chunks of a row are as few as that allows, and as even.  Rows
// are launched in batches so that no launch holds more than 2^31 work-items.
struct RowShape {
    int32_t threads;          // workgroup width
    int32_t chunks;           // column chunks per row
    int64_t rows_per_launch;  // rows of one launch
};

inline RowShape row_shape(int64_t items, int64_t max_threads) {
    RowShape s;
    const int64_t chunks = (items + max_threads - 1) / max_threads;
    int64_t threads = (items + chunks - 1) / chunks;
    threads = (threads + kWave - 1) / kWave * kWave;
    s.threads = (int32_t)threads;
    s.chunks = (int32_t)chunks;
    s.rows_per_launch = ((int64_t)1 << 31) / (chunks * threads);
    return s;
}

// Occupancy cap through LDS.  A CU of gfx950 has 160 KiB of LDS, so a launch
// that reserves b bytes of dynamic LDS per workgroup, which the kernel never
// touches, places at most about 160 KiB / b of its workgroups on one CU (the
// exact count also depends on allocation granularity, so the reservations
// were chosen by measurement, at each kernel's constant).  The row kernels
// hold no LDS of their own and their registers allow 32 waves per CU; the
// scattered writes of the row dispatch, the gathers of the combine, the
// padding fill and the FP8 dispatch each ran faster on MI355X with fewer
// waves in flight per CU.  Kernels without a cap pass 0.
constexpr size_t kLdsBytesPerCu = 160 * 1024;

// Launches kernel<<<grid, block, lds_bytes, stream>>>(args...).  With a start
// or a stop event it goes through hipExtLaunchKernelGGL, which records the
// events with the kernel dispatch's own begin and end timestamps: the elapsed
// time between them is the kernel's execution, without the launch gap an
// event record queued on the stream adds.
template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                          hipStream_t stream, hipEvent_t start, hipEvent_t stop, Args... args) {
    if (start != nullptr || stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, start, stop, 0u,
                              static_cast<KArgs>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, static_cast<KArgs>(args)...);
}

// Launches launch(row0, rows, grid, block, ev_start, ev_stop) for consecutive
// batches of rows, stopping at the first launch error.  `start` goes with the
// first launch and `stop` with the last (both may be null).
template <typename F>
hipError_t for_row_batches(int64_t rows, const RowShape& s, F&& launch,
                           hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
    for (int64_t r0 = 0; r0 < rows; r0 += s.rows_per_launch) {
        const int64_t n = rows - r0 < s.rows_per_launch ? rows - r0 : s.rows_per_launch;
        launch(r0, n, dim3((unsigned)(n * s.chunks), 1, 1), dim3((unsigned)s.threads, 1, 1),
               r0 == 0 ? start : nullptr, r0 + n >= rows ? stop : nullptr);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Row (within the launch) and column chunk of this workgroup.
__device__ __forceinline__ int64_t chunk_row(int32_t chunks, int64_t& chunk) {
    const uint32_t b = blockIdx.x;
    const uint32_t r = b / (uint32_t)chunks;
    chunk = (int64_t)(b - r * (uint32_t)chunks);
    return (int64_t)r;
}

// Cache policies of store16 (gfx950 policy bits: sc0 = 1, nt = 2, sc1 = 16).
//   kStream  sc0 nt sc1: non-temporal, system-coherent.
//   kKeep    sc1: allocating in the caches, system-coherent.
// For the scattered write-once destination rows of the row dispatch, kStream
// measured 1.5-2% faster on MI355X than a plain non-temporal global store as
// long as the source rows fit in the 256 MB Infinity Cache; beyond that,
// kKeep was 1.6-2.6% faster (T = 24576 to 65536 rows of 14 KiB), and below
// it 12-14% slower, since the allocated destination lines evict the source
// rows.  kCacheResidentBytes is the source size up to which the row dispatch
// uses kStream, and the output size up to which the combine uses kKeep.
enum StorePolicy : int { kStream = 1 | 2 | 16, kKeep = 16 };
constexpr int64_t kCacheResidentBytes = (int64_t)256 << 20;

inline StorePolicy dispatch_store_policy(int64_t source_bytes) {
    return source_bytes > kCacheResidentBytes ? kKeep : kStream;
}

// ---- bounds-checked build ----------------------------------------------------
// Built with MXMOE_CHECKED defined (libmxmoe_checked.so), every global load
// and store of the kernels is first checked against the buffers of the call
// that launched it, which the C ABI writes into this translation unit's
// g_check_table before its launches.  An access that does not lie wholly
// inside one of them (or that stores into a read-only one) is counted in
// g_check_report and skipped, a load giving zeros, so the kernel still ends
// normally; the entry point then returns MX_ERR_OUT_OF_BOUNDS.  Indices into
// LDS arrays that come from data are checked against the array's length the
// same way.  In the normal build every check is the constant `true` and the
// kernels compile to the same code as without them.
enum CheckSite : int {
    kSiteIds = 1,          // routing: topk ids
    kSiteTableLoad,        // routing: count table, loads
    kSiteTableStore,       // routing: count table, stores
    kSiteOutPerm,          // routing: output permutation
    kSiteInPerm,           // routing: input permutation (scatter and unused rows)
    kSiteMeta,             // routing: offsets, problem sizes, block-scale offsets
    kSiteTiles,            // routing: tile maps and totals
    kSiteLocal,            // routing: LDS arrays indexed by data
    kSiteRowSrc,           // row copies: source vectors
    kSiteRowIndex,         // row copies: destination / source row indices
    kSiteRowDst,           // row copies: destination vectors
    kSiteCombineIndex,     // combine: row indices
    kSiteCombineFactor,    // combine: weights
    kSiteCombineY,         // combine: expert output rows
    kSiteCombineOut,       // combine: output rows
    kSiteZeroIndex,        // zeroing: permutation entries and expert offsets
    kSiteZeroRows,         // zeroing: zeroed rows
    kSiteQuantSrc,         // fp8 dispatch: source rows
    kSiteQuantIndex,       // fp8 dispatch: destination row indices
    kSiteQuantCodes,       // fp8 dispatch: code rows
    kSiteQuantScales,      // fp8 dispatch: scale rows
};

#ifdef MXMOE_CHECKED
struct CheckRange {
    uint64_t lo, hi;       // [lo, hi) in bytes
    uint32_t writable, pad;
};
constexpr int kMaxCheckRanges = 16;
struct CheckTable {
    uint32_t n, pad;
    CheckRange r[kMaxCheckRanges];
};
// [0] loads outside, [1] stores outside, [2] the address and [3] the site of
// the first access counted (site 0: none yet).
constexpr int kCheckReportWords = 4;

static __device__ CheckTable g_check_table;
static __device__ unsigned long long g_check_report[kCheckReportWords];

[[maybe_unused]] static __device__ __noinline__ bool check_access(uint64_t lo, uint64_t bytes, bool store, int site) {
    const uint32_t n = g_check_table.n < kMaxCheckRanges ? g_check_table.n : kMaxCheckRanges;
    for (uint32_t i = 0; i < n; ++i) {
        const CheckRange& r = g_check_table.r[i];
        if (lo >= r.lo && lo + bytes <= r.hi && (r.writable || !store)) return true;
    }
    atomicAdd(&g_check_report[store ? 1 : 0], 1ull);
    if (atomicCAS(&g_check_report[3], 0ull, (unsigned long long)site) == 0ull)
        atomicExch(&g_check_report[2], (unsigned long long)lo);
    return false;
}

[[maybe_unused]] static __device__ __noinline__ bool check_index(int64_t i, int64_t n, int site) {
    if (i >= 0 && i < n) return true;
    atomicAdd(&g_check_report[1], 1ull);
    if (atomicCAS(&g_check_report[3], 0ull, (unsigned long long)site) == 0ull)
        atomicExch(&g_check_report[2], (unsigned long long)i);
    return false;
}

#define MX_CAN_LOAD(p, bytes, site) \
    ::mxmoe::check_access((uint64_t)(uintptr_t)(p), (uint64_t)(bytes), false, (site))
#define MX_CAN_STORE(p, bytes, site) \
    ::mxmoe::check_access((uint64_t)(uintptr_t)(p), (uint64_t)(bytes), true, (site))
#define MX_IN_RANGE(i, n, site) ::mxmoe::check_index((int64_t)(i), (int64_t)(n), (site))

// Host side: the C ABI sets the table and collects the report of every
// translation unit that launches kernels, through the hooks each one
// registers at load time (a `static __device__` variable is one per
// translation unit).
struct CheckHooks {
    hipError_t (*set_table)(const CheckTable&);
    hipError_t (*take_report)(unsigned long long (&)[kCheckReportWords]);
};
int register_check_hooks(const CheckHooks& hooks);   // api.hip

namespace {
hipError_t set_check_table(const CheckTable& t) {
    return hipMemcpyToSymbol(HIP_SYMBOL(g_check_table), &t, sizeof(t));
}
hipError_t take_check_report(unsigned long long (&r)[kCheckReportWords]) {
    hipError_t e = hipMemcpyFromSymbol(r, HIP_SYMBOL(g_check_report), sizeof(r));
    if (e != hipSuccess) return e;
    static const unsigned long long zero[kCheckReportWords] = {};
    return hipMemcpyToSymbol(HIP_SYMBOL(g_check_report), zero, sizeof(zero));
}
const int g_check_hooks_registered =
    register_check_hooks(CheckHooks{&set_check_table, &take_check_report});
}  // namespace
#else
#define MX_CAN_LOAD(p, bytes, site) true
#define MX_CAN_STORE(p, bytes, site) true
#define MX_IN_RANGE(i, n, site) true
#endif

// 16-byte store of vector v at byte offset `off` of a row that starts at
// `row` (the row base wave-uniform, the offset per lane), through a raw
// buffer store with cache policy P.  The buffer's extent is the row, so a
// store past row_bytes would be dropped by the hardware; callers only store
// inside it.  0x00020000 is the gfx9 raw-buffer format word.
template <int P>
__device__ __forceinline__ void store16(u32x4 v, uint8_t* row, int64_t row_bytes, int64_t off,
                                        int site) {
    if (!MX_CAN_STORE(row + off, 16, site)) return;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(row, (short)0, (int)row_bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, P);
}

// Number of lanes below this one whose bit is set in `mask`.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ int lane_id() { return lanes_below(~0ull); }

// Mask of the lanes of this wave holding the same key as this lane.  Keys are
// in [0, 2^nbits); a negative key marks an inactive lane, which matches no
// one and gets 0.  One ballot per key bit: the lanes that agree with this
// lane on every bit are exactly the lanes with an equal key.  Must be
// reached by the whole wave (nbits uniform).
__device__ __forceinline__ uint64_t match_key(int key, int nbits) {
    uint64_t m = __ballot(key >= 0);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t ones = __ballot(bit);
        m &= bit ? ones : ~ones;
    }
    return key >= 0 ? m : 0ull;
}

// ---- lane arithmetic with DPP ----------------------------------------------
// Data-parallel-primitive operand modifiers move values between lanes in
// registers (no LDS round trip, unlike ds_bpermute behind __shfl*).  Control
// codes (GFX9 DPP): quad_perm is 0x00-0xff (two bits per lane of a quad),
// row_shr:n is 0x110 + n, row_mirror 0x140, row_half_mirror 0x141,
// row_bcast:15 0x142, row_bcast:31 0x143.  With old = 0 a lane whose source
// lies outside its row, or whose row is masked off, adds 0.
template <int Ctrl, int RowMask = 0xf>
__device__ __forceinline__ int dpp(int v) {
    return __builtin_amdgcn_update_dpp(0, v, Ctrl, RowMask, 0xf, false);
}

// Inclusive prefix sum across the wave: Hillis-Steele inside each row of 16
// lanes (row_shr 1, 2, 4, 8), then row 1 and row 3 add the last lane of the
// row before them (row_bcast:15), then rows 2 and 3 add lane 31
// (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += dpp<0x111>(v);
    v += dpp<0x112>(v);
    v += dpp<0x114>(v);
    v += dpp<0x118>(v);
    v += dpp<0x142, 0xa>(v);
    v += dpp<0x143, 0xc>(v);
    return v;
}

// Sum over aligned groups of L lanes (L a power of two, 1..16, wave-uniform);
// every lane of a group gets the group's sum.  Butterfly: lane ^ 1 and
// lane ^ 2 by quad_perm [1,0,3,2] and [2,3,0,1], then the two quads of a
// half-row swap (row_half_mirror) and the two half-rows of a row swap
// (row_mirror).
__device__ __forceinline__ int group_sum(int v, int L) {
    if (L >= 2) v += dpp<0xb1>(v);
    if (L >= 4) v += dpp<0x4e>(v);
    if (L >= 8) v += dpp<0x141>(v);
    if (L >= 16) v += dpp<0x140>(v);
    return v;
}

// ---- number formats --------------------------------------------------------

struct BF16 { using storage = uint16_t; };
struct F16 { using storage = uint16_t; };
struct F32 { using storage = float; };

__device__ __forceinline__ float to_f32(BF16, uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}
__device__ __forceinline__ float to_f32(F16, uint16_t h) {
    _Float16 x;
    __builtin_memcpy(&x, &h, 2);
    return (float)x;
}
__device__ __forceinline__ float to_f32(F32, float f) { return f; }

// Round to nearest even (the hardware conversions on gfx950).
__device__ __forceinline__ uint16_t from_f32(BF16, float f) {
    __bf16 b = (__bf16)f;
    uint16_t h;
    __builtin_memcpy(&h, &b, 2);
    return h;
}
__device__ __forceinline__ uint16_t from_f32(F16, float f) {
    _Float16 x = (_Float16)f;
    uint16_t h;
    __builtin_memcpy(&h, &x, 2);
    return h;
}
__device__ __forceinline__ float from_f32(F32, float f) { return f; }

}  // namespace mxmoe
