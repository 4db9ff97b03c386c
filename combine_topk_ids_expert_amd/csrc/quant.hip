// Dispatch with FP8 quantization on the way: every bf16 token row is cut into
// 1 x 128 groups, each group quantized to OCP e4m3fn with one fp32 scale,
// and the codes and scales are written to the token's k dispatched rows (the
// input quantization the TensorRT-LLM page "Enable CuteDSL MoE with Large EP"
// runs before its MoE, fused into the row scatter; the 1 x 128 block scales
// of the sglang prepare_moe_input page's FP8 path).
//
// Per group: amax = max |x|, scale = amax / 448 (1 for an all-zero group),
// code = e4m3fn(x / scale) rounded to nearest even and saturated at 448.
// The division is the IEEE one (hipcc's default correctly rounded fp32
// division), so the codes do not depend on launch shapes.
//
// A workgroup holds one token row, or a chunk of at most 1024 threads of a
// longer one (the chunks of a row are neighbours in the grid), with about 21
// waves per CU.  Each thread
// owns 16 consecutive elements: two 16-byte loads, and one 16-byte store of
// codes per destination through store16 with the non-temporal,
// system-coherent policy at every size: 11% faster than a plain
// non-temporal store on MI355X at T = 4096, and 3% faster than the
// allocating policy the row dispatch switches to for sources larger than the
// Infinity Cache (946 against 974 us at T = 65536, H = 7168).
// 8 threads form a group, whose amax is reduced with lane shuffles inside the
// wave.  A wave covers 8 groups; their scales are gathered into lanes 0..7 so
// each destination gets one contiguous 32-byte scale store per wave.
#include "device_common.h"
#include "launch.h"

namespace mxmoe {
namespace {

constexpr int kGroupElems = 128;
constexpr int kElemsPerThread = 16;
constexpr int kThreadsPerGroup = kGroupElems / kElemsPerThread;   // 8
constexpr int kGroupsPerWave = kWave / kThreadsPerGroup;          // 8
// Workgroup width limit: a row of up to 16384 elements is one workgroup (448
// threads at 7168).  Chunks of 64 to 256 threads, which suit the plain row
// copies, made this kernel 1-10% slower on MI355X.
#ifndef MXMOE_QUANT_THREADS
#define MXMOE_QUANT_THREADS 1024
#endif
constexpr int kQuantThreads = MXMOE_QUANT_THREADS;
static_assert(kQuantThreads % kWave == 0 && kQuantThreads <= 1024, "whole waves, at most 1024");

// LDS reserved per workgroup so that about 21 waves share a CU (3 workgroups
// of the 7-wave rows of H = 7168, where the registers allow 4): 56.6 -> 55.6
// us at T = 4096, 104 -> 100.9 us at K-hot T = 8192 and 975 -> 954 us at T =
// 65536 on MI355X.  Chunks of 64 to 256 threads were slower at every cap
// tried.  The reservation stays within the 64 KiB a launch may ask for.
constexpr int kQuantWavesPerCu = 21;

size_t quant_lds(int threads) {
    const size_t waves = (size_t)(threads / kWave);
    const size_t b = kLdsBytesPerCu * waves / kQuantWavesPerCu / 512 * 512;
    return b < 64 * 1024 ? b : 64 * 1024;
}


// Four binary32 values -> four OCP e4m3fn codes (byte i = value i): round to
// nearest even, saturate at 448 (0x7e with the sign), NaN -> 0x7f.  The
// rounding is gfx950's v_cvt_pk_fp8_f32, which gives exactly these codes for
// every finite |v| < 464 (checked against an integer encoder over all 2^32
// inputs on MI355X); above that it returns NaN, and NaN keeps its sign.  So
// each value is first clamped to [-448, 448] (values in (448, 464) round to
// 448 anyway, larger ones saturate there), and NaN inputs get 0x7f after.
__device__ __forceinline__ uint32_t e4m3_codes4(float v0, float v1, float v2, float v3) {
    const float c0 = fminf(fmaxf(v0, -448.0f), 448.0f), c1 = fminf(fmaxf(v1, -448.0f), 448.0f);
    const float c2 = fminf(fmaxf(v2, -448.0f), 448.0f), c3 = fminf(fmaxf(v3, -448.0f), 448.0f);
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, (int)c, true);
    const uint32_t nan = (v0 != v0 ? 0x000000ffu : 0u) | (v1 != v1 ? 0x0000ff00u : 0u) |
                         (v2 != v2 ? 0x00ff0000u : 0u) | (v3 != v3 ? 0xff000000u : 0u);
    return (c & ~nan) | (0x7f7f7f7fu & nan);
}

// Token t, elements [(chunk * blockDim.x + tid) * 16, +16).
__global__ __launch_bounds__(kQuantThreads) void dispatch_quant_fp8_kernel(
    const uint16_t* __restrict__ src, int64_t hidden, int32_t topk,
    const int32_t* __restrict__ output_perm, uint8_t* __restrict__ dst_q,
    float* __restrict__ dst_scales, int64_t num_dst_rows, int32_t chunks) {
    int64_t chunk;
    const int64_t t = chunk_row(chunks, chunk);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t col = (chunk * blockDim.x + threadIdx.x) * kElemsPerThread;
    const bool live = col < hidden;                    // whole groups: a group is live or not
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (live && MX_CAN_LOAD(src + t * hidden + col, 32, kSiteQuantSrc)) {
        const u32x4* p = reinterpret_cast<const u32x4*>(src + t * hidden + col);
        v0 = __builtin_nontemporal_load(p);
        v1 = __builtin_nontemporal_load(p + 1);
    }
    float x[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(v0[i] << 16);
        x[2 * i + 1] = __uint_as_float(v0[i] & 0xffff0000u);
        x[8 + 2 * i] = __uint_as_float(v1[i] << 16);
        x[8 + 2 * i + 1] = __uint_as_float(v1[i] & 0xffff0000u);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int d = 1; d < kThreadsPerGroup; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, kWave));
    const float scale = amax > 0.0f ? amax / 448.0f : 1.0f;
    u32x4 codes;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        codes[w] = e4m3_codes4(x[4 * w] / scale, x[4 * w + 1] / scale, x[4 * w + 2] / scale,
                               x[4 * w + 3] / scale);
    // Lanes 0..7 take the scales of this wave's 8 groups, in group order.
    const float wave_scale = __shfl(scale, (lane & (kGroupsPerWave - 1)) * kThreadsPerGroup, kWave);
    const int64_t groups = hidden / kGroupElems;
    const int64_t wave_group0 = (col - (int64_t)lane * kElemsPerThread) / kGroupElems;
    const bool scale_lane = lane < kGroupsPerWave && wave_group0 + lane < groups;
    const int32_t* rows = output_perm + t * topk;
    for (int j0 = 0; j0 < topk; j0 += kWave) {         // wave-uniform
        const int nj = topk - j0 < kWave ? topk - j0 : kWave;
        int my_r = -1;
        if (lane < nj && MX_CAN_LOAD(rows + j0 + lane, 4, kSiteQuantIndex)) my_r = rows[j0 + lane];
        if (my_r >= num_dst_rows) my_r = -1;
        for (int j = 0; j < nj; ++j) {
            const int32_t r = __builtin_amdgcn_readlane(my_r, j);
            if (r < 0) continue;
            if (live)
                store16<kStream>(codes, dst_q + (int64_t)r * hidden, hidden, col, kSiteQuantCodes);
            if (scale_lane &&
                MX_CAN_STORE(dst_scales + (int64_t)r * groups + wave_group0 + lane, 4, kSiteQuantScales))
                __builtin_nontemporal_store(wave_scale, dst_scales + (int64_t)r * groups + wave_group0 + lane);
        }
    }
}

}  // namespace

hipError_t launch_dispatch_quant_fp8(const void* src, int64_t num_tokens, int32_t topk,
                                     int64_t hidden, const int32_t* output_perm, void* dst_q,
                                     float* dst_scales, int64_t num_dst_rows,
                                     hipStream_t stream) {
    if (num_tokens == 0 || num_dst_rows == 0) return hipSuccess;
    const RowShape sh = row_shape(hidden / kElemsPerThread, kQuantThreads);
    const uint16_t* s = static_cast<const uint16_t*>(src);
    return for_row_batches(num_tokens, sh, [&](int64_t t0, int64_t, dim3 grid, dim3 block,
                                               hipEvent_t e0, hipEvent_t e1) {
        launch_kernel(dispatch_quant_fp8_kernel, grid, block, quant_lds(sh.threads), stream, e0, e1, s + t0 * hidden,
                      hidden, topk, output_perm + t0 * topk, static_cast<uint8_t*>(dst_q),
                      dst_scales, num_dst_rows, sh.chunks);
    });
}

}  // namespace mxmoe
