// Device-side helpers shared by the mxmoe HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxmoe {

constexpr int kWave = 64;

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

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
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
