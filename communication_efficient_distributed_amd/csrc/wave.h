// wave.h -- wavefront (64-lane) primitives for gfx950 used by the kernels.
//
// Inside one wavefront LDS instructions execute in issue order, and wave_sync()
// keeps the compiler from moving LDS accesses across the point where lanes
// start reading what other lanes wrote.  Kernels whose wavefronts share LDS
// (the compressor's four wavefronts per chunk) use workgroup barriers and the
// workgroup-scope atomics below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sl {

constexpr int kWave = 64;

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_id() {
    return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// Number of set bits of mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint32_t read_lane(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        uint32_t y = (uint32_t)__shfl_xor((int)v, o, kWave);
        v = v > y ? v : y;
    }
    return v;
}

// Inclusive suffix sum over lanes: lane l gets sum of v over lanes >= l.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t y = (uint32_t)__shfl_down((int)v, o, kWave);
        if (lane + o < kWave) v += y;
    }
    return v;
}

// Inclusive prefix sum over lanes: lane l gets sum of v over lanes <= l.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        uint32_t y = (uint32_t)__shfl_up((int)v, o, kWave);
        if (lane >= o) v += y;
    }
    return v;
}

// LDS atomics at wavefront scope (only lanes of one wavefront touch a slice).
__device__ __forceinline__ void lds_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

__device__ __forceinline__ void lds_or(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
}

// LDS atomics at workgroup scope (several wavefronts update the same words;
// ordering against other accesses comes from the barriers around them).
__device__ __forceinline__ void block_lds_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void block_lds_or(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

}  // namespace sl
