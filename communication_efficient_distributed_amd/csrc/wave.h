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

// Cross-lane steps through DPP (data-parallel primitives: a VALU operand
// taken from another lane of the same wavefront) rather than ds_bpermute,
// which is an LDS round trip per step.  GFX9 controls: row_shr:n shifts
// within each row of 16 lanes; row_bcast:15 / row_bcast:31 feed lane 15 / 31
// to the rows after it.  Lanes whose source falls outside the row, or whose
// row is masked off, take 0, the identity of both + and max on uint32.
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive scan over the 64 lanes (lane l gets op over lanes 0..l): four
// shift steps within each row of 16, then two broadcasts across rows.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t v, Op op) {
    v = op(v, dpp_or_zero<kRowShr1, 0xf>(v));
    v = op(v, dpp_or_zero<kRowShr2, 0xf>(v));
    v = op(v, dpp_or_zero<kRowShr4, 0xf>(v));
    v = op(v, dpp_or_zero<kRowShr8, 0xf>(v));
    v = op(v, dpp_or_zero<kRowBcast15, 0xa>(v));
    v = op(v, dpp_or_zero<kRowBcast31, 0xc>(v));
    return v;
}

// Inclusive prefix sum over lanes: lane l gets the sum of v over lanes <= l.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
    return wave_scan(v, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive suffix sum over lanes: lane l gets the sum of v over lanes >= l.
__device__ __forceinline__ uint32_t wave_suffix_sum(uint32_t v) {
    const uint32_t incl = wave_prefix_sum(v);
    return read_lane(incl, kWave - 1) - incl + v;
}

// Maximum over the wavefront, the same (wave-uniform) value in every lane.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    return read_lane(wave_scan(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; }), kWave - 1);
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
