// validate.hip -- well-formedness and per-peer statistics of received chunk
// records.
//
// Untrusted peers can send anything ("What the Blockchain Does (and Doesn't
// Do)" in "The Sparse Frontier: SparseLoCo and the Compression Math Behind
// Permissionless Pre-Training" notes that nothing on the chain checks the
// updates, and the authors' post on the arXiv:2603.08163 listing names
// integrity checks among the validator's duties).  This is the cheap,
// structural part of such a check; reading of "well-formed": the 64 indices
// are strictly increasing (so distinct) and the scale is finite and not
// negative.  flags[p][c] gets
//   bit 0  indices not strictly increasing
//   bit 1  scale not finite
//   bit 2  scale negative
//
// Per-peer statistics (reading of the same section's remark that a crafted
// sparse update stands out to anomaly detection): per peer, the records
// flagged as above, the records whose scale is +-0, the entries at the
// magnitude level (code bit 0), the entries with the sign bit (code bit 1),
// and the largest scale among records whose scale is finite and not negative.
// Every statistic is an integer count or a maximum, so the per-workgroup
// partial results combine with integer atomics in any order and the totals are
// the same on every run.
//
// Mapping: one lane per record, 64 records per wavefront, one grid row per
// peer.  A lane loads its record's 96 index bytes (six 16-byte loads; the
// lanes' records are 112 bytes apart, so every line is fetched once and the
// later loads hit L2) and unpacks the 64 12-bit fields with compile-time
// shifts.  (Staging the wavefront's 7 KiB of records through LDS with fully
// coalesced loads measured no faster.)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr int kIndexWords = SL_INDEX_BYTES / 4;  // 24

__device__ __forceinline__ v4u load_global16(const uint8_t* p) {
    typedef const __attribute__((address_space(1))) v4u global_v4u;
    return *(global_v4u*)(p);
}

// Field j of the little-endian LSB-first stream of 12-bit indices.
__device__ __forceinline__ uint32_t index_field(const uint32_t (&w)[kIndexWords], int j) {
    const int bit = SL_INDEX_BITS * j;
    const int k = bit >> 5;
    const int sh = bit & 31;
    uint32_t v = w[k] >> sh;
    if (sh + SL_INDEX_BITS > 32) v |= w[k + 1] << (32 - sh);
    return v & ((1u << SL_INDEX_BITS) - 1u);
}

// Flags of one record (bit 0 order, bit 1 non-finite scale, bit 2 negative
// scale) from its 24 index dwords and its scale.
__device__ __forceinline__ uint32_t record_flags(const uint32_t (&w)[kIndexWords], float s) {
    bool increasing = true;
    uint32_t prev = index_field(w, 0);
#pragma unroll
    for (int j = 1; j < SL_TOPK; ++j) {
        const uint32_t cur = index_field(w, j);
        increasing = increasing && cur > prev;
        prev = cur;
    }
    uint32_t f = increasing ? 0u : 1u;
    if ((__float_as_uint(s) & 0x7f800000u) == 0x7f800000u) f |= 2u;
    if (s < 0.0f) f |= 4u;
    return f;
}

__device__ __forceinline__ void load_indices(const uint8_t* rec, uint32_t (&w)[kIndexWords]) {
#pragma unroll
    for (int q = 0; q < kIndexWords / 4; ++q) {
        const v4u v = load_global16(rec + 16 * q);
        w[4 * q + 0] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
    }
}

__global__ __launch_bounds__(kWave) void validate_kernel(PeerTable peers, int64_t n_chunks, uint8_t* flags) {
    const int p = (int)blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kWave + (int64_t)threadIdx.x;
    if (c >= n_chunks) return;
    const uint8_t* rec = peers.payload[p] + (size_t)c * SL_PAYLOAD_BYTES;
    uint32_t w[kIndexWords];
    load_indices(rec, w);
    const uint32_t f = record_flags(w, peers.scales[p][c]);
    flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)f;
}

constexpr int kStatWaves = 4;
constexpr int kStatThreads = kWave * kStatWaves;

// counts (uint64[n_peers][4]) and the scale maxima (fp32 bit patterns,
// uint32[n_peers]) start from 0 before the statistics kernel adds to them.
__global__ __launch_bounds__(kStatThreads) void clear_stats_kernel(uint64_t* counts, uint32_t* scale_max,
                                                                   int32_t n_peers) {
    for (int i = (int)threadIdx.x; i < 4 * n_peers; i += kStatThreads) counts[i] = 0ull;
    for (int i = (int)threadIdx.x; i < n_peers; i += kStatThreads) scale_max[i] = 0u;
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, o, kWave);
    return v;
}

// Grid (G, n_peers).  Workgroup g of peer p takes records g*256 + t +
// k*G*256; flags (if given) as validate_kernel writes them.
__global__ __launch_bounds__(kStatThreads) void stats_kernel(PeerTable peers, int64_t n_chunks, uint8_t* flags,
                                                             uint64_t* counts, uint32_t* scale_max) {
    __shared__ uint64_t part[kStatWaves][4];
    __shared__ uint32_t part_max[kStatWaves];
    const int p = (int)blockIdx.y;
    const int tid = (int)threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kStatThreads;
    uint32_t bad = 0, zero = 0, mag = 0, neg = 0, mx = 0;
#pragma unroll 2
    for (int64_t c = (int64_t)blockIdx.x * kStatThreads + tid; c < n_chunks; c += stride) {
        const uint8_t* rec = peers.payload[p] + (size_t)c * SL_PAYLOAD_BYTES;
        uint32_t w[kIndexWords];
        load_indices(rec, w);
        const v4u cw = load_global16(rec + SL_INDEX_BYTES);
        const float s = peers.scales[p][c];
        const uint32_t f = record_flags(w, s);
        if (flags) flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)f;
        bad += f ? 1u : 0u;
        zero += s == 0.0f ? 1u : 0u;
        // Code j sits at bits [2j, 2j+2): bit 0 (magnitude) on even bit
        // positions, bit 1 (sign) on odd ones.
        mag += __popc(cw.x & 0x55555555u) + __popc(cw.y & 0x55555555u) + __popc(cw.z & 0x55555555u) +
               __popc(cw.w & 0x55555555u);
        neg += __popc(cw.x & 0xaaaaaaaau) + __popc(cw.y & 0xaaaaaaaau) + __popc(cw.z & 0xaaaaaaaau) +
               __popc(cw.w & 0xaaaaaaaau);
        // For non-negative finite floats (and -0 mapped to +0) the bit
        // pattern orders like the value.
        const uint32_t key = __float_as_uint(s) & 0x7fffffffu;
        if ((f & 6u) == 0u && key > mx) mx = key;
    }
    const int wv = tid >> 6;
    const uint64_t t0 = wave_sum64(bad), t1 = wave_sum64(zero), t2 = wave_sum64(mag), t3 = wave_sum64(neg);
    const uint32_t tm = wave_max(mx);
    if ((tid & (kWave - 1)) == 0) {
        part[wv][0] = t0;
        part[wv][1] = t1;
        part[wv][2] = t2;
        part[wv][3] = t3;
        part_max[wv] = tm;
    }
    __syncthreads();
    // Lanes 0..3 add one count each, lane 4 the maximum: vector atomics,
    // skipped when there is nothing to add.
    if (tid < 5) {
        if (tid < 4) {
            uint64_t v = 0;
            for (int i = 0; i < kStatWaves; ++i) v += part[i][tid];
            if (v) atomicAdd((unsigned long long*)&counts[4 * (size_t)p + tid], (unsigned long long)v);
        } else {
            uint32_t m = 0;
            for (int i = 0; i < kStatWaves; ++i) m = part_max[i] > m ? part_max[i] : m;
            if (m) atomicMax(&scale_max[p], m);
        }
    }
}

}  // namespace

hipError_t launch_validate(const PeerTable& peers, int32_t n_peers, int64_t n_chunks, uint8_t* flags,
                           hipStream_t stream) {
    PeerTable t = peers;
    void* args[] = {(void*)&t, (void*)&n_chunks, (void*)&flags};
    const unsigned gx = (unsigned)((n_chunks + kWave - 1) / kWave);
    return hipLaunchKernel(reinterpret_cast<const void*>(&validate_kernel), dim3(gx, (unsigned)n_peers),
                           dim3(kWave), args, 0, stream);
}

hipError_t launch_peer_stats(const PeerTable& peers, int32_t n_peers, int64_t n_chunks, uint8_t* flags,
                             int64_t* counts, float* scale_max, hipStream_t stream) {
    uint64_t* cnt = reinterpret_cast<uint64_t*>(counts);
    uint32_t* mx = reinterpret_cast<uint32_t*>(scale_max);
    void* cargs[] = {(void*)&cnt, (void*)&mx, (void*)&n_peers};
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&clear_stats_kernel), dim3(1),
                                   dim3(kStatThreads), cargs, 0, stream);
    if (e != hipSuccess || n_chunks == 0) return e;
    // About 1024 workgroups in all, each lane taking several records.  The
    // totals are device-scope atomics, which are slow across the 8 XCDs: with
    // 4096 or 8192 workgroups at 24 peers the pass took 50 or 64 us, with 256
    // to 2048 it took 31-33 us (loop unrolled by 2: 31 us).
    const int64_t per_peer = (1024 + n_peers - 1) / n_peers;
    const int64_t needed = (n_chunks + kStatThreads - 1) / kStatThreads;
    const unsigned gx = (unsigned)(needed < per_peer ? needed : per_peer);
    PeerTable t = peers;
    void* args[] = {(void*)&t, (void*)&n_chunks, (void*)&flags, (void*)&cnt, (void*)&mx};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stats_kernel), dim3(gx, (unsigned)n_peers),
                           dim3(kStatThreads), args, 0, stream);
}

}  // namespace sl
