// validate.hip -- well-formedness of received chunk records.
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

__global__ __launch_bounds__(kWave) void validate_kernel(PeerTable peers, int64_t n_chunks, uint8_t* flags) {
    const int p = (int)blockIdx.y;
    const int64_t c = (int64_t)blockIdx.x * kWave + (int64_t)threadIdx.x;
    if (c >= n_chunks) return;
    const uint8_t* rec = peers.payload[p] + (size_t)c * SL_PAYLOAD_BYTES;
    uint32_t w[kIndexWords];
#pragma unroll
    for (int q = 0; q < kIndexWords / 4; ++q) {
        const v4u v = load_global16(rec + 16 * q);
        w[4 * q + 0] = v.x;
        w[4 * q + 1] = v.y;
        w[4 * q + 2] = v.z;
        w[4 * q + 3] = v.w;
    }
    const float s = peers.scales[p][c];
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
    flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)f;
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

}  // namespace sl
