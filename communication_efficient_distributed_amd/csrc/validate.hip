// validate.hip -- well-formedness of received chunk records.
//
// Untrusted peers can send anything ("What the Blockchain Does (and Doesn't
// Do)" in "The Sparse Frontier: SparseLoCo and the Compression Math Behind
// Permissionless Pre-Training" notes that nothing on the chain checks the
// updates, and the authors' post on the arXiv:2603.08163 listing names
// integrity checks among the validator's duties).  This is the cheap,
// structural part of such a check; reading of "well-formed": the 64 indices
// are strictly increasing (so distinct) and the scale is finite and not
// negative.  One wavefront per record; flags[c] gets
//   bit 0  indices not strictly increasing
//   bit 1  scale not finite
//   bit 2  scale negative
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "record.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

__global__ __launch_bounds__(kWave) void validate_kernel(const uint8_t* payload, const float* scales,
                                                         uint8_t* flags, int64_t n_chunks) {
    const int lane = (int)threadIdx.x;
    const int64_t chunk = (int64_t)blockIdx.x;
    if (chunk >= n_chunks) return;
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(payload + (size_t)chunk * SL_PAYLOAD_BYTES);
    const uint32_t idx = EntryPos(lane).read(rec) & 4095u;
    const uint32_t prev = (uint32_t)__shfl_up((int)idx, 1, kWave);
    const uint64_t bad_order = ballot(lane > 0 && idx <= prev);
    if (lane == 0) {
        const float s = scales[chunk];
        const uint32_t bits = __float_as_uint(s);
        uint32_t f = bad_order ? 1u : 0u;
        if ((bits & 0x7f800000u) == 0x7f800000u) f |= 2u;
        if (s < 0.0f) f |= 4u;
        flags[chunk] = (uint8_t)f;
    }
}

}  // namespace

hipError_t launch_validate(const uint8_t* payload, const float* scales, uint8_t* flags,
                           int64_t n_chunks, hipStream_t stream) {
    void* args[] = {(void*)&payload, (void*)&scales, (void*)&flags, (void*)&n_chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(&validate_kernel), dim3((unsigned)n_chunks),
                           dim3(kWave), args, 0, stream);
}

}  // namespace sl
