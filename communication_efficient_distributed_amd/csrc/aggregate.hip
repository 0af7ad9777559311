// aggregate.hip -- decode N peers' chunk records and sum them into a dense
// fp32 update, plus the elementwise outer update.
//
// "The Sparse Frontier: SparseLoCo and the Compression Math Behind
// Permissionless Pre-Training", section "Why Extreme Sparsity Doesn't Break
// Convergence", paragraph "Sparse aggregation can improve model quality": the
// receivers combine the union of the peers' selected coordinates.  The sum is
// accumulated from +0.0 in ascending peer order for every coordinate.
//
// Mapping: one 64-lane wavefront owns one output chunk and a 16 KiB LDS tile of
// its 4096 sums.  For each peer in order, lane j decodes entry j of that
// peer's record and adds it into the tile.  Indices within one record are
// distinct, so the 64 read-modify-writes of a peer never collide, and LDS
// instructions of one wavefront execute in order, so peer p+1 sees peer p's
// sums: the result is deterministic and needs no atomics.  The tile is then
// streamed to HBM with 16-byte stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

constexpr int kSlots = SL_CHUNK / (4 * kWave);  // 16 float4 per lane

__global__ __launch_bounds__(kWave) void aggregate_kernel(PeerTable peers, int32_t n_peers,
                                                          float* out, int64_t n_chunks) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    const int lane = (int)threadIdx.x;
    const int64_t chunk = (int64_t)blockIdx.x;
    if (chunk >= n_chunks) return;

    float4* t4 = reinterpret_cast<float4*>(tile);
#pragma unroll
    for (int m = 0; m < kSlots; ++m) t4[m * kWave + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    wave_sync();

    // Entry j = lane: its 12-bit index sits in the 3-byte group of the pair
    // (j & ~1, j | 1) at byte 3*(j >> 1), low half for even j; its 2-bit code
    // is field (j & 15) of code word 24 + (j >> 4).
    const int grp = 3 * (lane >> 1);
    const int w0 = grp >> 2;
    const int sh = (grp & 3) * 8 + ((lane & 1) ? 12 : 0);
    const int cw = SL_INDEX_BYTES / 4 + (lane >> 4);
    const int csh = 2 * (lane & 15);
    const size_t rec = (size_t)chunk * SL_PAYLOAD_BYTES;

    for (int p = 0; p < n_peers; ++p) {
        const uint32_t* pw = reinterpret_cast<const uint32_t*>(peers.payload[p] + rec);
        const uint32_t a = pw[w0];
        const uint32_t b = pw[w0 + 1];
        const uint32_t c = pw[cw];
        const float s = peers.scales[p][chunk];
        const uint32_t idx = (uint32_t)((((uint64_t)b << 32) | a) >> sh) & 4095u;
        const uint32_t code = (c >> csh) & 3u;
        const float s3 = s / 3.0f;
        const float mag = (code & 1u) ? s : s3;
        const float v = (code & 2u) ? -mag : mag;
        tile[idx] = tile[idx] + v;
    }
    wave_sync();

    float4* o4 = reinterpret_cast<float4*>(out + (size_t)chunk * SL_CHUNK);
#pragma unroll
    for (int m = 0; m < kSlots; ++m) o4[m * kWave + lane] = t4[m * kWave + lane];
}

// theta <- theta - out / n_peers, 16 bytes per lane per step.
__global__ __launch_bounds__(256) void apply_mean_kernel(float* theta, const float* out, float nf,
                                                         int64_t n4) {
    float4* t4 = reinterpret_cast<float4*>(theta);
    const float4* o4 = reinterpret_cast<const float4*>(out);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 t = t4[i];
        const float4 o = o4[i];
        t.x = t.x - o.x / nf;
        t.y = t.y - o.y / nf;
        t.z = t.z - o.z / nf;
        t.w = t.w - o.w / nf;
        t4[i] = t;
    }
}

}  // namespace

hipError_t launch_aggregate(const PeerTable& peers, int32_t n_peers, float* out,
                            int64_t n_chunks, hipStream_t stream) {
    PeerTable t = peers;
    void* args[] = {(void*)&t, (void*)&n_peers, (void*)&out, (void*)&n_chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(&aggregate_kernel),
                           dim3((unsigned)n_chunks), dim3(kWave), args, 0, stream);
}

hipError_t launch_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n,
                             hipStream_t stream) {
    const int64_t n4 = n / 4;
    float nf = (float)n_peers;
    int64_t blocks = (n4 + 255) / 256;
    const int64_t cap = 256 * 32;  // 32 workgroups per CU over 256 CUs
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    void* args[] = {(void*)&theta, (void*)&out, (void*)&nf, (void*)&n4};
    return hipLaunchKernel(reinterpret_cast<const void*>(&apply_mean_kernel),
                           dim3((unsigned)blocks), dim3(256), args, 0, stream);
}

}  // namespace sl
