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
// its 4096 sums:
//   1. the peers' 112-byte records are fetched seven lanes x 16 bytes per
//      peer, nine peers per load instruction, and staged in the tile;
//   2. lane j reads entry j's 12-bit index and 2-bit code of every peer from
//      the staged records into registers;
//   3. the tile is cleared, then peer by peer in order lane j adds entry j.
//      Indices within one record are distinct, so the 64 read-modify-writes of
//      a peer never collide, and LDS instructions of one wavefront execute in
//      order, so peer p+1 sees peer p's sums: deterministic, no atomics;
//   4. the tile is streamed to HBM with 16-byte stores.
//
// Records are 112 bytes, so neighbouring chunks share 128-byte lines.  Work-
// groups are dispatched to the 8 XCDs round-robin; the chunk numbering gives
// each XCD a contiguous range so a shared line is read through one L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "record.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

constexpr int kSlots = SL_CHUNK / (4 * kWave);     // 16 float4 per lane
constexpr int kXcds = 8;
constexpr int kRecWords = SL_PAYLOAD_BYTES / 4;     // 28 dwords per record
constexpr int kQuads = SL_PAYLOAD_BYTES / 16;       // 7 x 16 bytes per record
constexpr int kPeersPerLoad = kWave / kQuads;       // 9 records per load instruction
constexpr int kStagePeers = 3 * kPeersPerLoad;      // 27 records staged at once
#ifndef SL_AGG_CHUNKS_PER_WAVE
#define SL_AGG_CHUNKS_PER_WAVE 4
#endif
constexpr int kChunksPerWave = SL_AGG_CHUNKS_PER_WAVE;
// The fused update also holds theta's chunk in registers; one chunk per
// wavefront measured fastest for it (341 us against 350 us at two and 360 us
// at four, 8192 x 28672 parameters, 24 peers).
#ifndef SL_AGG_APPLY_CHUNKS_PER_WAVE
#define SL_AGG_APPLY_CHUNKS_PER_WAVE 1
#endif
constexpr int kApplyChunksPerWave = SL_AGG_APPLY_CHUNKS_PER_WAVE;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void add_entry(float* tile, uint32_t f, float s, float s3) {
    const uint32_t idx = f & 4095u;
    const uint32_t code = f >> 12;
    const float mag = (code & 1u) ? s : s3;
    const float v = (code & 2u) ? -mag : mag;
    tile[idx] = tile[idx] + v;
}

__device__ __forceinline__ void clear_tile(float* tile, int lane) {
    float4* t4 = reinterpret_cast<float4*>(tile);
#pragma unroll
    for (int m = 0; m < kSlots; ++m) t4[m * kWave + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Stores of a dense 16 KiB chunk go through a buffer resource spanning exactly
// that chunk (range-checked by the hardware) so that they can carry explicit
// cache-policy bits: nontemporal (nt) with device scope (sc1).  The update (or
// theta) is written once and not read back by this kernel; at 8192 x 28672
// parameters these stores measured 20% faster than plain stores, and 2-3%
// (aggregate) and 0.5% (fused update) faster than nontemporal stores without
// the scope bit.
constexpr int kStorePolicy = 2 | 16;      // nt | sc1
constexpr int kRsrcWord3 = 0x00020000;    // raw 32-bit buffer, gfx9 family

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(float* chunk_base) {
    return __builtin_amdgcn_make_buffer_rsrc(chunk_base, (short)0, SL_CHUNK * (int)sizeof(float),
                                             kRsrcWord3);
}

template <int POLICY>
__device__ __forceinline__ void store_slot(__amdgpu_buffer_rsrc_t r, int m, int lane, v4f w) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4u, w), r, 16 * (m * kWave + lane), 0,
                                           POLICY);
}

__device__ __forceinline__ void store_tile(const float* tile, float* out_chunk, int lane) {
    const float4* t4 = reinterpret_cast<const float4*>(tile);
    const __amdgpu_buffer_rsrc_t r = chunk_rsrc(out_chunk);
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        const float4 v = t4[m * kWave + lane];
        store_slot<kStorePolicy>(r, m, lane, v4f{v.x, v.y, v.z, v.w});
    }
}

__device__ __forceinline__ int64_t xcd_chunk(int64_t per_xcd) {
    const int64_t b = (int64_t)blockIdx.x;
    return (b % kXcds) * per_xcd + b / kXcds;
}

// Finish a chunk: store the tile as the dense update, or (APPLY) update theta
// in place with theta - sum / n_peers, the same two fp32 operations as
// apply_mean_kernel.  th holds theta's chunk when APPLY (loaded early).
template <bool APPLY>
__device__ __forceinline__ void finish_chunk(const float* tile, float* dst_chunk, const v4f (&th)[kSlots],
                                             float nf, int lane) {
    if constexpr (APPLY) {
        const float4* t4 = reinterpret_cast<const float4*>(tile);
        const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(dst_chunk);
#pragma unroll
        for (int m = 0; m < kSlots; ++m) {
            const float4 o = t4[m * kWave + lane];
            v4f r;
            r.x = th[m].x - o.x / nf;
            r.y = th[m].y - o.y / nf;
            r.z = th[m].z - o.z / nf;
            r.w = th[m].w - o.w / nf;
            store_slot<kStorePolicy>(rs, m, lane, r);
        }
    } else {
        store_tile(tile, dst_chunk, lane);
    }
}

template <bool APPLY>
__device__ __forceinline__ void load_theta(const float* theta_chunk, v4f (&th)[kSlots], int lane) {
    if constexpr (APPLY) {
#pragma unroll
        for (int m = 0; m < kSlots; ++m)
            th[m] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(theta_chunk + 4 * (m * kWave + lane)));
    }
}

// Up to 9*NG <= 27 peers.  A workgroup (one wavefront) handles CPW
// consecutive chunks: all their records are loaded up front (the records of
// neighbouring chunks share lines, and the later chunks' loads are in flight
// while the first is decoded), then the chunks are summed one after another in
// the same tile.  dst is the dense update (0 peers allowed) or, with APPLY,
// theta (n_peers >= 1).
template <int NG, bool APPLY, int CPW>
__global__ __launch_bounds__(kWave) void aggregate_kernel(PeerTable peers, int32_t n_peers,
                                                          float* dst, int64_t n_chunks,
                                                          int64_t per_xcd, float nf) {
    constexpr int NP = kPeersPerLoad * NG;
    __shared__ __align__(16) float tile[SL_CHUNK];
    uint32_t* stage = reinterpret_cast<uint32_t*>(tile);  // records staged in the tile
    const int lane = (int)threadIdx.x;
    const int64_t c0 = CPW * xcd_chunk(per_xcd);  // per_xcd counts groups of CPW chunks
    if (c0 >= n_chunks) return;

    if (!APPLY && n_peers == 0) {  // the empty sum
        clear_tile(tile, lane);
        wave_sync();
#pragma unroll
        for (int h = 0; h < CPW; ++h)
            if (c0 + h < n_chunks) store_tile(tile, dst + (size_t)(c0 + h) * SL_CHUNK, lane);
        return;
    }
    // Record-load role of this lane: peer 9g + rp, bytes [16 rq, 16 rq + 16).
    // Every lane loads: lanes without a live peer re-read peer 0's record into
    // a staging slot nobody reads, which keeps the loads and the staging
    // registers out of divergent branches.  Chunks past the end re-read the
    // last chunk.
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
    const uint8_t* src[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) src[g] = peers.payload[0];
    const float* ssrc = peers.scales[0];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
        if (p < n_peers) {
            const uint8_t* pp = peers.payload[p];
            if (rp == p % kPeersPerLoad) src[p / kPeersPerLoad] = pp;
            if (lane == p) ssrc = peers.scales[p];
        }
    }
    v4u r[CPW][NG];  // native vectors: stays in registers (HIP's uint4 would not)
    float sv[CPW];  // lane p < n_peers: peer p's scale of chunk c0 + h
#pragma unroll
    for (int h = 0; h < CPW; ++h) {
        const int64_t c = c0 + h < n_chunks ? c0 + h : n_chunks - 1;
        const size_t off = (size_t)c * SL_PAYLOAD_BYTES + 16 * (size_t)rq;
#pragma unroll
        for (int g = 0; g < NG; ++g) r[h][g] = *reinterpret_cast<const v4u*>(src[g] + off);
        sv[h] = ssrc[c];
    }
    const EntryPos pos(lane);
#pragma unroll
    for (int h = 0; h < CPW; ++h) {
        if (c0 + h < n_chunks) {
            float* dst_chunk = dst + (size_t)(c0 + h) * SL_CHUNK;
            // Slots 0..9*NG hold 9*NG*112 bytes at most, well inside the tile.
#pragma unroll
            for (int g = 0; g < NG; ++g)
                *reinterpret_cast<v4u*>(stage + (kPeersPerLoad * g + rp) * kRecWords + 4 * rq) = r[h][g];
            v4f th[kSlots];
            load_theta<APPLY>(dst_chunk, th, lane);  // in flight while the records are decoded
            wave_sync();
            uint32_t f[NP];
#pragma unroll
            for (int p = 0; p < NP; ++p)
                if (p < n_peers) f[p] = pos.read(stage + p * kRecWords);
            wave_sync();
            clear_tile(tile, lane);
            const float s3v = sv[h] / 3.0f;  // lane p: peer p's s/3, correctly rounded
            wave_sync();
#pragma unroll
            for (int p = 0; p < NP; ++p)
                if (p < n_peers)
                    add_entry(tile, f[p], __uint_as_float(read_lane(__float_as_uint(sv[h]), p)),
                              __uint_as_float(read_lane(__float_as_uint(s3v), p)));
            wave_sync();
            finish_chunk<APPLY>(tile, dst_chunk, th, nf, lane);
            wave_sync();  // the next chunk stages into the tile
        }
    }
}

// More than 27 peers: one chunk per workgroup, records staged 27 peers at a
// time in a separate 3 KiB area so the tile keeps its partial sums.
template <bool APPLY>
__global__ __launch_bounds__(kWave) void aggregate_many_kernel(PeerTable peers, int32_t n_peers,
                                                               float* dst, int64_t n_chunks,
                                                               int64_t per_xcd, float nf) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[kStagePeers * kRecWords];
    const int lane = (int)threadIdx.x;
    const int64_t chunk = xcd_chunk(per_xcd);
    if (chunk >= n_chunks) return;
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
    const EntryPos pos(lane);
    const size_t off = (size_t)chunk * SL_PAYLOAD_BYTES + 16 * (size_t)rq;
    clear_tile(tile, lane);
    for (int p0 = 0; p0 < n_peers; p0 += kStagePeers) {
        const uint8_t* src[3] = {nullptr, nullptr, nullptr};
        const float* ssrc = nullptr;
        for (int q = 0; q < kStagePeers && p0 + q < n_peers; ++q) {
            const uint8_t* pp = peers.payload[p0 + q];
            if (rp == q % kPeersPerLoad) src[q / kPeersPerLoad] = pp;
            if (lane == q) ssrc = peers.scales[p0 + q];
        }
#pragma unroll
        for (int g = 0; g < 3; ++g)
            if (rp < kPeersPerLoad && p0 + kPeersPerLoad * g + rp < n_peers)
                *reinterpret_cast<uint4*>(stage + (kPeersPerLoad * g + rp) * kRecWords + 4 * rq) =
                    *reinterpret_cast<const uint4*>(src[g] + off);
        const float sv = (lane < kStagePeers && p0 + lane < n_peers) ? ssrc[chunk] : 0.0f;
        const float s3v = sv / 3.0f;
        wave_sync();
        for (int q = 0; q < kStagePeers && p0 + q < n_peers; ++q)
            add_entry(tile, pos.read(stage + q * kRecWords),
                      __uint_as_float(read_lane(__float_as_uint(sv), q)),
                      __uint_as_float(read_lane(__float_as_uint(s3v), q)));
        wave_sync();
    }
    float* dst_chunk = dst + (size_t)chunk * SL_CHUNK;
    v4f th[kSlots];
    load_theta<APPLY>(dst_chunk, th, lane);
    finish_chunk<APPLY>(tile, dst_chunk, th, nf, lane);
}

// theta <- theta - out / n_peers over one 4096-element chunk per wavefront,
// streaming loads and stores.
__global__ __launch_bounds__(kWave) void apply_mean_kernel(float* theta, const float* out, float nf,
                                                           int64_t n_chunks) {
    const int lane = (int)threadIdx.x;
    const int64_t chunk = (int64_t)blockIdx.x;
    if (chunk >= n_chunks) return;
    const size_t base = (size_t)chunk * SL_CHUNK;
    v4f t[kSlots], o[kSlots];
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        const size_t off = base + 4 * (size_t)(m * kWave + lane);
        t[m] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(theta + off));
        o[m] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(out + off));
    }
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        const size_t off = base + 4 * (size_t)(m * kWave + lane);
        v4f r;
        r.x = t[m].x - o[m].x / nf;
        r.y = t[m].y - o[m].y / nf;
        r.z = t[m].z - o[m].z / nf;
        r.w = t[m].w - o[m].w / nf;
        __builtin_nontemporal_store(r, reinterpret_cast<v4f*>(theta + off));
    }
}

template <bool APPLY, int CPW = kChunksPerWave>
hipError_t launch_aggregate_impl(const PeerTable& peers, int32_t n_peers, float* dst,
                                 int64_t n_chunks, hipStream_t stream) {
    PeerTable t = peers;
    float nf = (float)n_peers;
    if (n_peers > kStagePeers) {
        const int64_t per_xcd = (n_chunks + kXcds - 1) / kXcds;
        void* args[] = {(void*)&t, (void*)&n_peers, (void*)&dst, (void*)&n_chunks, (void*)&per_xcd,
                        (void*)&nf};
        return hipLaunchKernel(reinterpret_cast<const void*>(&aggregate_many_kernel<APPLY>),
                               dim3((unsigned)(per_xcd * kXcds)), dim3(kWave), args, 0, stream);
    }
    const int64_t groups = (n_chunks + CPW - 1) / CPW;
    const int64_t per_xcd = (groups + kXcds - 1) / kXcds;
    void* args[] = {(void*)&t, (void*)&n_peers, (void*)&dst, (void*)&n_chunks, (void*)&per_xcd,
                    (void*)&nf};
    const void* k = n_peers > 2 * kPeersPerLoad ? reinterpret_cast<const void*>(&aggregate_kernel<3, APPLY, CPW>)
                    : n_peers > kPeersPerLoad   ? reinterpret_cast<const void*>(&aggregate_kernel<2, APPLY, CPW>)
                                                : reinterpret_cast<const void*>(&aggregate_kernel<1, APPLY, CPW>);
    return hipLaunchKernel(k, dim3((unsigned)(per_xcd * kXcds)), dim3(kWave), args, 0, stream);
}

}  // namespace

hipError_t launch_aggregate(const PeerTable& peers, int32_t n_peers, float* out,
                            int64_t n_chunks, hipStream_t stream) {
    return launch_aggregate_impl<false>(peers, n_peers, out, n_chunks, stream);
}

hipError_t launch_aggregate_apply(const PeerTable& peers, int32_t n_peers, float* theta,
                                  int64_t n_chunks, hipStream_t stream) {
    return launch_aggregate_impl<true, kApplyChunksPerWave>(peers, n_peers, theta, n_chunks, stream);
}

hipError_t launch_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n,
                             hipStream_t stream) {
    int64_t n_chunks = n / SL_CHUNK;
    float nf = (float)n_peers;
    void* args[] = {(void*)&theta, (void*)&out, (void*)&nf, (void*)&n_chunks};
    return hipLaunchKernel(reinterpret_cast<const void*>(&apply_mean_kernel),
                           dim3((unsigned)n_chunks), dim3(kWave), args, 0, stream);
}

}  // namespace sl
