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

#include <mutex>

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
constexpr int kStatValues = 5;  // four counts and the scale maximum (fp32 bits, widened)

// Scratch layout: the slots (G * n_peers <= kStatGroups + SL_MAX_PEERS - 1,
// kStatValues uint64 each), then one uint32 arrival counter per peer.  The
// counters must be zero before the first call; every completed call leaves
// them at zero.
// About 256 workgroups in all: at 24 peers x 57344 records 256, 512 and 1024
// took 31.3, 32.6-33.3 and 32.2-32.9 us.
constexpr int kStatGroups = 256;
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima): every vector
// memory access issued so far has completed.
constexpr int kWaitStoresDone = 0x0F70;
constexpr size_t kStatSlotBytes = (size_t)(kStatGroups + SL_MAX_PEERS) * kStatValues * sizeof(uint64_t);
constexpr size_t kStatScratchBytes = kStatSlotBytes + SL_MAX_PEERS * sizeof(uint32_t);

// sl_peer_stats_noalloc's scratch: one copy on every GPU the library runs on,
// zero when the code object is loaded (its counters must start at zero, and
// every completed call leaves them at zero).  Host code uses the address
// hipGetSymbolAddress returns for the current device, never this name.
static __device__ __align__(256) uint8_t scratch[kStatScratchBytes];

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += (uint64_t)__shfl_xor((unsigned long long)v, o, kWave);
    return v;
}

// Grid (G, n_peers).  Workgroup g of peer p takes records g*256 + t +
// k*G*256; flags (if given) as validate_kernel writes them.  Each workgroup
// stores its five partial results in its own slot of the scratch, then counts
// itself in the peer's arrival counter; the workgroup that arrives last (the
// G-th) adds up the peer's G slots, writes the totals over
// counts[4p..4p+3] and scale_max[p], and sets the counter back to zero for the
// next call.  One launch, no clearing pass, and the totals do not depend on
// the arrival order.
__global__ __launch_bounds__(kStatThreads) void stats_kernel(PeerTable peers, int64_t n_chunks, uint8_t* flags,
                                                             uint64_t* counts, uint32_t* scale_max,
                                                             uint64_t* slots, uint32_t* arrived) {
    __shared__ uint64_t part[kStatWaves][kStatValues];
    __shared__ uint32_t last;
    const int p = (int)blockIdx.y;
    const int G = (int)gridDim.x;
    const int tid = (int)threadIdx.x;
    const int64_t stride = (int64_t)G * kStatThreads;
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
        part[wv][4] = tm;
    }
    __syncthreads();
    uint64_t* peer_slots = slots + (size_t)p * (size_t)G * kStatValues;
    if (tid == 0) {
        uint64_t* mine = peer_slots + (size_t)blockIdx.x * kStatValues;
        uint64_t vals[kStatValues];
        uint64_t m = 0;
        for (int k = 0; k < 4; ++k) vals[k] = part[0][k] + part[1][k] + part[2][k] + part[3][k];
        for (int i = 0; i < kStatWaves; ++i) m = part[i][4] > m ? part[i][4] : m;
        vals[4] = m;
        // The slots are the only data passed between workgroups, and they go
        // through agent-scope atomic stores and loads, which the non-coherent
        // caches do not hold back or serve stale.  So the hand-over needs the
        // slot stores completed before the count is raised (the wait below),
        // not the cache write-back and invalidation that release / acquire
        // orderings add; with those on every workgroup's count the pass took
        // 35-63 us at 24 peers x 57344 records instead of 31 us.
        for (int k = 0; k < kStatValues; ++k)
            __hip_atomic_store(&mine[k], vals[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // no reordering by the compiler
        __builtin_amdgcn_s_waitcnt(kWaitStoresDone);
        const uint32_t before = __hip_atomic_fetch_add(&arrived[p], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == (uint32_t)(G - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (last == 0u) return;  // the whole workgroup
    // Integer sums and a maximum: any grouping gives the same totals.
    uint64_t v[kStatValues] = {0, 0, 0, 0, 0};
    for (int g = tid; g < G; g += kStatThreads) {
        uint64_t* s = peer_slots + (size_t)g * kStatValues;
        uint64_t x[kStatValues];
#pragma unroll
        for (int k = 0; k < kStatValues; ++k) x[k] = __hip_atomic_load(&s[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] += x[k];
        v[4] = x[4] > v[4] ? x[4] : v[4];
    }
    const uint64_t r0 = wave_sum64(v[0]), r1 = wave_sum64(v[1]), r2 = wave_sum64(v[2]), r3 = wave_sum64(v[3]);
    const uint32_t r4 = wave_max((uint32_t)v[4]);
    __syncthreads();  // every wavefront is done reading part[] above
    if ((tid & (kWave - 1)) == 0) {
        part[wv][0] = r0;
        part[wv][1] = r1;
        part[wv][2] = r2;
        part[wv][3] = r3;
        part[wv][4] = r4;
    }
    __syncthreads();
    if (tid < kStatValues) {
        uint64_t t = 0;
        for (int i = 0; i < kStatWaves; ++i) t = tid < 4 ? t + part[i][tid] : (part[i][4] > t ? part[i][4] : t);
        if (tid < 4)
            counts[4 * (size_t)p + tid] = t;
        else
            scale_max[p] = (uint32_t)t;
    }
    if (tid == 0) __hip_atomic_store(&arrived[p], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunk-major statistics (records r = c * n_peers + p in memory order, as
// sl_aggregate_interleaved reads them).  A block of cpb = floor(256 / n_peers)
// whole chunks is cpb * n_peers consecutive records, one per lane, so lane t of
// a block always meets peer t % n_peers and keeps that peer's partial results
// in registers; a wavefront's loads cover consecutive records, as in
// validate_kernel.  Workgroup g takes blocks g, g + G, g + 2G, ..., so the grid
// reads the buffer front to back.  At the end the workgroup folds its lanes'
// results per peer in LDS and adds them with agent-scope atomics to copy
// g % kIlCopies of the per-peer totals in the scratch (integer sums and a
// maximum: the totals do not depend on the order).  Same-address atomics
// serialize, so the copies keep the number landing on one address at G /
// kIlCopies.  The workgroup that arrives last adds up the copies, writes
// counts / scale_max and zeroes the copies and its arrival counter for the next
// call.
// At 24 peers x 57344 records, four rotating sets (records from HBM): 256
// workgroups with one copy 49 us, 256 with 8 copies 44 us, 512 with 4 or 8
// copies 39 us, 768 with 8 or 16 copies 42-45 us, 1024 with 16 or 32 copies
// 44-50 us; each workgroup on its own contiguous range of chunks (256
// workgroups, one copy) 50 us.  Two to eight records per lane in flight
// (unrolling) measured the same.
constexpr int kIlGroups = 512;
constexpr int kIlCopies = 8;
constexpr size_t kIlTotalsBytes = (size_t)kIlCopies * SL_MAX_PEERS * 4 * sizeof(uint64_t);
constexpr size_t kIlMaxBytes = (size_t)kIlCopies * SL_MAX_PEERS * sizeof(uint32_t);
constexpr size_t kIlScratchBytes = kIlTotalsBytes + kIlMaxBytes + 256;

__global__ __launch_bounds__(kStatThreads) void stats_interleaved_kernel(const uint8_t* records, const float* scales,
                                                                         int32_t n_peers, int64_t n_chunks,
                                                                         uint8_t* flags,
                                                                         uint64_t* counts, uint32_t* scale_max,
                                                                         uint64_t* totals, uint32_t* maxima,
                                                                         uint32_t* arrived) {
    __shared__ uint64_t acc[4][SL_MAX_PEERS];
    __shared__ uint32_t amax[SL_MAX_PEERS];
    __shared__ uint32_t last;
    const int tid = (int)threadIdx.x;
    const int n = (int)n_peers;
    const int cpb = kStatThreads / n;  // whole chunks per block
    const int p = tid % n;
    const int dc = tid / n;  // this lane's chunk within a block (lanes with dc >= cpb are idle)
    for (int i = tid; i < n; i += kStatThreads) {
        acc[0][i] = 0;
        acc[1][i] = 0;
        acc[2][i] = 0;
        acc[3][i] = 0;
        amax[i] = 0;
    }
    uint32_t bad = 0, zero = 0, mag = 0, neg = 0, mx = 0;
    const int64_t c_step = (int64_t)gridDim.x * cpb;
    if (dc < cpb) {
#pragma unroll 2
        for (int64_t c = (int64_t)blockIdx.x * cpb + dc; c < n_chunks; c += c_step) {
            const size_t r = (size_t)c * (size_t)n + (size_t)p;
            const uint8_t* rec = records + r * SL_PAYLOAD_BYTES;
            uint32_t w[kIndexWords];
            load_indices(rec, w);
            const v4u cw = load_global16(rec + SL_INDEX_BYTES);
            const float s = scales[r];
            const uint32_t f = record_flags(w, s);
            if (flags) flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)f;
            bad += f ? 1u : 0u;
            zero += s == 0.0f ? 1u : 0u;
            mag += __popc(cw.x & 0x55555555u) + __popc(cw.y & 0x55555555u) + __popc(cw.z & 0x55555555u) +
                   __popc(cw.w & 0x55555555u);
            neg += __popc(cw.x & 0xaaaaaaaau) + __popc(cw.y & 0xaaaaaaaau) + __popc(cw.z & 0xaaaaaaaau) +
                   __popc(cw.w & 0xaaaaaaaau);
            const uint32_t key = __float_as_uint(s) & 0x7fffffffu;
            if ((f & 6u) == 0u && key > mx) mx = key;
        }
    }
    __syncthreads();  // acc and amax are zero
    if (dc < cpb) {
        if (bad) __hip_atomic_fetch_add(&acc[0][p], (uint64_t)bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (zero) __hip_atomic_fetch_add(&acc[1][p], (uint64_t)zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (mag) __hip_atomic_fetch_add(&acc[2][p], (uint64_t)mag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (neg) __hip_atomic_fetch_add(&acc[3][p], (uint64_t)neg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (mx) __hip_atomic_fetch_max(&amax[p], mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __syncthreads();
    // One lane per peer (n_peers <= 128 < 256).  Zero contributions are
    // skipped; the totals are agent-scope atomics, coherent across the XCDs'
    // caches, and the wait below holds the arrival until they are done (see
    // stats_kernel for why no release / acquire is needed).
    const int cp = (int)(blockIdx.x % kIlCopies);
    if (tid < n) {
        uint64_t* tot = totals + (size_t)(cp * SL_MAX_PEERS + tid) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t v = acc[k][tid];
            if (v) __hip_atomic_fetch_add(&tot[k], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t m = amax[tid];
        if (m) __hip_atomic_fetch_max(&maxima[cp * SL_MAX_PEERS + tid], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // no reordering by the compiler
    __builtin_amdgcn_s_waitcnt(kWaitStoresDone);
    __syncthreads();
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (last == 0u) return;  // the whole workgroup
    // This runs after every other workgroup has finished, so its latency is
    // the kernel's tail: all the copies' loads are issued first and waited for
    // once, then the zeroing stores.  (Zeroing each copy right after loading
    // it made the compiler wait for every load in turn: 33 round trips, 13-16
    // us at 24 peers.)
    if (tid < n) {
        uint64_t t[4] = {0, 0, 0, 0};
        uint32_t tm = 0;
#pragma unroll
        for (int q = 0; q < kIlCopies; ++q) {
            const uint64_t* tot = totals + (size_t)(q * SL_MAX_PEERS + tid) * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) t[k] += __hip_atomic_load(&tot[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t v = __hip_atomic_load(&maxima[q * SL_MAX_PEERS + tid], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            tm = v > tm ? v : tm;
        }
#pragma unroll
        for (int q = 0; q < kIlCopies; ++q) {
            uint64_t* tot = totals + (size_t)(q * SL_MAX_PEERS + tid) * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) __hip_atomic_store(&tot[k], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&maxima[q * SL_MAX_PEERS + tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) counts[4 * (size_t)tid + k] = t[k];
        scale_max[tid] = tm;
    }
    if (tid == 0) __hip_atomic_store(arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

size_t peer_stats_scratch_bytes() { return kStatScratchBytes; }

hipError_t peer_stats_static_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}


hipError_t launch_peer_stats(const PeerTable& peers, int32_t n_peers, int64_t n_chunks, uint8_t* flags,
                             int64_t* counts, float* scale_max, void* scratch_ptr, hipStream_t stream) {
    const int64_t per_peer = (kStatGroups + n_peers - 1) / n_peers;
    const int64_t needed = (n_chunks + kStatThreads - 1) / kStatThreads;
    const int64_t gx = needed < 1 ? 1 : needed < per_peer ? needed : per_peer;
    static_assert((size_t)(kStatGroups + SL_MAX_PEERS - 1) * kStatValues * sizeof(uint64_t) <= kStatSlotBytes,
                  "the slots of every valid call fit the scratch");
    if (gx * n_peers > kStatGroups + SL_MAX_PEERS - 1) return hipErrorInvalidValue;
    uint64_t* cnt = reinterpret_cast<uint64_t*>(counts);
    uint32_t* mx = reinterpret_cast<uint32_t*>(scale_max);
    uint64_t* slots = reinterpret_cast<uint64_t*>(scratch_ptr);
    uint32_t* arrived = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(scratch_ptr) + kStatSlotBytes);
    PeerTable t = peers;
    void* args[] = {(void*)&t,     (void*)&n_chunks, (void*)&flags, (void*)&cnt,
                    (void*)&mx,    (void*)&slots,    (void*)&arrived};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stats_kernel), dim3((unsigned)gx, (unsigned)n_peers),
                           dim3(kStatThreads), args, 0, stream);
}

size_t interleaved_stats_scratch_bytes() { return kIlScratchBytes; }

hipError_t launch_peer_stats_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                         int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                                         void* scratch_ptr, hipStream_t stream) {
    if (n_peers < 1 || n_peers > SL_MAX_PEERS || n_chunks < 0) return hipErrorInvalidValue;
    const int64_t cpb = kStatThreads / n_peers;
    const int64_t blocks = (n_chunks + cpb - 1) / cpb;
    const int64_t gx = blocks < 1 ? 1 : blocks < kIlGroups ? blocks : kIlGroups;
    uint64_t* cnt = reinterpret_cast<uint64_t*>(counts);
    uint32_t* mx = reinterpret_cast<uint32_t*>(scale_max);
    uint8_t* base = static_cast<uint8_t*>(scratch_ptr);
    uint64_t* totals = reinterpret_cast<uint64_t*>(base);
    uint32_t* maxima = reinterpret_cast<uint32_t*>(base + kIlTotalsBytes);
    uint32_t* arrived = reinterpret_cast<uint32_t*>(base + kIlTotalsBytes + kIlMaxBytes);
    void* args[] = {(void*)&records, (void*)&scales, (void*)&n_peers, (void*)&n_chunks, (void*)&flags,
                    (void*)&cnt,     (void*)&mx,     (void*)&totals,  (void*)&maxima,   (void*)&arrived};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stats_interleaved_kernel), dim3((unsigned)gx),
                           dim3(kStatThreads), args, 0, stream);
}

}  // namespace sl
