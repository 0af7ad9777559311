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
// Validation mapping: one lane per record, 64 records per wavefront, one grid
// row per peer.  A lane loads its record's 96 index bytes (six 16-byte loads;
// the lanes' records are 112 bytes apart, so every line is fetched once and
// the later loads hit L2) and unpacks the 64 12-bit fields with compile-time
// shifts.  (Staging the wavefront's 7 KiB of records through LDS with fully
// coalesced loads measured no faster.)  The statistics kernels use the same
// per-record checks; their mappings are described where they are defined.
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

// Both statistics kernels read the records in memory order with a grid of
// kStatGroups workgroups, fold their partial results per peer in LDS, and add
// them with agent-scope integer atomics to copy g % kStatCopies of the
// per-peer totals in the scratch.  Same-address atomics serialize, so the
// copies keep the number landing on one address at G / kStatCopies.  The
// workgroup that arrives last adds up the copies, writes counts / scale_max
// and zeroes the copies and the arrival counter for the next call.  Every
// statistic is an integer sum or a maximum, so the totals do not depend on the
// order in which the workgroups arrive.
// Chunk-major records, 24 peers x 57344, four rotating sets (records from
// HBM): 256 workgroups with one copy 49 us, with 8 copies 44 us, 512 with 4 or
// 8 copies 39 us, 768 with 8 or 16 copies 42-45 us, 1024 with 16 or 32 copies
// 44-50 us.
constexpr int kStatGroups = 512;
constexpr int kStatCopies = 8;
// Scratch layout: kStatCopies copies of uint64 totals[SL_MAX_PEERS][4], then
// kStatCopies copies of uint32 maxima[SL_MAX_PEERS], then the arrival counter.
// All zero before the first call; every completed call leaves them zero.
constexpr size_t kStatTotalsBytes = (size_t)kStatCopies * SL_MAX_PEERS * 4 * sizeof(uint64_t);
constexpr size_t kStatMaxBytes = (size_t)kStatCopies * SL_MAX_PEERS * sizeof(uint32_t);
constexpr size_t kStatScratchBytes = kStatTotalsBytes + kStatMaxBytes + 256;
// s_waitcnt vmcnt(0) (expcnt and lgkmcnt at their maxima): every vector
// memory access issued so far has completed.
constexpr int kWaitStoresDone = 0x0F70;

// sl_peer_stats_noalloc's scratch: one copy on every GPU the library runs on,
// zero when the code object is loaded (it must start at zero, and every
// completed call leaves it at zero).  Host code uses the address
// hipGetSymbolAddress returns for the current device, never this name.
static __device__ __align__(256) uint8_t scratch[kStatScratchBytes];

struct StatScratch {
    uint64_t* totals;
    uint32_t* maxima;
    uint32_t* arrived;
};

__host__ __device__ inline StatScratch stat_scratch(void* base) {
    uint8_t* b = static_cast<uint8_t*>(base);
    return {reinterpret_cast<uint64_t*>(b), reinterpret_cast<uint32_t*>(b + kStatTotalsBytes),
            reinterpret_cast<uint32_t*>(b + kStatTotalsBytes + kStatMaxBytes)};
}

// Per-peer partial results of one workgroup, in LDS.
struct StatLds {
    uint64_t acc[4][SL_MAX_PEERS];  // flagged, zero-scale, magnitude-level, sign-bit counts
    uint32_t amax[SL_MAX_PEERS];    // largest valid scale (fp32 bits)
    uint32_t last;
};

__device__ __forceinline__ void stat_lds_clear(StatLds& l, int n, int tid) {
    for (int i = tid; i < n; i += kStatThreads) {
        l.acc[0][i] = 0;
        l.acc[1][i] = 0;
        l.acc[2][i] = 0;
        l.acc[3][i] = 0;
        l.amax[i] = 0;
    }
}

__device__ __forceinline__ void stat_lds_add(StatLds& l, int p, uint64_t bad, uint64_t zero, uint64_t mag,
                                             uint64_t neg, uint32_t mx) {
    if (bad) __hip_atomic_fetch_add(&l.acc[0][p], bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (zero) __hip_atomic_fetch_add(&l.acc[1][p], zero, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (mag) __hip_atomic_fetch_add(&l.acc[2][p], mag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (neg) __hip_atomic_fetch_add(&l.acc[3][p], neg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (mx) __hip_atomic_fetch_max(&l.amax[p], mx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One record's checks and counts: the flags (bit 0 order, bit 1 non-finite
// scale, bit 2 negative scale), and the code bits.  Code j sits at bits
// [2j, 2j+2): bit 0 (magnitude) on even positions, bit 1 (sign) on odd ones.
// For non-negative finite floats (and -0 mapped to +0) the bit pattern orders
// like the value, so the maximum is taken on the bits.
struct RecordStats {
    uint32_t flags, zero, mag, neg, key;
};

__device__ __forceinline__ RecordStats record_stats(const uint8_t* rec, float s) {
    uint32_t w[kIndexWords];
    load_indices(rec, w);
    const v4u cw = load_global16(rec + SL_INDEX_BYTES);
    RecordStats r;
    r.flags = record_flags(w, s);
    r.zero = s == 0.0f ? 1u : 0u;
    r.mag = __popc(cw.x & 0x55555555u) + __popc(cw.y & 0x55555555u) + __popc(cw.z & 0x55555555u) +
            __popc(cw.w & 0x55555555u);
    r.neg = __popc(cw.x & 0xaaaaaaaau) + __popc(cw.y & 0xaaaaaaaau) + __popc(cw.z & 0xaaaaaaaau) +
            __popc(cw.w & 0xaaaaaaaau);
    r.key = (r.flags & 6u) == 0u ? __float_as_uint(s) & 0x7fffffffu : 0u;
    return r;
}

// The end phase shared by both kernels (call with every lane of the
// workgroup, after its last stat_lds_add and a barrier).  The totals are
// agent-scope atomics, which the XCDs' non-coherent caches do not hold back or
// serve stale, so the hand-over needs the atomics completed before the count
// is raised (the wait below), not the cache write-back and invalidation that
// release / acquire orderings add (with those on every workgroup's count the
// per-peer pass took 35-63 us at 24 peers x 57344 records instead of 31 us).
__device__ __forceinline__ void stat_finish(StatLds& l, int n, int tid, const StatScratch& sc, uint64_t* counts,
                                            uint32_t* scale_max) {
    const int cp = (int)(blockIdx.x % kStatCopies);
    if (tid < n) {  // one lane per peer (n_peers <= 128 < 256)
        uint64_t* tot = sc.totals + (size_t)(cp * SL_MAX_PEERS + tid) * 4;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint64_t v = l.acc[k][tid];
            if (v) __hip_atomic_fetch_add(&tot[k], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const uint32_t m = l.amax[tid];
        if (m)
            __hip_atomic_fetch_max(&sc.maxima[cp * SL_MAX_PEERS + tid], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");  // no reordering by the compiler
    __builtin_amdgcn_s_waitcnt(kWaitStoresDone);
    __syncthreads();
    if (tid == 0) {
        const uint32_t before = __hip_atomic_fetch_add(sc.arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        l.last = before == gridDim.x - 1 ? 1u : 0u;
    }
    __syncthreads();
    if (l.last == 0u) return;  // the whole workgroup
    // This runs after every other workgroup has finished, so its latency is
    // the kernel's tail: all the copies' loads are issued first and waited for
    // once, then the zeroing stores.  (Zeroing each copy right after loading
    // it made the compiler wait for every load in turn: 33 round trips, 13-16
    // us at 24 peers.)
    if (tid < n) {
        uint64_t t[4] = {0, 0, 0, 0};
        uint32_t tm = 0;
#pragma unroll
        for (int q = 0; q < kStatCopies; ++q) {
            const uint64_t* tot = sc.totals + (size_t)(q * SL_MAX_PEERS + tid) * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) t[k] += __hip_atomic_load(&tot[k], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t v = __hip_atomic_load(&sc.maxima[q * SL_MAX_PEERS + tid], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
            tm = v > tm ? v : tm;
        }
#pragma unroll
        for (int q = 0; q < kStatCopies; ++q) {
            uint64_t* tot = sc.totals + (size_t)(q * SL_MAX_PEERS + tid) * 4;
#pragma unroll
            for (int k = 0; k < 4; ++k) __hip_atomic_store(&tot[k], (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&sc.maxima[q * SL_MAX_PEERS + tid], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) counts[4 * (size_t)tid + k] = t[k];
        scale_max[tid] = tm;
    }
    if (tid == 0) __hip_atomic_store(sc.arrived, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Per-peer records, taken peer after peer in memory order: super-block b is
// peer b / nsb's records [(b % nsb) * 1024, + 1024), four per lane (lane t
// takes records t, t + 256, t + 512, t + 768).  Workgroup g takes super-blocks
// g, g + G, ..., so the grid reads a few peers' buffers at a time, front to
// back, not all of them at once.  After each super-block the workgroup's
// wavefronts sum their lanes' counts (DPP scans) and add them to the peer's
// LDS totals.
// At 24 peers x 57344 records (scratch harness, one box): 36 us from HBM (four
// rotating sets) and 29.4 us with one set re-read, against 43-44 and 31.6 us
// for a grid of (G, n_peers) workgroups that each walk one peer's records.
// One record per lane per super-block: 35 / 32 us; two: 35 / 31 us; eight:
// 40 / 32 us; 1024 workgroups with two or four: 39-41 / 34 us; 256 with four:
// 47 / 37 us.
constexpr int kStatPerLane = 4;
constexpr int64_t kStatSuperBlock = (int64_t)kStatPerLane * kStatThreads;

__global__ __launch_bounds__(kStatThreads) void stats_kernel(PeerTable peers, int32_t n_peers, int64_t n_chunks,
                                                             int64_t nsb, uint8_t* flags, uint64_t* counts,
                                                             uint32_t* scale_max, StatScratch sc) {
    __shared__ StatLds l;
    const int tid = (int)threadIdx.x;
    const int n = (int)n_peers;
    stat_lds_clear(l, n, tid);
    __syncthreads();
    const int64_t total = (int64_t)n * nsb;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int p = (int)(b / nsb);
        const int64_t c0 = (b - (int64_t)p * nsb) * kStatSuperBlock + tid;
        uint32_t bad = 0, zero = 0, mag = 0, neg = 0, mx = 0;
        for (int j = 0; j < kStatPerLane; ++j) {
            const int64_t c = c0 + (int64_t)j * kStatThreads;
            if (c >= n_chunks) break;
            const RecordStats r = record_stats(peers.payload[p] + (size_t)c * SL_PAYLOAD_BYTES, peers.scales[p][c]);
            if (flags) flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)r.flags;
            bad += r.flags ? 1u : 0u;
            zero += r.zero;
            mag += r.mag;
            neg += r.neg;
            mx = r.key > mx ? r.key : mx;
        }
        // At most 64 * 4 per lane, so the wavefront's sums fit 32 bits.
        const uint32_t t0 = __builtin_amdgcn_readlane(wave_prefix_sum(bad), kWave - 1);
        const uint32_t t1 = __builtin_amdgcn_readlane(wave_prefix_sum(zero), kWave - 1);
        const uint32_t t2 = __builtin_amdgcn_readlane(wave_prefix_sum(mag), kWave - 1);
        const uint32_t t3 = __builtin_amdgcn_readlane(wave_prefix_sum(neg), kWave - 1);
        const uint32_t tm = wave_max(mx);
        if ((tid & (kWave - 1)) == 0) stat_lds_add(l, p, t0, t1, t2, t3, tm);
    }
    __syncthreads();
    stat_finish(l, n, tid, sc, counts, scale_max);
}

// Chunk-major records (records r = c * n_peers + p in memory order, as
// sl_aggregate_interleaved reads them).  A block of cpb = floor(256 / n_peers)
// whole chunks is cpb * n_peers consecutive records, one per lane, so lane t of
// a block always meets peer t % n_peers and keeps that peer's partial results
// in registers; a wavefront's loads cover consecutive records, as in
// validate_kernel.  Workgroup g takes blocks g, g + G, g + 2G, ..., so the grid
// reads the buffer front to back.  Each workgroup on its own contiguous range
// of chunks measured 50 us (256 workgroups, one copy, 24 peers, from HBM), two
// to eight records per lane in flight (unrolling) the same as one.
__global__ __launch_bounds__(kStatThreads) void stats_interleaved_kernel(const uint8_t* records, const float* scales,
                                                                         int32_t n_peers, int64_t n_chunks,
                                                                         uint8_t* flags, uint64_t* counts,
                                                                         uint32_t* scale_max, StatScratch sc) {
    __shared__ StatLds l;
    const int tid = (int)threadIdx.x;
    const int n = (int)n_peers;
    const int cpb = kStatThreads / n;  // whole chunks per block
    const int p = tid % n;
    const int dc = tid / n;  // this lane's chunk within a block (lanes with dc >= cpb are idle)
    stat_lds_clear(l, n, tid);
    uint64_t bad = 0, zero = 0, mag = 0, neg = 0;
    uint32_t mx = 0;
    const int64_t c_step = (int64_t)gridDim.x * cpb;
    if (dc < cpb) {
#pragma unroll 2
        for (int64_t c = (int64_t)blockIdx.x * cpb + dc; c < n_chunks; c += c_step) {
            const size_t r = (size_t)c * (size_t)n + (size_t)p;
            const RecordStats st = record_stats(records + r * SL_PAYLOAD_BYTES, scales[r]);
            if (flags) flags[(size_t)p * (size_t)n_chunks + (size_t)c] = (uint8_t)st.flags;
            bad += st.flags ? 1u : 0u;
            zero += st.zero;
            mag += st.mag;
            neg += st.neg;
            mx = st.key > mx ? st.key : mx;
        }
    }
    __syncthreads();  // the LDS totals are zero
    if (dc < cpb) stat_lds_add(l, p, bad, zero, mag, neg, mx);
    __syncthreads();
    stat_finish(l, n, tid, sc, counts, scale_max);
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
    if (n_peers < 1 || n_peers > SL_MAX_PEERS || n_chunks < 0) return hipErrorInvalidValue;
    const int64_t nsb = (n_chunks + kStatSuperBlock - 1) / kStatSuperBlock;
    const int64_t total = nsb * n_peers;
    const int64_t gx = total < 1 ? 1 : total < kStatGroups ? total : kStatGroups;
    uint64_t* cnt = reinterpret_cast<uint64_t*>(counts);
    uint32_t* mx = reinterpret_cast<uint32_t*>(scale_max);
    StatScratch sc = stat_scratch(scratch_ptr);
    PeerTable t = peers;
    void* args[] = {(void*)&t,   (void*)&n_peers, (void*)&n_chunks, (void*)&nsb,
                    (void*)&flags, (void*)&cnt,   (void*)&mx,       (void*)&sc};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stats_kernel), dim3((unsigned)gx), dim3(kStatThreads),
                           args, 0, stream);
}

size_t interleaved_stats_scratch_bytes() { return kStatScratchBytes; }

hipError_t launch_peer_stats_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                         int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                                         void* scratch_ptr, hipStream_t stream) {
    if (n_peers < 1 || n_peers > SL_MAX_PEERS || n_chunks < 0) return hipErrorInvalidValue;
    const int64_t cpb = kStatThreads / n_peers;
    const int64_t blocks = (n_chunks + cpb - 1) / cpb;
    const int64_t gx = blocks < 1 ? 1 : blocks < kStatGroups ? blocks : kStatGroups;
    uint64_t* cnt = reinterpret_cast<uint64_t*>(counts);
    uint32_t* mx = reinterpret_cast<uint32_t*>(scale_max);
    StatScratch sc = stat_scratch(scratch_ptr);
    void* args[] = {(void*)&records, (void*)&scales, (void*)&n_peers, (void*)&n_chunks,
                    (void*)&flags,   (void*)&cnt,    (void*)&mx,      (void*)&sc};
    return hipLaunchKernel(reinterpret_cast<const void*>(&stats_interleaved_kernel), dim3((unsigned)gx),
                           dim3(kStatThreads), args, 0, stream);
}

}  // namespace sl
