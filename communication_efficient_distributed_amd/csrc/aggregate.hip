// aggregate.hip -- decode N peers' chunk records and sum them into a dense
// fp32 update, plus the elementwise outer update.
//
// "The Sparse Frontier: SparseLoCo and the Compression Math Behind
// Permissionless Pre-Training", section "Why Extreme Sparsity Doesn't Break
// Convergence", sparse-aggregation paragraph: the receivers combine the union
// of the peers' selected coordinates.  The sum is
// accumulated from +0.0 in ascending peer order for every coordinate.
//
// Mapping: one 64-lane wavefront owns one output chunk and a 16 KiB LDS tile of
// its 4096 sums:
//   1. every peer's 112-byte record is loaded into registers up front, seven
//      lanes x 16 bytes per record, nine peers per load instruction;
//   2. the tile is cleared; then, nine peers at a time, the records are staged
//      in a 1.1 KiB LDS area, lane j reads entry j's 12-bit index and 2-bit code
//      of each of them into registers, and peer by peer in order lane j adds
//      entry j to the tile.  Indices within one record are distinct, so the 64
//      read-modify-writes of a peer never collide, and LDS instructions of one
//      wavefront execute in order, so peer p+1 sees peer p's sums:
//      deterministic, no atomics;
//   3. the tile is streamed to HBM with 16-byte stores (or, fused, theta is
//      updated in place).
// The fused update for up to 27 peers uses four wavefronts per chunk instead:
// wavefront 0 runs steps 1-2 while each wavefront loads its own quarter of
// theta, then each updates its quarter from the tile.  When a call's records
// are too large to stay in the last-level cache, a wavefront sums three (up to
// 54 peers) or two (up to 81) neighbouring chunks in turn, with every chunk's
// records loaded in step 1.
//
// Records are 112 bytes, so neighbouring chunks share 128-byte lines.  Work-
// groups are dispatched to the 8 XCDs round-robin; the chunk numbering gives
// each XCD a contiguous range so a shared line is read through one L2.  The
// kernels for records laid out chunk-major across peers (one contiguous span
// per chunk) and the fused update up to 81 peers, whose theta stream
// dominates, take the chunks in linear order instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "record.h"
#include "residency.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

constexpr int kSlots = SL_CHUNK / (4 * kWave);     // 16 float4 per lane
constexpr int kXcds = 8;
constexpr int kRecWords = SL_PAYLOAD_BYTES / 4;     // 28 dwords per record
constexpr int kQuads = SL_PAYLOAD_BYTES / 16;       // 7 x 16 bytes per record
constexpr int kPeersPerLoad = kWave / kQuads;       // 9 records per load instruction

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// 16 bytes of a peer's record through a global (address space 1) pointer.  The
// peer pointers are picked per lane from the table, which leaves them generic;
// a generic load would also count against the LDS wait counter, so the first
// LDS wait of the sums would stall on records still in flight.
__device__ __forceinline__ v4u load_record16(const uint8_t* p) {
    typedef const __attribute__((address_space(1))) v4u global_v4u;
    return *(global_v4u*)(p);
}

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

// One chunk's slices of every peer's record, in registers: lane 7 q + i holds
// bytes [16 i, 16 i + 16) of peer 9 g + q's record in r[g] (lane 63 and lanes
// past the last peer re-read peer 0, so no load sits in a divergent branch),
// and lane q < 9 holds that peer's scale in sv[g].
template <int NGMAX>
struct ChunkRecords {
    v4u r[NGMAX];
    float sv[NGMAX];
};

template <int NGMAX>
__device__ __forceinline__ void load_records(const PeerTable& peers, int32_t n_peers, int64_t chunk, int lane,
                                             ChunkRecords<NGMAX>& cr) {
    constexpr int kMaxPeers = kPeersPerLoad * NGMAX;
    static_assert(kMaxPeers <= SL_MAX_PEERS + kPeersPerLoad, "peer index range");
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
    const size_t off = (size_t)chunk * SL_PAYLOAD_BYTES + 16 * (size_t)rq;

    // Group by group: the nine peers' pointers (scalar registers, from the
    // kernel arguments) are used right where they are loaded, and the
    // scheduling barrier keeps the next group's from being hoisted above this
    // group's loads.  With every peer's pointers live at once the 9 x NGMAX
    // pairs overflowed the scalar registers and spilled to vector lanes.
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
        const uint8_t* src = peers.payload[0];
        const float* ssrc = peers.scales[0];
#pragma unroll
        for (int q = 0; q < kPeersPerLoad; ++q) {
            const int p = kPeersPerLoad * g + q;
            if (p >= 1 && p < SL_MAX_PEERS && p < n_peers) {
                if (rp == q) src = peers.payload[p];
                if (lane == q) ssrc = peers.scales[p];
            }
        }
        cr.r[g] = load_record16(src + off);
        cr.sv[g] = ssrc[chunk];
        __builtin_amdgcn_sched_barrier(0);
    }
}

// A lane's record and scale pointers for each group of nine peers, selected
// once (the run kernel loads several chunks' records from the same peers):
// lane 7 q + i reads bytes [16 i, 16 i + 16) of peer 9 g + q's records, lane
// q < 9 reads peer 9 g + q's scales; other lanes read peer 0's.
template <int NGMAX>
struct LanePeers {
    const uint8_t* rec[NGMAX];
    const float* sc[NGMAX];
};

template <int NGMAX>
__device__ __forceinline__ void lane_peers(const PeerTable& peers, int32_t n_peers, int lane, LanePeers<NGMAX>& lp) {
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
        const uint8_t* src = peers.payload[0];
        const float* ssrc = peers.scales[0];
#pragma unroll
        for (int q = 0; q < kPeersPerLoad; ++q) {
            const int p = kPeersPerLoad * g + q;
            if (p >= 1 && p < SL_MAX_PEERS && p < n_peers) {
                if (rp == q) src = peers.payload[p];
                if (lane == q) ssrc = peers.scales[p];
            }
        }
        lp.rec[g] = src + 16 * rq;
        lp.sc[g] = ssrc;
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NGMAX>
__device__ __forceinline__ void load_records_at(const LanePeers<NGMAX>& lp, int64_t chunk, ChunkRecords<NGMAX>& cr) {
    typedef const __attribute__((address_space(1))) float gfloat;
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
        cr.r[g] = load_record16(lp.rec[g] + (size_t)chunk * SL_PAYLOAD_BYTES);
        cr.sv[g] = *(gfloat*)(lp.sc[g] + chunk);
    }
}

// Make the compiler wait for every load of cr at this point.
template <int NGMAX>
__device__ __forceinline__ void await_records(const ChunkRecords<NGMAX>& cr) {
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) asm volatile("" ::"v"(cr.r[g]), "v"(cr.sv[g]));
}

// The sums of one chunk over up to 9 * NGMAX peers from its loaded records,
// into the LDS tile (cleared here), in ascending peer order; run by one
// wavefront.  The peers are staged 9 at a time in `stage` (1.1 KiB).
//
// From 9 groups up the peer count is taken through an opaque copy on every
// call, so the compiler cannot compute the per-peer tests of every group (and
// every chunk of a run) ahead of the sums, where their 64-bit lane masks
// spilled into vector lanes; full groups then add their nine peers without a
// test.  That measured 1-3% faster from 55 to 128 peers with records from HBM
// and about 1% slower below 55 peers, where it is left out.
template <int NGMAX>
__device__ __forceinline__ void sum_records(const ChunkRecords<NGMAX>& cr, int32_t n_peers_in, float* tile,
                                            uint32_t* stage, int lane) {
    int32_t n_peers = n_peers_in;
    if constexpr (NGMAX >= 9) asm volatile("" : "+s"(n_peers));
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
    const EntryPos pos(lane);
    const int slot = rp < kPeersPerLoad ? rp : kPeersPerLoad;  // lane 63: dummy slot 9
    clear_tile(tile, lane);
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
        const int p0 = kPeersPerLoad * g;
        if (p0 < n_peers) {
            *reinterpret_cast<v4u*>(stage + slot * kRecWords + 4 * rq) = cr.r[g];
            wave_sync();
            uint32_t f[kPeersPerLoad];  // slots past the last peer hold stale bytes, never used
#pragma unroll
            for (int q = 0; q < kPeersPerLoad; ++q) f[q] = pos.read(stage + q * kRecWords);
            const float s3v = cr.sv[g] / 3.0f;
            wave_sync();
            auto add = [&](int q) {
                add_entry(tile, f[q], __uint_as_float(read_lane(__float_as_uint(cr.sv[g]), q)),
                          __uint_as_float(read_lane(__float_as_uint(s3v), q)));
            };
            if (NGMAX >= 9 && p0 + kPeersPerLoad <= n_peers) {
#pragma unroll
                for (int q = 0; q < kPeersPerLoad; ++q) add(q);
            } else {
#pragma unroll
                for (int q = 0; q < kPeersPerLoad; ++q)
                    if (p0 + q < n_peers) add(q);
            }
        }
    }
}

// The sums of chunk `chunk` into the tile: its records are loaded, `issued()`
// runs once the loads are in flight, then the sums.  With 9 or more loads per
// lane every load is awaited ahead of the sums: otherwise the compiler sinks
// the last load into the group that consumes it, and its latency lands in the
// middle of the sums.  (With fewer loads the staggered issue measured faster.)
template <int NGMAX, typename Issued>
__device__ __forceinline__ void sum_chunk(const PeerTable& peers, int32_t n_peers, int64_t chunk, float* tile,
                                          uint32_t* stage, int lane, Issued issued) {
    ChunkRecords<NGMAX> cr;
    load_records<NGMAX>(peers, n_peers, chunk, lane, cr);
    if constexpr (NGMAX >= 9) {
#pragma unroll
        for (int g = 0; g < NGMAX; ++g) asm volatile("" ::"v"(cr.r[g]));
    }
    issued();
    sum_records<NGMAX>(cr, n_peers, tile, stage, lane);
}

// One chunk per workgroup of one wavefront.  The tile keeps the partial sums:
// 17.1 KiB of LDS per workgroup leaves room for 9 of them per CU.  dst is the
// dense update (0 peers allowed) or, with APPLY, theta (n_peers >= 1).
template <int NGMAX, bool APPLY>
__global__ __launch_bounds__(kWave) void aggregate_kernel(PeerTable peers, int32_t n_peers, float* dst,
                                                          int64_t n_chunks, int64_t per_xcd, float nf) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int lane = (int)threadIdx.x;
    // The fused update takes its chunks in linear order up to 81 peers (8192 x
    // 28672, records from HBM: 36 / 64 peers 0.725-0.727 / 0.671-0.678 of HBM
    // against 0.705-0.708 / 0.662-0.664 with XCD ranges); at 128 peers the
    // records' shared lines weigh more and the XCD ranges won (0.556-0.561
    // against 0.544-0.547).
    const int64_t chunk = (APPLY && NGMAX <= 9) ? (int64_t)blockIdx.x : xcd_chunk(per_xcd);
    if (chunk >= n_chunks) return;
    float* dst_chunk = dst + (size_t)chunk * SL_CHUNK;
    if (!APPLY && n_peers == 0) {  // the empty sum; the peer table is empty
        clear_tile(tile, lane);
        wave_sync();
        store_tile(tile, dst_chunk, lane);
        return;
    }
    // theta is loaded early unless the records already hold most registers.
    constexpr bool kEarlyTheta = NGMAX <= 9;
    v4f th[kSlots];
    sum_chunk<NGMAX>(peers, n_peers, chunk, tile, stage, lane, [&] {
        if constexpr (kEarlyTheta) load_theta<APPLY>(dst_chunk, th, lane);
    });
    if constexpr (!kEarlyTheta) load_theta<APPLY>(dst_chunk, th, lane);
    wave_sync();
    finish_chunk<APPLY>(tile, dst_chunk, th, nf, lane);
}

// CPW neighbouring chunks per wavefront, for records that come from HBM.
// Every chunk's records are loaded up front, so the later chunks' arrive while
// the first is summed; they are awaited before the first chunk's stores are
// issued, so that no wait on a load covers any store.  Each chunk goes through
// the same operations, in the same order, as in aggregate_kernel.  In a full
// run a lane fetches its peer's CPW adjacent scales with one 8- or 12-byte
// load instead of one load per chunk: that cut the kernel's time by 6-8% at
// 36-64 peers and 1.7% at the decoder block (8192 x 28672 with records from
// HBM: 248 / 276 / 288 / 310 us at 36 / 48 / 54 / 64 peers against 234 / 254 /
// 264 / 289 us; decoder block, 24 peers, 765 against 752 us), since every
// scale load of nine peers is nine separate cache-line requests.
template <int NGMAX, int CPW>
__global__ __launch_bounds__(kWave) void aggregate_run_kernel(PeerTable peers, int32_t n_peers, float* out,
                                                              int64_t n_chunks, int64_t per_xcd) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int lane = (int)threadIdx.x;
    const int64_t c0 = CPW * xcd_chunk(per_xcd);
    if (c0 >= n_chunks) return;
    const int64_t count = n_chunks - c0 < CPW ? n_chunks - c0 : CPW;  // the same in every lane
    ChunkRecords<NGMAX> cr[CPW];
    LanePeers<NGMAX> lp;
    lane_peers<NGMAX>(peers, n_peers, lane, lp);
    if (count == CPW) {
        // A full run: every chunk's records, then each peer's CPW scales,
        // which are adjacent, in one load per group of nine peers.
        typedef const __attribute__((address_space(1))) float gfloat;
        typedef float f3 __attribute__((ext_vector_type(3), aligned(4)));
        typedef float f2 __attribute__((ext_vector_type(2), aligned(4)));
        typedef const __attribute__((address_space(1))) f3 gf3;
        typedef const __attribute__((address_space(1))) f2 gf2;
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
#pragma unroll
            for (int g = 0; g < NGMAX; ++g)
                cr[i].r[g] = load_record16(lp.rec[g] + (size_t)(c0 + i) * SL_PAYLOAD_BYTES);
        }
#pragma unroll
        for (int g = 0; g < NGMAX; ++g) {
            if constexpr (CPW == 3) {
                const f3 v = *(gf3*)(lp.sc[g] + c0);
                cr[0].sv[g] = v.x;
                cr[1].sv[g] = v.y;
                cr[2].sv[g] = v.z;
            } else if constexpr (CPW == 2) {
                const f2 v = *(gf2*)(lp.sc[g] + c0);
                cr[0].sv[g] = v.x;
                cr[1].sv[g] = v.y;
            } else {
#pragma unroll
                for (int i = 0; i < CPW; ++i) cr[i].sv[g] = *(gfloat*)(lp.sc[g] + c0 + i);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < CPW; ++i) load_records_at<NGMAX>(lp, i < count ? c0 + i : c0, cr[i]);
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        if (i < count) {
            sum_records<NGMAX>(cr[i], n_peers, tile, stage, lane);
            if (i == 0) {
#pragma unroll
                for (int j = 1; j < CPW; ++j) await_records<NGMAX>(cr[j]);
            }
            wave_sync();
            store_tile(tile, out + (size_t)(c0 + i) * SL_CHUNK, lane);
        }
    }
}

// Records laid out chunk-major across peers (interleaved): chunk c's record
// from peer p at records + (c * n_peers + p) * 112, its scale at
// scales[c * n_peers + p].  A chunk's records are then one contiguous span, and
// group g of nine peers is 63 consecutive 16-byte quads of it, so lane l reads
// quad 63 g + l (peer 9 g + l / 7, bytes 16 (l % 7)) and lane q < 9 peer 9 g + q's
// scale.  Lanes past the last peer (and lane 63) re-read peer 0's, as in
// load_records.  The addresses are computed, so no per-lane pointer table is
// held.
template <int NGMAX>
__device__ __forceinline__ void load_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                                 int64_t chunk, int lane, ChunkRecords<NGMAX>& cr) {
    typedef const __attribute__((address_space(1))) float gfloat;
    const int rp = lane / kQuads;
    const int rq = lane - kQuads * rp;
    const uint8_t* rbase = records + (size_t)chunk * (size_t)n_peers * SL_PAYLOAD_BYTES;
    const float* sbase = scales + (size_t)chunk * (size_t)n_peers;
#pragma unroll
    for (int g = 0; g < NGMAX; ++g) {
        const int p = kPeersPerLoad * g + rp;
        const int quad = rp < kPeersPerLoad && p < n_peers ? kQuads * p + rq : rq;
        const int ps = kPeersPerLoad * g + (lane < kPeersPerLoad ? lane : 0);
        cr.r[g] = load_record16(rbase + 16 * (size_t)quad);
        cr.sv[g] = *(gfloat*)(sbase + (ps < n_peers ? ps : 0));
    }
}

// sl_aggregate_interleaved: CPW neighbouring chunks per wavefront from the
// interleaved layout, the same sums in the same order as aggregate_kernel.
// Workgroup b takes run b: consecutive workgroups, which the dispatcher deals
// round-robin over the XCDs, take neighbouring chunks, so the whole device
// reads and writes one front of contiguous memory.  (The per-peer layout keeps
// each XCD on a contiguous range instead, since its neighbouring records share
// cache lines; here only one line per chunk span is shared.)  At 8192 x 28672
// with records from HBM the linear order measured 189 / 221 / 229 / 250 / 343
// us at 24 / 48 / 64 / 81 / 128 peers against 198 / 238 / 251 / 268 / 387 us
// with the XCD ranges, and 686 against 704 us at the decoder block; the same
// with records cached (162-163 against 162-165 us).
template <int NGMAX, int CPW>
__global__ __launch_bounds__(kWave) void aggregate_interleaved_kernel(const uint8_t* records, const float* scales,
                                                                      int32_t n_peers, float* out, int64_t n_chunks) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int lane = (int)threadIdx.x;
    const int64_t c0 = CPW * (int64_t)blockIdx.x;
    if (c0 >= n_chunks) return;
    const int64_t count = n_chunks - c0 < CPW ? n_chunks - c0 : CPW;  // the same in every lane
    ChunkRecords<NGMAX> cr[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i)
        load_interleaved<NGMAX>(records, scales, n_peers, i < count ? c0 + i : c0, lane, cr[i]);
    if constexpr (CPW == 1 && NGMAX >= 9) {
#pragma unroll
        for (int g = 0; g < NGMAX; ++g) asm volatile("" ::"v"(cr[0].r[g]));
    }
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
        if (i < count) {
            sum_records<NGMAX>(cr[i], n_peers, tile, stage, lane);
            if (i == 0) {
#pragma unroll
                for (int j = 1; j < CPW; ++j) await_records<NGMAX>(cr[j]);
            }
            wave_sync();
            store_tile(tile, out + (size_t)(c0 + i) * SL_CHUNK, lane);
        }
    }
}

// The run kernel is used when a launch's records and scales exceed 224 MiB,
// about what the 256 MB last-level cache keeps of them between calls: they
// then come from HBM, and the later chunks' loads hide that latency.  Records
// that fit are likely still cached from the step that received or validated
// them; there one chunk per wavefront is faster.  On 8192 x 28672 parameters
// with distinct records per peer, one chunk per wavefront against three:
//   1-27 peers (up to 180 MB)   152-159 us   against 169-181 us
//   32 peers (213 MB)           173-175 us   against 178-179 us
//   36 peers (239 MB)           267-268 us   against 234-236 us
//   40 / 48 peers               274-276 / 307 us   against 257 / 259-260 us
// and, one / two / three / four chunks per wavefront, 24 peers:
//   decoder block (582 MB)      0.82-0.86   0.75-0.77   0.72-0.75   0.75-0.76 ms
//   16e9 parameters (10.9 GB)   15.0-15.2   12.3-12.5   12.0-13.3   11.8 ms
// Three chunks per wavefront hold 98 registers per lane at 24 peers and 151 at
// 54.  From 55 to 81 peers two chunks per wavefront (147 registers) measured
// 300-363 us against 330-373 us for one (55-81 peers at 8192 x 28672).
// Beyond 81 peers one chunk per wavefront: the run kernel's form (each lane's
// peer pointers selected once, then the loads) took 496-498 us at 128 peers
// against 509-532 us for aggregate_kernel, whose pointers are selected group
// by group; two chunks per wavefront took 533 us.
constexpr uint64_t kCachedRecordBytes = 224ull << 20;
constexpr int kChunksPerWave = 3;
constexpr int kRunMaxPeers = kPeersPerLoad * 6;       // three chunks per wavefront up to here
constexpr int kPairMaxPeers = kPeersPerLoad * 9;      // two chunks per wavefront up to here

// Fused outer update with four wavefronts per chunk: wavefront 0 sums the
// peers into the tile as above, while every wavefront w loads its own
// contiguous quarter of theta (slots 4w..4w+3, four float4 per lane); after
// one barrier each updates and stores its quarter.  Same fp32 operations per
// element as aggregate_kernel<NGMAX, true>.
constexpr int kApplyWaves = 4;
constexpr int kQuarterSlots = kSlots / kApplyWaves;

template <int NGMAX>
__global__ __launch_bounds__(kWave * kApplyWaves) void aggregate_apply4_kernel(PeerTable peers, int32_t n_peers,
                                                                               float* theta, int64_t n_chunks,
                                                                               int64_t per_xcd, float nf) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int tid = (int)threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Linear chunk order: theta's read and write are 8 of the 8.68 bytes per
    // parameter at 24 peers, and the device streams them best as one front
    // (decoder block, 24 peers, records from HBM: 0.767 of HBM against 0.731
    // with each XCD on its own range; 8192 x 28672 cached 0.803 against 0.798).
    const int64_t chunk = (int64_t)blockIdx.x;
    (void)per_xcd;
    if (chunk >= n_chunks) return;  // the whole workgroup
    float* th_chunk = theta + (size_t)chunk * SL_CHUNK;
    v4f th[kQuarterSlots];
    auto load_quarter = [&] {
#pragma unroll
        for (int m = 0; m < kQuarterSlots; ++m)
            th[m] = __builtin_nontemporal_load(
                reinterpret_cast<const v4f*>(th_chunk + 4 * ((kQuarterSlots * w + m) * kWave + lane)));
    };
    if (w == 0)
        sum_chunk<NGMAX>(peers, n_peers, chunk, tile, stage, lane, load_quarter);
    else
        load_quarter();
    __syncthreads();
    const float4* t4 = reinterpret_cast<const float4*>(tile);
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(th_chunk);
#pragma unroll
    for (int m = 0; m < kQuarterSlots; ++m) {
        const int slot = kQuarterSlots * w + m;
        const float4 o = t4[slot * kWave + lane];
        v4f r;
        r.x = th[m].x - o.x / nf;
        r.y = th[m].y - o.y / nf;
        r.z = th[m].z - o.z / nf;
        r.w = th[m].w - o.w / nf;
        store_slot<kStorePolicy>(rs, slot, lane, r);
    }
}

// The fused update on interleaved records: the same operations as
// aggregate_apply4_kernel (up to 27 peers) and aggregate_kernel<NGMAX, true>
// (beyond), with the records loaded by load_interleaved.
template <int NGMAX>
__global__ __launch_bounds__(kWave * kApplyWaves) void apply4_interleaved_kernel(const uint8_t* records,
                                                                                 const float* scales, int32_t n_peers,
                                                                                 float* theta, int64_t n_chunks,
                                                                                 float nf) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int tid = (int)threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t chunk = (int64_t)blockIdx.x;  // linear order, as the interleaved aggregate
    if (chunk >= n_chunks) return;  // the whole workgroup
    float* th_chunk = theta + (size_t)chunk * SL_CHUNK;
    v4f th[kQuarterSlots];
    auto load_quarter = [&] {
#pragma unroll
        for (int m = 0; m < kQuarterSlots; ++m)
            th[m] = __builtin_nontemporal_load(
                reinterpret_cast<const v4f*>(th_chunk + 4 * ((kQuarterSlots * w + m) * kWave + lane)));
    };
    if (w == 0) {
        ChunkRecords<NGMAX> cr;
        load_interleaved<NGMAX>(records, scales, n_peers, chunk, lane, cr);
        load_quarter();
        sum_records<NGMAX>(cr, n_peers, tile, stage, lane);
    } else {
        load_quarter();
    }
    __syncthreads();
    const float4* t4 = reinterpret_cast<const float4*>(tile);
    const __amdgpu_buffer_rsrc_t rs = chunk_rsrc(th_chunk);
#pragma unroll
    for (int m = 0; m < kQuarterSlots; ++m) {
        const int slot = kQuarterSlots * w + m;
        const float4 o = t4[slot * kWave + lane];
        v4f r;
        r.x = th[m].x - o.x / nf;
        r.y = th[m].y - o.y / nf;
        r.z = th[m].z - o.z / nf;
        r.w = th[m].w - o.w / nf;
        store_slot<kStorePolicy>(rs, slot, lane, r);
    }
}

template <int NGMAX>
__global__ __launch_bounds__(kWave) void apply_interleaved_kernel(const uint8_t* records, const float* scales,
                                                                  int32_t n_peers, float* theta, int64_t n_chunks,
                                                                  float nf) {
    __shared__ __align__(16) float tile[SL_CHUNK];
    __shared__ __align__(16) uint32_t stage[(kPeersPerLoad + 1) * kRecWords];
    const int lane = (int)threadIdx.x;
    const int64_t chunk = (int64_t)blockIdx.x;  // linear order, as the interleaved aggregate
    if (chunk >= n_chunks) return;
    float* th_chunk = theta + (size_t)chunk * SL_CHUNK;
    ChunkRecords<NGMAX> cr;
    load_interleaved<NGMAX>(records, scales, n_peers, chunk, lane, cr);
    if constexpr (NGMAX >= 9) {
#pragma unroll
        for (int g = 0; g < NGMAX; ++g) asm volatile("" ::"v"(cr.r[g]));
    }
    constexpr bool kEarlyTheta = NGMAX <= 9;
    v4f th[kSlots];
    if constexpr (kEarlyTheta) load_theta<true>(th_chunk, th, lane);
    sum_records<NGMAX>(cr, n_peers, tile, stage, lane);
    if constexpr (!kEarlyTheta) load_theta<true>(th_chunk, th, lane);
    wave_sync();
    finish_chunk<true>(tile, th_chunk, th, nf, lane);
}

// theta <- theta - out / n_peers.  One workgroup of four wavefronts per
// 4096-element chunk; wavefront w streams its own contiguous quarter (four
// float4 of each stream per lane, 1 KiB per instruction), nontemporal loads
// and stores.  (Interleaving the four wavefronts at 1 KiB within each 4 KiB
// measured 3% slower: 443-446 us against 430-431 us at 8192 x 28672.)
constexpr int kMeanWaves = 4;
constexpr int kMeanSlots = SL_CHUNK / (4 * kWave * kMeanWaves);  // 4

__global__ __launch_bounds__(kWave * kMeanWaves) void apply_mean_kernel(float* theta, const float* out, float nf,
                                                                        int64_t n_chunks) {
    const int tid = (int)threadIdx.x;
    const int64_t chunk = (int64_t)blockIdx.x;
    if (chunk >= n_chunks) return;
    const size_t base = (size_t)chunk * SL_CHUNK + (size_t)(SL_CHUNK / kMeanWaves) * (size_t)(tid >> 6) +
                        4 * (size_t)(tid & (kWave - 1));
    v4f t[kMeanSlots], o[kMeanSlots];
#pragma unroll
    for (int m = 0; m < kMeanSlots; ++m) {
        const size_t off = base + (size_t)(4 * kWave) * m;
        t[m] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(theta + off));
        o[m] = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(out + off));
    }
#pragma unroll
    for (int m = 0; m < kMeanSlots; ++m) {
        const size_t off = base + (size_t)(4 * kWave) * m;
        v4f r;
        r.x = t[m].x - o[m].x / nf;
        r.y = t[m].y - o[m].y / nf;
        r.z = t[m].z - o[m].z / nf;
        r.w = t[m].w - o[m].w / nf;
        __builtin_nontemporal_store(r, reinterpret_cast<v4f*>(theta + off));
    }
}

// Residency cap of apply_mean (workgroups per CU, through unused dynamic
// LDS).  On 8192 x 28672 parameters: 429-431 us at 2 or 3, 441-442 us at 4;
// the earlier one-wavefront-per-chunk kernel ran 463-466 us.  The aggregator
// is left uncapped (9 workgroups per CU by its own LDS): capping it at 8 gained
// 1%, at 6 or 4 it lost 11% and 52%.
constexpr int kCapApplyMean = 3;
static_assert(cap_is_exact(kCapApplyMean, 0), "residency cap");

// One launch over chunks [0, n_chunks) of the given buffers.
template <bool APPLY>
hipError_t launch_aggregate_one(const PeerTable& peers, int32_t n_peers, float* dst,
                                int64_t n_chunks, hipStream_t stream) {
    PeerTable t = peers;
    float nf = (float)n_peers;
    int64_t per_xcd = (n_chunks + kXcds - 1) / kXcds;
    void* args[] = {(void*)&t, (void*)&n_peers, (void*)&dst, (void*)&n_chunks, (void*)&per_xcd,
                    (void*)&nf};
    // The smallest variant that holds every peer's record slice.
    static_assert(kPeersPerLoad * 15 >= SL_MAX_PEERS, "the widest variant covers SL_MAX_PEERS");
    const void* k = n_peers <= kPeersPerLoad * 1 ? reinterpret_cast<const void*>(&aggregate_kernel<1, APPLY>)
                    : n_peers <= kPeersPerLoad * 2 ? reinterpret_cast<const void*>(&aggregate_kernel<2, APPLY>)
                    : n_peers <= kPeersPerLoad * 3 ? reinterpret_cast<const void*>(&aggregate_kernel<3, APPLY>)
                    : n_peers <= kPeersPerLoad * 6 ? reinterpret_cast<const void*>(&aggregate_kernel<6, APPLY>)
                    : n_peers <= kPeersPerLoad * 9 ? reinterpret_cast<const void*>(&aggregate_kernel<9, APPLY>)
                                                   : reinterpret_cast<const void*>(&aggregate_kernel<15, APPLY>);
    const dim3 grid((unsigned)(per_xcd * kXcds));
    // The fused update for up to 27 peers runs four wavefronts per chunk,
    // with a residency cap that depends on the chain length.  At 8192 x 28672
    // (one wavefront per chunk: 312-316 us for 1-27 peers) it took 294-298 us
    // for 1-18 peers at 5 workgroups per CU (cap 7: 308 us), and 308-311 us
    // for 24-27 peers at 7 (cap 5: 314-319 us; uncapped 310-312 us).
    // Beyond 27 peers the chain needs the one-wavefront kernel's 9 chunks in
    // flight per CU.
    if constexpr (APPLY) {
        if (n_peers <= kPeersPerLoad * 3) {
            constexpr size_t kStatic = sizeof(float) * SL_CHUNK + sizeof(uint32_t) * (kPeersPerLoad + 1) * kRecWords;
            static_assert(cap_is_exact(5, kStatic) && cap_is_exact(7, kStatic), "residency caps");
            const void* k4 = n_peers <= kPeersPerLoad * 1 ? reinterpret_cast<const void*>(&aggregate_apply4_kernel<1>)
                             : n_peers <= kPeersPerLoad * 2 ? reinterpret_cast<const void*>(&aggregate_apply4_kernel<2>)
                                                            : reinterpret_cast<const void*>(&aggregate_apply4_kernel<3>);
            const int cap = n_peers <= kPeersPerLoad * 2 ? 5 : 7;
            return hipLaunchKernel(k4, grid, dim3(kWave * kApplyWaves), args, residency_lds(cap, kStatic), stream);
        }
    }
    if constexpr (!APPLY) {
        if ((uint64_t)n_peers * (uint64_t)n_chunks * (SL_PAYLOAD_BYTES + sizeof(float)) > kCachedRecordBytes) {
            const int R = n_peers <= kRunMaxPeers ? kChunksPerWave : n_peers <= kPairMaxPeers ? 2 : 1;
            const int64_t runs = (n_chunks + R - 1) / R;
            int64_t run_per_xcd = (runs + kXcds - 1) / kXcds;
            void* pargs[] = {(void*)&t, (void*)&n_peers, (void*)&dst, (void*)&n_chunks, (void*)&run_per_xcd};
            constexpr int R3 = kChunksPerWave;
            const void* kp = n_peers <= kPeersPerLoad * 1 ? reinterpret_cast<const void*>(&aggregate_run_kernel<1, R3>)
                             : n_peers <= kPeersPerLoad * 2 ? reinterpret_cast<const void*>(&aggregate_run_kernel<2, R3>)
                             : n_peers <= kPeersPerLoad * 3 ? reinterpret_cast<const void*>(&aggregate_run_kernel<3, R3>)
                             : n_peers <= kRunMaxPeers      ? reinterpret_cast<const void*>(&aggregate_run_kernel<6, R3>)
                             : n_peers <= kPairMaxPeers     ? reinterpret_cast<const void*>(&aggregate_run_kernel<9, 2>)
                                                            : reinterpret_cast<const void*>(&aggregate_run_kernel<15, 1>);
            return hipLaunchKernel(kp, dim3((unsigned)(run_per_xcd * kXcds)), dim3(kWave), pargs, 0, stream);
        }
    }
    return hipLaunchKernel(k, grid, dim3(kWave), args, 0, stream);
}

// One launch per kLaunchChunks chunks, each on its own slice of the records,
// scales and dense buffer.
template <bool APPLY>
hipError_t launch_aggregate_impl(const PeerTable& peers, int32_t n_peers, float* dst,
                                 int64_t n_chunks, hipStream_t stream) {
    for (int64_t c0 = 0; c0 < n_chunks; c0 += kLaunchChunks) {
        const int64_t m = n_chunks - c0 < kLaunchChunks ? n_chunks - c0 : kLaunchChunks;
        PeerTable t = {};
        for (int32_t p = 0; p < n_peers; ++p) {
            t.payload[p] = peers.payload[p] + (size_t)c0 * SL_PAYLOAD_BYTES;
            t.scales[p] = peers.scales[p] + c0;
        }
        const hipError_t e = launch_aggregate_one<APPLY>(t, n_peers, dst + (size_t)c0 * SL_CHUNK, m, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// One chunk per wavefront except from 28 to 54 peers, where two measured
// faster.  At 8192 x 28672 with records from HBM (two or four record sets
// alternated), in the linear order, one / two chunks per wavefront, us:
//   24 peers   189   201        36 peers   216   212        48 peers   241   221
//   55 peers   231   226        64 peers   229   244        81 peers   250   267
//   128 peers  343   363        decoder block, 24 peers: 686 / 731
// against, for the same records laid out per peer (sl_aggregate), 213-217,
// 237-240, 257-274, 267-297, 285-319, 318-356, 471-512 and 760-770.
hipError_t launch_interleaved_one(const uint8_t* records, const float* scales, int32_t n_peers, float* out,
                                  int64_t n_chunks, hipStream_t stream) {
    const int R = n_peers > kPeersPerLoad * 3 && n_peers <= kRunMaxPeers ? 2 : 1;
    const int64_t runs = (n_chunks + R - 1) / R;
    void* args[] = {(void*)&records, (void*)&scales, (void*)&n_peers, (void*)&out, (void*)&n_chunks};
    const void* k = n_peers <= kPeersPerLoad * 1 ? reinterpret_cast<const void*>(&aggregate_interleaved_kernel<1, 1>)
                    : n_peers <= kPeersPerLoad * 2 ? reinterpret_cast<const void*>(&aggregate_interleaved_kernel<2, 1>)
                    : n_peers <= kPeersPerLoad * 3 ? reinterpret_cast<const void*>(&aggregate_interleaved_kernel<3, 1>)
                    : n_peers <= kRunMaxPeers      ? reinterpret_cast<const void*>(&aggregate_interleaved_kernel<6, 2>)
                    : n_peers <= kPairMaxPeers     ? reinterpret_cast<const void*>(&aggregate_interleaved_kernel<9, 1>)
                                                   : reinterpret_cast<const void*>(&aggregate_interleaved_kernel<15, 1>);
    return hipLaunchKernel(k, dim3((unsigned)runs), dim3(kWave), args, 0, stream);
}

}  // namespace

hipError_t launch_aggregate(const PeerTable& peers, int32_t n_peers, float* out,
                            int64_t n_chunks, hipStream_t stream) {
    return launch_aggregate_impl<false>(peers, n_peers, out, n_chunks, stream);
}

hipError_t launch_aggregate_apply(const PeerTable& peers, int32_t n_peers, float* theta,
                                  int64_t n_chunks, hipStream_t stream) {
    return launch_aggregate_impl<true>(peers, n_peers, theta, n_chunks, stream);
}

// Fused update on interleaved records, with the same workgroup shapes and
// residency caps as the per-peer layout's fused update.
hipError_t launch_apply_interleaved_one(const uint8_t* records, const float* scales, int32_t n_peers, float* theta,
                                        int64_t n_chunks, hipStream_t stream) {
    float nf = (float)n_peers;
    void* args[] = {(void*)&records, (void*)&scales, (void*)&n_peers, (void*)&theta, (void*)&n_chunks, (void*)&nf};
    const dim3 grid((unsigned)n_chunks);
    if (n_peers <= kPeersPerLoad * 3) {
        constexpr size_t kStatic = sizeof(float) * SL_CHUNK + sizeof(uint32_t) * (kPeersPerLoad + 1) * kRecWords;
        const void* k4 = n_peers <= kPeersPerLoad * 1 ? reinterpret_cast<const void*>(&apply4_interleaved_kernel<1>)
                         : n_peers <= kPeersPerLoad * 2 ? reinterpret_cast<const void*>(&apply4_interleaved_kernel<2>)
                                                        : reinterpret_cast<const void*>(&apply4_interleaved_kernel<3>);
        const int cap = n_peers <= kPeersPerLoad * 2 ? 5 : 7;
        return hipLaunchKernel(k4, grid, dim3(kWave * kApplyWaves), args, residency_lds(cap, kStatic), stream);
    }
    const void* k = n_peers <= kRunMaxPeers    ? reinterpret_cast<const void*>(&apply_interleaved_kernel<6>)
                    : n_peers <= kPairMaxPeers ? reinterpret_cast<const void*>(&apply_interleaved_kernel<9>)
                                               : reinterpret_cast<const void*>(&apply_interleaved_kernel<15>);
    return hipLaunchKernel(k, grid, dim3(kWave), args, 0, stream);
}

// Split like the streaming kernels (the chunks are taken in linear order):
// the 16e9-parameter span, 24 peers, ran 12.76 ms = 0.733 of HBM in 60
// launches against 13.22 ms = 0.708 in one.
hipError_t launch_aggregate_interleaved(const uint8_t* records, const float* scales, int32_t n_peers, float* out,
                                        int64_t n_chunks, hipStream_t stream) {
    const int64_t per = stream_launch_chunks(n_chunks);
    for (int64_t c0 = 0; c0 < n_chunks; c0 += per) {
        const int64_t m = n_chunks - c0 < per ? n_chunks - c0 : per;
        const hipError_t e = launch_interleaved_one(records + (size_t)c0 * (size_t)n_peers * SL_PAYLOAD_BYTES,
                                                    scales + (size_t)c0 * (size_t)n_peers, n_peers,
                                                    out + (size_t)c0 * SL_CHUNK, m, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

// Split like the streaming kernels: at the decoder block, 24 and 36 peers,
// four launches measured 0.785-0.787 and 0.760-0.763 of HBM against
// 0.756-0.759 and 0.736-0.742 in one (records from HBM).
hipError_t launch_aggregate_apply_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                              float* theta, int64_t n_chunks, hipStream_t stream) {
    const int64_t per = stream_launch_chunks(n_chunks);
    for (int64_t c0 = 0; c0 < n_chunks; c0 += per) {
        const int64_t m = n_chunks - c0 < per ? n_chunks - c0 : per;
        const hipError_t e = launch_apply_interleaved_one(records + (size_t)c0 * (size_t)n_peers * SL_PAYLOAD_BYTES,
                                                          scales + (size_t)c0 * (size_t)n_peers, n_peers,
                                                          theta + (size_t)c0 * SL_CHUNK, m, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n,
                             hipStream_t stream) {
    const int64_t n_chunks = n / SL_CHUNK;
    float nf = (float)n_peers;
    const int64_t per = stream_launch_chunks(n_chunks);
    for (int64_t c0 = 0; c0 < n_chunks; c0 += per) {
        int64_t m = n_chunks - c0 < per ? n_chunks - c0 : per;
        float* st = theta + (size_t)c0 * SL_CHUNK;
        const float* so = out + (size_t)c0 * SL_CHUNK;
        void* args[] = {(void*)&st, (void*)&so, (void*)&nf, (void*)&m};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&apply_mean_kernel), dim3((unsigned)m),
                                             dim3(kWave * kMeanWaves), args, residency_lds(kCapApplyMean, 0), stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sl
