// compress.hip -- the SparseLoCo compressor kernel for gfx950.
//
// One pass over each 4096-parameter chunk ("The Sparse Frontier: SparseLoCo and
// the Compression Math Behind Permissionless Pre-Training", section "SparseLoCo:
// Three Compression Levers in One Pass"): error-feedback update, top-64 by
// |value|, per-chunk scale with four 2-bit levels, 12-bit indices packed into a
// 112-byte record, and the residual written back to the error-feedback buffer
// (same page, "Why Extreme Sparsity Doesn't Break Convergence").
//
// Mapping: one workgroup of four 64-lane wavefronts owns one chunk.
// Wavefront w holds elements 1024 w + 256 m + 4 l + j (m, j = 0..3) in 16
// registers per lane, so every global load and store instruction touches one
// contiguous KiB.  The selection's partial results cross wavefronts through
// LDS (11.3 KiB, a region per phase) and workgroup barriers; no barrier ties
// workgroups together.  (On 8192 x 28672 parameters four wavefronts per chunk
// measured 5% faster than one, which needs 167 registers per lane and runs
// three wavefronts per SIMD; two and eight wavefronts per chunk were slower
// than four.)  A residency cap keeps at most 6 workgroups on a CU (5 for the
// weights variant), see the launchers.
//
// Selection (exact, deterministic): find the 64th element of the order
// (|acc| descending, index ascending) -- the "cut" -- by an MSB-first radix
// select over the 31-bit magnitude key bits(acc) & 0x7fffffff:
//   level 0  2048-bin LDS histogram of key bits 30..20 (exponent + 3 mantissa
//            bits), shared by the four wavefronts.  Exact zeros are counted
//            with ballots instead of atomics.
//   then     if the boundary bin holds exactly the entries still needed, the
//            cut is "key >= bin start"; if it holds at most 64 entries, they
//            are compacted to LDS and ranked exactly by (key, index) with
//            cross-lane reads; otherwise refine with 1024-bin histograms of
//            key bits 19..10 and 9..0, and finally by index among equal keys.
// An all-zero chunk (max key 0) keeps indices 0..63 directly.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "residency.h"
#include "sparseloco.h"
#include "wave.h"

namespace sl {
namespace {

constexpr int kWaves = 4;                      // wavefronts per chunk
constexpr int kThreads = kWave * kWaves;
constexpr int kPerLane = SL_CHUNK / kThreads;  // 16 elements per lane
constexpr int kSlots = kPerLane / 4;           // 4 float4 per lane
constexpr int kSpan = SL_CHUNK / kWaves;       // 1024 elements per wavefront
constexpr int kLdsWords = 2048;
constexpr uint32_t kKeyMask = 0x7fffffffu;
constexpr uint32_t kSignBit = 0x80000000u;

static_assert(SL_TOPK == kWave, "one kept entry per lane");
static_assert(SL_INDEX_BITS == 12 && SL_CODE_BITS == 2, "payload layout");
// Every phase has LDS of its own, so a phase never waits for the previous
// one's readers before writing: the common path (boundary bin of at most 64
// entries) crosses five workgroup barriers.
struct Shared {
    uint32_t hist[kLdsWords];        // level-0 histogram; refinement histograms reuse it
    uint32_t cand[SL_TOPK * kWaves]; // candidates, wavefront w's at [64 w, 64 w + 64); or the index bitmap
    uint32_t ent[SL_TOPK * kWaves];  // kept entries, same segments
    uint32_t bmp[SL_CHUNK / 32];     // packing: index bitmap
    uint32_t pre[SL_TOPK];           //          per-64-index prefix counts
    uint32_t sorted[SL_TOPK];        //          entries in index order
    uint32_t part_max[kWaves];       // per-wavefront maximum key
    uint32_t part_cnt[kWaves];       // per-wavefront candidate count
    uint32_t part_sel[kWaves];       // per-wavefront kept-entry count
    uint32_t cut[3];                 // the cut, broadcast by wavefront 0
};

__device__ __forceinline__ uint32_t key_of(float v) { return __float_as_uint(v) & kKeyMask; }

// In-chunk index of register slot q = 4 m + j of lane `lane` in wavefront w.
__device__ __forceinline__ uint32_t elem_index(int w, int q, int lane) {
    return (uint32_t)(kSpan * w + 256 * (q >> 2) + 4 * lane + (q & 3));
}

// The kept set is {x : key > key_cut} plus, when tie is set, the entries with
// key == key_cut and index <= idx_cut; without tie it is {x : key >= key_cut}.
struct Cut {
    uint32_t key;
    uint32_t idx;
    bool tie;
};

struct Boundary {
    uint32_t digit;  // histogram bin holding the cut
    uint32_t above;  // entries in higher bins
    uint32_t count;  // entries in the bin itself
};

__device__ __forceinline__ void clear_shared(uint32_t* p, int words, int tid) {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid * 4; i < words; i += kThreads * 4) *reinterpret_cast<uint4*>(p + i) = z;
}

// Bin d with count(bins > d) < need <= count(bins >= d).  Lane l owns bins
// [l*B, l*B + B); each lane reads its bins starting at a lane-dependent
// rotation so that the 16-byte reads spread over the LDS banks.  Every
// wavefront computes the same answer from the same histogram.
template <int B>
__device__ __forceinline__ Boundary find_boundary(const uint32_t* hist, uint32_t need, int lane) {
    static_assert(B % 4 == 0 && ((B / 4) & (B / 4 - 1)) == 0, "bins per lane");
    // Each call recomputes its addresses: kept live across the refinement
    // passes between two calls, they would cost registers.
    int rl = lane;
    asm volatile("" : "+v"(rl));
    uint32_t sum = 0;
    const uint4* h4 = reinterpret_cast<const uint4*>(hist + rl * B);
#pragma unroll
    for (int r = 0; r < B / 4; ++r) {
        const uint4 v = h4[(r + rl) & (B / 4 - 1)];
        sum += v.x + v.y + v.z + v.w;
    }
    const uint32_t S = wave_suffix_sum(sum);
    int L = __popcll(ballot(S >= need)) - 1;
    L = L < 0 ? 0 : L;
    const uint32_t above_lane = read_lane(S, L) - read_lane(sum, L);
    const uint32_t h = lane < B ? hist[L * B + lane] : 0u;
    const uint32_t T = wave_suffix_sum(h);
    int t = __popcll(ballot(lane < B && T + above_lane >= need)) - 1;
    t = t < 0 ? 0 : t;
    Boundary b;
    b.count = read_lane(h, t);
    b.digit = (uint32_t)(L * B + t);
    b.above = above_lane + read_lane(T, t) - b.count;
    return b;
}

// The cut written by wavefront 0, read by every wavefront after a barrier.
__device__ __forceinline__ Cut broadcast_cut(const Shared& sh) {
    __syncthreads();
    Cut c;
    c.key = sh.cut[0];
    c.idx = sh.cut[1];
    c.tie = sh.cut[2] != 0u;
    return c;
}

// Histogram of key bits [SHIFT, SHIFT+10) over entries whose resolved bits
// match prefix.  A slot where every matching lane falls in the same bin adds
// its count with one atomic (heavy ties, e.g. many exact zeros).
template <int SHIFT>
__device__ __forceinline__ void refine_histogram(const float (&acc)[kPerLane], uint32_t* hist, uint32_t pmask,
                                                 uint32_t prefix, int lane) {
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const uint32_t k = key_of(acc[q]);
        const bool c = (k & pmask) == prefix;
        const uint64_t bm = ballot(c);
        if (bm) {
            const uint32_t bin = (k >> SHIFT) & 1023u;
            const int first = __ffsll((unsigned long long)bm) - 1;
            const uint32_t b0 = read_lane(bin, first);
            const uint64_t same = ballot(c && bin == b0);
            if (same == bm) {
                if (lane == first) block_lds_add(&hist[b0], (uint32_t)__popcll(bm));
            } else if (c) {
                block_lds_add(&hist[bin], 1u);
            }
        }
    }
}

// Entry j (0..63) of the concatenation of the four wavefronts' segments, with
// count[v] entries in segment v: segment and offset.
__device__ __forceinline__ uint32_t segment_slot(const uint32_t* count, uint32_t j) {
    uint32_t seg = 0, first = 0, start = 0;
    for (int v = 0; v < kWaves; ++v) {
        if (j >= start) {
            seg = (uint32_t)v;
            first = start;
        }
        start += count[v];
    }
    return SL_TOPK * seg + ((j - first) & (SL_TOPK - 1));
}

// At most 64 candidates (resolved bits == prefix) across the four wavefronts:
// each wavefront compacts its own into its segment of sh.cand; wavefront 0
// ranks them all by (key descending, index ascending) and broadcasts the one
// at position need-1.  Candidates share the resolved bits, so (low key bits,
// 4095 - index) fits one 32-bit sort word.
__device__ __forceinline__ Cut rank_cut(const float (&acc)[kPerLane], Shared& sh, uint32_t pmask, uint32_t prefix,
                                        uint32_t lowmask, uint32_t need, uint32_t cnt, int w, int lane) {
    uint32_t* seg = sh.cand + SL_TOPK * w;
    uint32_t mine = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const uint32_t k = key_of(acc[q]);
        const bool c = (k & pmask) == prefix;
        const uint64_t bm = ballot(c);
        if (bm) {
            const uint32_t pos = mine + lanes_below(bm);
            if (c && pos < (uint32_t)SL_TOPK) seg[pos] = ((k & lowmask) << 12) | (4095u - elem_index(w, q, lane));
            mine += (uint32_t)__popcll(bm);
        }
    }
    if (lane == 0) sh.part_cnt[w] = mine;
    __syncthreads();
    if (w == 0) {
        const bool mine_c = (uint32_t)lane < cnt;
        const uint32_t sk = mine_c ? sh.cand[segment_slot(sh.part_cnt, (uint32_t)lane)] : 0u;
        uint32_t rank = 0;
        for (uint32_t f = 0; f < cnt; ++f) rank += read_lane(sk, (int)f) > sk ? 1u : 0u;
        const uint64_t hit = ballot(mine_c && rank == need - 1u);
        const int wl = hit ? __ffsll((unsigned long long)hit) - 1 : 0;
        const uint32_t sk_cut = read_lane(sk, wl);
        const uint64_t same = ballot(mine_c && (sk >> 12) == (sk_cut >> 12));
        if (lane == 0) {
            sh.cut[0] = prefix | (sk_cut >> 12);
            sh.cut[1] = 4095u - (sk_cut & 4095u);
            sh.cut[2] = __popcll(same) > 1 ? 1u : 0u;
        }
    }
    return broadcast_cut(sh);
}

// More than 64 entries share the exact key K: a 4096-bit LDS bitmap of their
// indices from all four wavefronts; wavefront 0 finds the need-th smallest.
__device__ __forceinline__ Cut index_cut(const float (&acc)[kPerLane], Shared& sh, uint32_t K, uint32_t need,
                                         int w, int lane, int tid) {
    if (tid < kWave) reinterpret_cast<uint2*>(sh.cand)[tid] = make_uint2(0u, 0u);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        if (key_of(acc[q]) == K) {
            const uint32_t i = elem_index(w, q, lane);
            block_lds_or(&sh.cand[i >> 5], 1u << (i & 31));
        }
    }
    __syncthreads();
    if (w == 0) {
        const uint2 wv = reinterpret_cast<const uint2*>(sh.cand)[lane];  // indices [64l, 64l+64)
        const uint64_t wd = ((uint64_t)wv.y << 32) | wv.x;
        const uint32_t c = (uint32_t)__popcll(wd);
        const uint32_t incl = wave_prefix_sum(c);
        const uint64_t reach = ballot(incl >= need);
        const int L = reach ? __ffsll((unsigned long long)reach) - 1 : 0;
        const uint32_t r = need - (read_lane(incl, L) - read_lane(c, L));  // 1..64
        uint64_t wl = ((uint64_t)read_lane(wv.y, L) << 32) | read_lane(wv.x, L);
        for (uint32_t i = 1; i < r && i < 64u; ++i) wl &= wl - 1;
        if (lane == 0) {
            sh.cut[0] = K;
            sh.cut[1] = 64u * (uint32_t)L + (uint32_t)__builtin_ctzll(wl);
            sh.cut[2] = 1u;
        }
    }
    return broadcast_cut(sh);
}

// Every wavefront returns the same cut.  The level-0 histogram was cleared
// before the barrier that published the wavefronts' maxima.
__device__ __forceinline__ Cut select_cut(const float (&acc)[kPerLane], Shared& sh, uint32_t mx, int w, int lane,
                                          int tid) {
    Cut cut;
    cut.idx = 0u;
    cut.tie = false;
    if (mx == 0u) {  // all keys are 0: the lower-index rule keeps 0..63
        cut.key = 0u;
        cut.idx = 63u;
        cut.tie = true;
        return cut;
    }
    // Level 0: key bits 30..20.
    uint32_t zeros = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const uint32_t k = key_of(acc[q]);
        const bool nz = k != 0u;
        zeros += (uint32_t)(kWave - __popcll(ballot(nz)));
        if (nz) block_lds_add(&sh.hist[k >> 20], 1u);
    }
    if (lane == 0 && zeros) block_lds_add(&sh.hist[0], zeros);
    __syncthreads();
    Boundary b = find_boundary<kLdsWords / kWave>(sh.hist, (uint32_t)SL_TOPK, lane);
    uint32_t need = (uint32_t)SL_TOPK - b.above;
    uint32_t prefix = b.digit << 20;
    uint32_t pmask = 0x7ff00000u;
    if (b.count == need) {
        cut.key = prefix;
        return cut;
    }
    if (b.count <= (uint32_t)kWave) return rank_cut(acc, sh, pmask, prefix, 0x000fffffu, need, b.count, w, lane);

    // Level 1: key bits 19..10 of the boundary bin.  The histogram is reused
    // once every wavefront has read it.
    __syncthreads();
    clear_shared(sh.hist, 1024, tid);
    __syncthreads();
    refine_histogram<10>(acc, sh.hist, pmask, prefix, lane);
    __syncthreads();
    b = find_boundary<1024 / kWave>(sh.hist, need, lane);
    need -= b.above;
    prefix |= b.digit << 10;
    pmask = 0x7ffffc00u;
    if (b.count == need) {
        cut.key = prefix;
        return cut;
    }
    if (b.count <= (uint32_t)kWave) return rank_cut(acc, sh, pmask, prefix, 0x3ffu, need, b.count, w, lane);

    // Level 2: key bits 9..0.
    __syncthreads();
    clear_shared(sh.hist, 1024, tid);
    __syncthreads();
    refine_histogram<0>(acc, sh.hist, pmask, prefix, lane);
    __syncthreads();
    b = find_boundary<1024 / kWave>(sh.hist, need, lane);
    need -= b.above;
    prefix |= b.digit;
    pmask = kKeyMask;
    if (b.count == need) {
        cut.key = prefix;
        return cut;
    }
    if (b.count <= (uint32_t)kWave) return rank_cut(acc, sh, pmask, prefix, 0u, need, b.count, w, lane);
    return index_cut(acc, sh, prefix, need, w, lane, tid);
}

// Smallest key k with 3 * value(k) > 2s, so that "magnitude bit set" is the
// integer test key >= k.  Decided in binary64, where 3v and 2s are exact.  The
// start is within one step of the answer for finite s; the bounds keep a
// non-finite s (outside the contract) from looping.
__device__ __forceinline__ uint32_t magnitude_threshold(float s) {
    const double two_s = 2.0 * (double)s;
    uint32_t k = __float_as_uint((float)(two_s / 3.0)) & kKeyMask;
    for (int i = 0; i < 4 && k > 0u && 3.0 * (double)__uint_as_float(k - 1u) > two_s; ++i) --k;
    for (int i = 0; i < 4 && !(3.0 * (double)__uint_as_float(k) > two_s); ++i) ++k;
    return k;
}

// Spread the 16 low bits of x to the even bit positions of a 32-bit word.
__device__ __forceinline__ uint32_t spread16(uint32_t x) {
    x = (x | (x << 8)) & 0x00ff00ffu;
    x = (x | (x << 4)) & 0x0f0f0f0fu;
    x = (x | (x << 2)) & 0x33333333u;
    x = (x | (x << 1)) & 0x55555555u;
    return x;
}

typedef float v4f __attribute__((ext_vector_type(4)));

// Streaming accesses: delta, ef and the records are touched once per round,
// so loads and stores carry the nontemporal hint.
__device__ __forceinline__ float4 stream_load(const float* p) {
    const v4f v = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void stream_store(float* p, float a, float b, float c, float d) {
    const v4f v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<v4f*>(p));
}

// Residual write-back of this wavefront's 1024 elements (ef_part points at
// the first) and compaction of its kept entries (index | code << 12) into ent.
template <bool TIE>
__device__ __forceinline__ uint32_t write_residual(const float (&acc)[kPerLane], const Cut& cut, uint32_t kmag,
                                                   uint32_t sbits, uint32_t s3bits, float* ef_part, uint32_t* ent,
                                                   int w, int lane) {
    uint32_t nsel = 0;
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = 4 * m + j;
            const uint32_t bits = __float_as_uint(acc[q]);
            const uint32_t k = bits & kKeyMask;
            const uint32_t idx = elem_index(w, q, lane);
            const bool sel = TIE ? (k > cut.key || (k == cut.key && idx <= cut.idx)) : (k >= cut.key);
            const bool mag = k >= kmag;
            const uint32_t dbits = (mag ? sbits : s3bits) | (bits & kSignBit);
            const float r = acc[q] - __uint_as_float(dbits);
            o[j] = sel ? r : acc[q];
            const uint64_t bm = ballot(sel);
            if (bm) {
                const uint32_t pos = nsel + lanes_below(bm);
                if (sel && pos < (uint32_t)SL_TOPK) ent[pos] = idx | ((((bits >> 31) << 1) | (mag ? 1u : 0u)) << 12);
                nsel += (uint32_t)__popcll(bm);
            }
        }
        stream_store(ef_part + 4 * (m * kWave + lane), o[0], o[1], o[2], o[3]);
    }
    return nsel;
}

// Entry e (index | code << 12, one per lane, any order) of the 64 kept
// entries: order them by index with a counting sort through a 4096-bit bitmap
// and write the 112-byte record (24 dwords of 12-bit indices, then 4 dwords of
// 2-bit codes).  bmp (128 words), pre (64) and sorted (64) are LDS scratch
// that only the calling wavefront touches.
__device__ __forceinline__ void order_and_pack(uint32_t e, uint32_t* bmp, uint32_t* pre, uint32_t* sorted,
                                               uint8_t* record, int lane) {
    reinterpret_cast<uint2*>(bmp)[lane] = make_uint2(0u, 0u);
    wave_sync();
    const uint32_t id = e & 4095u;
    lds_or(&bmp[id >> 5], 1u << (id & 31));
    wave_sync();
    const uint2 wv = reinterpret_cast<const uint2*>(bmp)[lane];
    const uint32_t cnt = (uint32_t)__popcll(((uint64_t)wv.y << 32) | wv.x);
    pre[lane] = wave_prefix_sum(cnt) - cnt;
    wave_sync();
    const uint2 gv = reinterpret_cast<const uint2*>(bmp)[id >> 6];
    const uint64_t gw = ((uint64_t)gv.y << 32) | gv.x;
    const uint32_t rank = pre[id >> 6] + (uint32_t)__popcll(gw & ((1ull << (id & 63)) - 1ull));
    sorted[rank & 63u] = e;
    wave_sync();
    const uint32_t es = sorted[lane];

    uint32_t word = 0;
    if (lane < 24) {
        const int j0 = (32 * lane) / 12;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int j = j0 + t;
            const int off = 12 * j - 32 * lane;
            if (j < SL_TOPK && off < 32) {
                const uint32_t v = sorted[j] & 4095u;
                word |= off >= 0 ? (v << off) : (v >> (-off));
            }
        }
    }
    const uint32_t code = es >> 12;
    const uint64_t bmag = ballot((code & 1u) != 0u);
    const uint64_t bsgn = ballot((code & 2u) != 0u);
    if (lane >= 24 && lane < 28) {
        const int q = lane - 24;
        word = spread16((uint32_t)(bmag >> (16 * q)) & 0xffffu) |
               (spread16((uint32_t)(bsgn >> (16 * q)) & 0xffffu) << 1);
    }
    if (lane < SL_PAYLOAD_BYTES / 4) reinterpret_cast<uint32_t*>(record)[lane] = word;
}

// One chunk per workgroup.  WEIGHTS: delta = a - b is formed on the fly with
// one fp32 subtraction, a = theta_pre and b = theta_post (pseudo-gradient as in
// "The Sparse Frontier", section "Why DiLoCo Alone Isn't Enough"; the sign,
// pre minus post, is a reading); otherwise a is delta and b is unused.  Then
// acc = beta * ef + delta with one rounding.
template <bool WEIGHTS>
__global__ __launch_bounds__(kThreads) void compress_kernel(const float* a, const float* b, float* ef, float beta,
                                                            uint8_t* payload, float* scales, int64_t n_chunks) {
    __shared__ __align__(16) Shared sh;
    const int tid = (int)threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t chunk = (int64_t)blockIdx.x;
    if (chunk >= n_chunks) return;  // the whole workgroup
    const size_t base = (size_t)chunk * SL_CHUNK + (size_t)kSpan * (size_t)w;
    float acc[kPerLane];
#pragma unroll
    for (int m = 0; m < kSlots; ++m) {
        const size_t off = base + 4 * (size_t)(m * kWave + lane);
        float4 dv = stream_load(a + off);
        if constexpr (WEIGHTS) {
            const float4 bv = stream_load(b + off);
            dv = make_float4(dv.x - bv.x, dv.y - bv.y, dv.z - bv.z, dv.w - bv.w);
        }
        const float4 ev = stream_load(ef + off);
        acc[4 * m + 0] = __builtin_fmaf(beta, ev.x, dv.x);
        acc[4 * m + 1] = __builtin_fmaf(beta, ev.y, dv.y);
        acc[4 * m + 2] = __builtin_fmaf(beta, ev.z, dv.z);
        acc[4 * m + 3] = __builtin_fmaf(beta, ev.w, dv.w);
    }

    // Scale: s = max |acc| over the chunk (= the largest kept magnitude).
    uint32_t mx = 0;
#pragma unroll
    for (int q = 0; q < kPerLane; ++q) {
        const uint32_t k = key_of(acc[q]);
        mx = k > mx ? k : mx;
    }
    mx = wave_max(mx);
    clear_shared(sh.hist, kLdsWords, tid);
    if (lane == 0) sh.part_max[w] = mx;
    __syncthreads();
    for (int v = 0; v < kWaves; ++v) mx = sh.part_max[v] > mx ? sh.part_max[v] : mx;

    const Cut cut = select_cut(acc, sh, mx, w, lane, tid);

    const float s = __uint_as_float(mx);
    const float s3 = s / 3.0f;
    const uint32_t kmag = magnitude_threshold(s);
    uint32_t* ent = sh.ent + SL_TOPK * w;  // this wavefront's kept entries
    const uint32_t nsel =
        cut.tie ? write_residual<true>(acc, cut, kmag, __float_as_uint(s), __float_as_uint(s3), ef + base, ent, w, lane)
                : write_residual<false>(acc, cut, kmag, __float_as_uint(s), __float_as_uint(s3), ef + base, ent, w, lane);
    if (lane == 0) sh.part_sel[w] = nsel;
    __syncthreads();
    if (w == 0) {
        const uint32_t e = sh.ent[segment_slot(sh.part_sel, (uint32_t)lane)];
        order_and_pack(e, sh.bmp, sh.pre, sh.sorted, payload + (size_t)chunk * SL_PAYLOAD_BYTES, lane);
        if (lane == 0) scales[chunk] = s;
    }
}

// Residency caps (workgroups per CU, through unused dynamic LDS).  On
// 8192 x 28672 parameters the weights variant, with three input streams, ran
// 611-623 us uncapped (8 workgroups per CU) and 580-587 us at 4 or 5; the
// compressor gained less from 6 (medians 461 -> 451 us; 4 or 5 lost 6%).
constexpr int kCapCompress = 6;
constexpr int kCapWeights = 5;
static_assert(cap_is_exact(kCapCompress, sizeof(Shared)) && cap_is_exact(kCapWeights, sizeof(Shared)),
              "residency caps");

// Equal launches of at most kStreamLaunchChunks chunks, each on its own slice
// of every buffer.
template <bool WEIGHTS>
hipError_t launch_segments(const float* a, const float* b, float* ef, float beta, uint8_t* payload, float* scales,
                           int64_t n_chunks, int cap, hipStream_t stream) {
    const int64_t per = stream_launch_chunks(n_chunks);
    for (int64_t c0 = 0; c0 < n_chunks; c0 += per) {
        const int64_t m = n_chunks - c0 < per ? n_chunks - c0 : per;
        const size_t e0 = (size_t)c0 * SL_CHUNK;
        const float* sa = a + e0;
        const float* sb = WEIGHTS ? b + e0 : b;
        float* sef = ef + e0;
        uint8_t* sp = payload + (size_t)c0 * SL_PAYLOAD_BYTES;
        float* ss = scales + c0;
        void* args[] = {(void*)&sa, (void*)&sb, (void*)&sef, (void*)&beta, (void*)&sp, (void*)&ss, (void*)&m};
        const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&compress_kernel<WEIGHTS>),
                                             dim3((unsigned)m), dim3(kThreads), args, residency_lds(cap, sizeof(Shared)),
                                             stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_compress_weights(const float* theta_pre, const float* theta_post, float* ef,
                                   float beta, uint8_t* payload, float* scales, int64_t n_chunks,
                                   hipStream_t stream) {
    return launch_segments<true>(theta_pre, theta_post, ef, beta, payload, scales, n_chunks, kCapWeights, stream);
}

hipError_t launch_compress(const float* delta, float* ef, float beta, uint8_t* payload,
                           float* scales, int64_t n_chunks, hipStream_t stream) {
    return launch_segments<false>(delta, nullptr, ef, beta, payload, scales, n_chunks, kCapCompress, stream);
}

}  // namespace sl
