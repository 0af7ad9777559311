/*
 * sparseloco.h -- C ABI of libsparseloco.so: the SparseLoCo pseudo-gradient
 * compressor and its aggregator, hand-written HIP for AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *  [SF] "The Sparse Frontier: SparseLoCo and the Compression Math Behind
 *       Permissionless Pre-Training" (blokz.dev)
 *  [CV] "Covenant-72B: Decentralized Training is No Longer Just a Dream"
 *       (wispaper.ai)
 *
 * Conventions for every entry point:
 *  - All buffer pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no state between calls and is reentrant.
 *  - `stream` is a hipStream_t (NULL = the default stream), declared as void*
 *    so that this header compiles as plain C99 without the HIP headers.  Work
 *    is enqueued on it and the call returns before the GPU finishes;
 *    synchronise the stream before reading outputs.
 *  - Argument errors are detected on the host before anything is enqueued and
 *    returned as a status; SL_ERR_HIP reports a launch failure.
 *  - Element counts are int64; n must be a multiple of SL_CHUNK.
 *  - Inputs must be finite: NaN and Inf are outside the contract (they are
 *    not detected and give unspecified codes, never out-of-bounds accesses).
 *  - Results do not depend on the launch configuration: each chunk is owned by
 *    one workgroup and no floating-point atomics are used, so repeated calls
 *    are bitwise identical.
 */
#ifndef SPARSELOCO_H
#define SPARSELOCO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* [SF] "Three Compression Levers", lever 1: non-overlapping chunks of 4,096
 * parameters, the top 64 kept.  Lever 3: 12-bit in-chunk index.  Lever 2: four
 * 2-bit levels.  Layout formula: 64 x (2 + 12) bits = 112 bytes per chunk. */
#define SL_CHUNK 4096
#define SL_TOPK 64
#define SL_INDEX_BITS 12
#define SL_CODE_BITS 2
#define SL_INDEX_BYTES 96     /* 64 x 12 bits */
#define SL_CODE_BYTES 16      /* 64 x 2 bits */
#define SL_PAYLOAD_BYTES 112  /* SL_INDEX_BYTES + SL_CODE_BYTES */

/* Peers per sl_aggregate call.  [SF] "Three Compression Levers" reports 24.4
 * active peers on average out of 70+ unique participants. */
#define SL_MAX_PEERS 128

#define SL_DEFAULT_BETA 0.95f

typedef enum {
    SL_OK = 0,
    SL_ERR_INVALID_ARG = 1,    /* null pointer, non-finite beta, aliasing */
    SL_ERR_SHAPE = 2,          /* n < 0 or n % SL_CHUNK != 0 */
    SL_ERR_ALIGN = 3,          /* a buffer is not aligned as documented */
    SL_ERR_TOO_MANY_PEERS = 4, /* n_peers outside the allowed range */
    SL_ERR_HIP = 5             /* the HIP runtime reported a launch error */
} sl_status;

/*
 * sl_compress -- one SparseLoCo compression round over n parameters.
 *
 * Computes, for every chunk c of SL_CHUNK consecutive elements:
 *   acc[i]   = fma(beta, ef[i], delta[i])       error feedback ([SF] "Why
 *              Extreme Sparsity Doesn't Break Convergence", error-feedback
 *              paragraph; beta = 1 is the pages' plain accumulation, the decay
 *              beta and its single rounding are readings)
 *   keep the SL_TOPK entries of largest |acc| ([SF] lever 1); ties at the cut
 *              go to the lower index (reading)
 *   s        = max |acc| over the chunk (the per-chunk scale of [SF] lever 2;
 *              reading: the largest kept magnitude)
 *   code     = (signbit(acc) << 1) | (3|acc| > 2s)   four levels {-s, -s/3,
 *              +s/3, +s}, s/3 correctly rounded (reading of [SF] lever 2)
 *   ef[i]    = acc[i] - decoded[i] where kept, acc[i] elsewhere (the
 *              untransmitted remainder rolls into the next round)
 *
 * delta    in   float32[n], 16-byte aligned, read only
 * ef       in/out float32[n], 16-byte aligned, updated in place; may be the
 *          same pointer as delta, must not otherwise overlap it
 * beta     in   finite decay of the error-feedback buffer (default 0.95)
 * payload  out  uint8[n/4096][112], 16-byte aligned.  Chunk c's record holds
 *          the 64 kept in-chunk indices in ascending order as 12-bit fields,
 *          entry j at bits [12j, 12j+12) of bytes 0..95, then the 64 codes as
 *          2-bit fields, entry j at bits [2j, 2j+2) of bytes 96..111; both are
 *          little-endian, least-significant-bit-first bit streams
 * scales   out  float32[n/4096], 4-byte aligned: s of each chunk (not part of
 *          the 112-byte record; [SF] prices the payload without it)
 * n        number of parameters, a multiple of SL_CHUNK (0 is a no-op)
 *
 * payload and scales must not overlap delta or ef.
 */
sl_status sl_compress(const float* delta, float* ef, float beta, uint8_t* payload,
                      float* scales, int64_t n, void* stream);

/*
 * sl_compress_weights -- sl_compress with the pseudo-gradient formed on the fly.
 *
 * The step before compression ([SF], section "Why DiLoCo Alone Isn't Enough",
 * which defines the pseudo-gradient from the weights on either side of the
 * inner loop).  Reading: delta[i] = theta_pre[i] - theta_post[i] (one fp32
 * subtraction), then exactly sl_compress(delta, ef, ...), so the results are
 * bitwise those of materialising delta first; delta never reaches HBM.
 *
 * theta_pre, theta_post  in  float32[n], 16-byte aligned, read only (may alias
 *          each other)
 * ef, beta, payload, scales, n   as for sl_compress; ef, payload and scales must
 *          not overlap any other buffer
 */
sl_status sl_compress_weights(const float* theta_pre, const float* theta_post, float* ef,
                              float beta, uint8_t* payload, float* scales, int64_t n,
                              void* stream);

/*
 * sl_aggregate -- decode n_peers payloads and sum them into a dense update.
 *
 * [SF] "Why Extreme Sparsity Doesn't Break Convergence", sparse-aggregation
 * paragraph: the receivers combine the union of the peers' selected
 * coordinates.  Reading: the result is the plain sum,
 * accumulated from +0.0 in ascending peer order for every coordinate, in fp32
 * with round-to-nearest-even.  out[i] is +0.0 where no peer selected i.
 *
 * payloads in  HOST array of n_peers DEVICE pointers, each uint8[n/4096][112]
 *          in the sl_compress layout, 16-byte aligned
 * scales   in  HOST array of n_peers DEVICE pointers, each float32[n/4096]
 * n_peers  0..SL_MAX_PEERS (0 writes all +0.0)
 * out      out float32[n], 16-byte aligned, fully overwritten; must not overlap
 *          any payload or scale buffer
 * n        number of parameters, a multiple of SL_CHUNK
 *
 * Payloads are trusted: malformed records (non-increasing indices, negative or
 * non-finite scales) give unspecified values but every access stays inside the
 * chunk's own 4096 outputs, since a 12-bit field cannot leave the chunk.  Use
 * sl_validate_payloads (or sl_validate_payload) for records from untrusted
 * peers.
 */
sl_status sl_aggregate(const uint8_t* const* payloads, const float* const* scales,
                       int32_t n_peers, float* out, int64_t n, void* stream);

/*
 * sl_aggregate_apply_interleaved -- sl_aggregate_apply with the records laid
 * out chunk-major across peers, as for sl_aggregate_interleaved.
 *
 * Same reading and the same results, bit for bit, as sl_aggregate_apply on
 * the per-peer buffers: theta[i] <- theta[i] - out[i] / n_peers.
 *
 * records, scales  as for sl_aggregate_interleaved
 * n_peers  1..SL_MAX_PEERS, else SL_ERR_TOO_MANY_PEERS
 * theta    in/out float32[n], 16-byte aligned; must not overlap records or
 *          scales
 * n        number of parameters, a multiple of SL_CHUNK
 */
sl_status sl_aggregate_apply_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                         float* theta, int64_t n, void* stream);

/*
 * sl_apply_mean -- outer update with the aggregated sum.
 *
 * The pages do not describe the outer optimizer.  Reading: the pseudo-gradient
 * is pre-loop minus post-loop weights ([SF] "Why DiLoCo Alone Isn't Enough"),
 * so theta[i] <- theta[i] - out[i] / n_peers with a correctly rounded fp32
 * division (learning rate 1, no momentum); without compression this is the
 * mean of the peers' post-loop weights.
 *
 * theta    in/out float32[n], 16-byte aligned
 * out      in  float32[n], 16-byte aligned (the sl_aggregate result)
 * n_peers  1..SL_MAX_PEERS
 */
sl_status sl_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n,
                        void* stream);

/*
 * sl_aggregate_interleaved -- sl_aggregate with the peers' records laid out
 * chunk-major across peers.
 *
 * Same sums as sl_aggregate, bit for bit, for the same records ([SF] "Why
 * Extreme Sparsity Doesn't Break Convergence"; same reading).  Only the
 * layout differs: chunk c's record from peer p is at records + (c * n_peers +
 * p) * 112 and its scale at scales[c * n_peers + p], so every chunk's records
 * are one contiguous span.  When the records come from HBM rather than the
 * last-level cache, that span is served faster than n_peers separate record
 * streams.  A receiver that uploads peers' records from host memory can write
 * this layout directly: one 2-D copy per peer (hipMemcpy2DAsync, destination
 * records + p * 112 with pitch n_peers * 112, source pitch 112, width 112,
 * height n / 4096; scales likewise with 4-byte rows).
 *
 * records  in  DEVICE uint8[n/4096][n_peers][112], 16-byte aligned
 * scales   in  DEVICE float32[n/4096][n_peers], 4-byte aligned
 * n_peers  0..SL_MAX_PEERS (0 writes all +0.0 and reads neither input)
 * out      out float32[n], 16-byte aligned, fully overwritten; must not overlap
 *          records or scales
 * n        number of parameters, a multiple of SL_CHUNK
 * Payloads are trusted, as for sl_aggregate.  Records in this layout are
 * validated by sl_validate_payload over the buffers viewed as
 * n / 4096 * n_peers records: each record is checked on its own, so the flags
 * come back in the same chunk-major order.
 */
sl_status sl_aggregate_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                   float* out, int64_t n, void* stream);

/*
 * sl_aggregate_apply -- sl_aggregate followed by sl_apply_mean without the dense
 * update ever reaching HBM.
 *
 * The step after aggregation (the outer update; reading as for sl_apply_mean).
 * For every i: sum = the peer-ordered fp32 sum sl_aggregate would write to
 * out[i]; theta[i] <- theta[i] - sum / n_peers.  The results are bitwise those
 * of the two separate calls.  HBM traffic drops from 4 + 12 to 8 bytes per
 * parameter (plus the records).
 *
 * payloads, scales  as for sl_aggregate (host arrays of device pointers)
 * n_peers  1..SL_MAX_PEERS
 * theta    in/out float32[n], 16-byte aligned; must not overlap any record or
 *          scale buffer
 * n        number of parameters, a multiple of SL_CHUNK
 */
sl_status sl_aggregate_apply(const uint8_t* const* payloads, const float* const* scales,
                             int32_t n_peers, float* theta, int64_t n, void* stream);

/*
 * sl_validate_payload -- structural checks of received records (untrusted peers).
 *
 * [SF] "What the Blockchain Does (and Doesn't Do)": nothing on the chain checks
 * the updates; the authors' post on the arXiv:2603.08163 listing names integrity
 * checks among the validator's duties.  Reading of a well-formed record: its 64
 * indices are strictly increasing and its scale is finite and not negative.
 *
 * payload  in  uint8[n_chunks][112], 16-byte aligned
 * scales   in  float32[n_chunks], 4-byte aligned
 * n_chunks number of records (0 is a no-op)
 * flags    out uint8[n_chunks], must not overlap payload or scales; flags[c] is 0
 *          for a well-formed record, else bit 0 = indices not strictly
 *          increasing, bit 1 = scale not finite, bit 2 = scale negative.
 *          One byte per record rather than a single device counter of bad
 *          records: the caller learns which records failed and which check,
 *          and the count is the number of non-zero flags (sl_peer_stats
 *          returns it per peer in the same pass).
 */
sl_status sl_validate_payload(const uint8_t* payload, const float* scales, int64_t n_chunks,
                              uint8_t* flags, void* stream);

/*
 * sl_validate_payloads -- sl_validate_payload for n_peers peers in one launch,
 * so that a round's records are checked before they are aggregated.  Same
 * reading and checks as sl_validate_payload.
 *
 * payloads in  HOST array of n_peers DEVICE pointers, each uint8[n_chunks][112],
 *          16-byte aligned
 * scales   in  HOST array of n_peers DEVICE pointers, each float32[n_chunks],
 *          4-byte aligned
 * n_peers  0..SL_MAX_PEERS (0 is a no-op), else SL_ERR_TOO_MANY_PEERS
 * n_chunks records per peer (0 is a no-op)
 * flags    out uint8[n_peers][n_chunks] (peer-major), must not overlap any
 *          payload or scale buffer; flags[p * n_chunks + c] as for
 *          sl_validate_payload
 */
sl_status sl_validate_payloads(const uint8_t* const* payloads, const float* const* scales,
                               int32_t n_peers, int64_t n_chunks, uint8_t* flags, void* stream);

/*
 * sl_peer_stats -- per-peer statistics of a round's received records, with
 * the validation flags of sl_validate_payloads in the same pass.
 *
 * [SF] "What the Blockchain Does (and Doesn't Do)": the defence against
 * poisoned updates was that a crafted sparse update looks different to anomaly
 * detection.  Reading: the statistics such screening starts from, exact and
 * independent of the launch, for each peer p over its n_chunks records:
 *   counts[4p + 0]  records with any validation flag set
 *   counts[4p + 1]  records whose scale is +0 or -0 (empty chunks)
 *   counts[4p + 2]  entries at the magnitude level, code bit 0 (all records)
 *   counts[4p + 3]  entries with the sign bit, code bit 1 (all records)
 *   scale_max[p]    the largest scale among records whose scale is finite and
 *                   not negative (-0 counts as +0); +0 if there is none
 *
 * payloads, scales  as for sl_validate_payloads
 * n_peers   0..SL_MAX_PEERS (0 is a no-op), else SL_ERR_TOO_MANY_PEERS
 * n_chunks  records per peer; with 0 the statistics are all written as 0
 * flags     out uint8[n_peers][n_chunks] as for sl_validate_payloads, or NULL
 *           to skip them
 * counts    out int64[n_peers][4] (device, 8-byte aligned), overwritten
 * scale_max out float32[n_peers] (device, 4-byte aligned), overwritten
 * No output may overlap another output or any payload or scale buffer.
 *
 * One kernel launch that takes the peers' records peer after peer, each in
 * memory order.  Its workgroups add their per-peer sums and maxima to eight
 * copies of the totals with device-scope integer atomics (the totals do not
 * depend on the order), and the last one to finish writes counts and
 * scale_max and zeroes the copies.  The copies live in a 37,120-byte part of a
 * device buffer that the library allocates and zeroes on the first call of
 * sl_peer_stats or sl_peer_stats_interleaved on each device and keeps until
 * the process ends (74,240 bytes in all).  That first call must not be made
 * while its stream is being captured into a graph (SL_ERR_HIP); later calls
 * allocate nothing.  All sl_peer_stats calls on one device share that part, so
 * calls that overlap in time (streams with no ordering between them) race.
 */
sl_status sl_peer_stats(const uint8_t* const* payloads, const float* const* scales, int32_t n_peers,
                        int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                        void* stream);

/*
 * sl_peer_stats_interleaved -- sl_peer_stats for records laid out chunk-major
 * across peers (the layout of sl_aggregate_interleaved).
 *
 * The same statistics ([SF] "What the Blockchain Does (and Doesn't Do)"; same
 * reading) and the same flags as sl_peer_stats, for records where chunk
 * c's record from peer p is at records + (c * n_peers + p) * 112 and its scale
 * at scales[c * n_peers + p].  flags, counts and scale_max are laid out per
 * peer, exactly as sl_peer_stats writes them.
 *
 * records    in  DEVICE uint8[n_chunks][n_peers][112], 16-byte aligned
 * scales     in  DEVICE float32[n_chunks][n_peers], 4-byte aligned
 * n_peers        0..SL_MAX_PEERS (0 does nothing)
 * n_chunks       records per peer, 0..2^31-1
 * flags      out DEVICE uint8[n_peers][n_chunks] or NULL
 * counts     out DEVICE int64[n_peers][4], 8-byte aligned
 * scale_max  out DEVICE float32[n_peers], 4-byte aligned
 * No output may overlap an input or another output.  Errors as for
 * sl_peer_stats.
 *
 * One kernel launch that reads the records in memory order, 256 lanes over
 * whole chunks, so each lane meets one peer; the totals are formed as in
 * sl_peer_stats, in the 37,120-byte second part of its device buffer
 * (allocated as described there), so calls of sl_peer_stats_interleaved on
 * one device must not overlap in time; they may overlap sl_peer_stats calls.
 */
sl_status sl_peer_stats_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                    int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                                    void* stream);

/*
 * sl_peer_stats_noalloc -- sl_peer_stats for callers that cannot allocate
 * device memory: code under graph capture (including a first call), tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, checks,
 * results and single kernel launch as sl_peer_stats; it calls no hipMalloc,
 * hipFree or other allocating routine.
 *
 * Its scratch is a static device array of 37,120 bytes on every GPU the library
 * runs on, held until the process ends.  Every valid call fits in it
 * (n_peers <= SL_MAX_PEERS, any n_chunks), so no size is refused beyond the
 * checks above.  All calls on one GPU share that GPU's array: calls that
 * overlap in time there (streams with no ordering between them, or with a
 * concurrent sl_peer_stats_noalloc from another thread) race.  Its totals and
 * arrival counter are zero when the library is loaded and every completed call
 * leaves them at zero.  It does not share scratch with sl_peer_stats.
 * Returns SL_ERR_HIP if the array's device address cannot be found.
 */
sl_status sl_peer_stats_noalloc(const uint8_t* const* payloads, const float* const* scales,
                                int32_t n_peers, int64_t n_chunks, uint8_t* flags, int64_t* counts,
                                float* scale_max, void* stream);

/*
 * sl_host_device_pointer -- device address of pinned, mapped host memory.
 *
 * Error-feedback offload ([CV] "SparseLoCo: Breaking the Bandwidth Barrier":
 * the error-feedback buffers are moved off the GPU while they are not needed):
 * an ef buffer in pinned host memory can be passed to sl_compress /
 * sl_compress_weights through the address returned here; the kernel then reads
 * and writes it over the host link while delta and the records stay in HBM.
 *
 * host_ptr    in  an address inside a pinned host allocation (hipHostMalloc)
 * device_ptr  out the address the GPU uses for it (NULL on error)
 * Returns SL_ERR_INVALID_ARG if host_ptr is not pinned and mapped; no kernel
 * should be given such an address.
 */
sl_status sl_host_device_pointer(const void* host_ptr, void** device_ptr);

/* Human-readable name of a status code (static storage, never NULL).  Takes an
 * int rather than sl_status so that any stored value, including one outside
 * the enumeration, is well defined to pass; unknown values give
 * "unknown sl_status". */
const char* sl_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSELOCO_H */
