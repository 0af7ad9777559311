/*
 * oracle.h -- plain, slow, obviously-correct CPU model of the SparseLoCo
 * pseudo-gradient compressor and its aggregator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke entry point and the
 * benchmark's CPU-baseline leg may load this library.  The product (the HIP
 * library under communication_efficient_distributed_amd/) never calls it and
 * shares no code, header, table or helper with it.
 *
 * Sources (cited by page title and section):
 *  [SF]  "The Sparse Frontier: SparseLoCo and the Compression Math Behind
 *         Permissionless Pre-Training" (blokz.dev)
 *        - "SparseLoCo: Three Compression Levers in One Pass": chunks of 4,096
 *          parameters, top-64 by absolute magnitude, four 2-bit levels with a
 *          per-chunk scale, 12-bit in-chunk indices, 64 x 14 bits = 112 bytes
 *          per chunk, 146.3x versus fp32.
 *        - "Why Extreme Sparsity Doesn't Break Convergence", error-feedback
 *          paragraph: what is not sent rolls into the next round.
 *        - same section, sparse-aggregation paragraph: receivers sum the
 *          union of the peers' selected coordinates.
 *  [CV]  "Covenant-72B: Decentralized Training is No Longer Just a Dream"
 *        (wispaper.ai), "SparseLoCo: Breaking the Bandwidth Barrier".
 *
 * Where the pages leave a step open this model takes one plain reading; each is
 * marked "reading:" in oracle.cpp.  Parity status of every function is listed
 * in the header comment of oracle.cpp.
 *
 * All pointers are host pointers owned by the caller.  Functions return 0 on
 * success and a negative value on an argument error.
 */
#ifndef SPARSELOCO_ORACLE_H
#define SPARSELOCO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Generic chunked compressor for any chunk size and k (tiny chunks are used by
 * the exhaustive tests).  n must be a multiple of chunk, 1 <= k <= chunk.
 * On return, for chunk c:
 *   idx[c*k + j]  j-th kept in-chunk index, ascending in j
 *   code[c*k + j] its 2-bit code (bit 0 = magnitude, bit 1 = sign)
 *   scale[c]      the chunk scale
 * and ef[] holds the new error-feedback residual (updated in place). */
int orc_compress_unpacked(const float* delta, float* ef, int64_t n, int32_t chunk,
                          int32_t k, float beta, int32_t* idx, uint8_t* code,
                          float* scale);

/* 4096/64 payload packing: 96 bytes of 12-bit indices then 16 bytes of 2-bit
 * codes, both little-endian LSB-first bit streams (112 bytes per chunk). */
void orc_pack(const int32_t* idx, const uint8_t* code, int64_t n_chunks,
              uint8_t* payload);
void orc_unpack(const uint8_t* payload, int64_t n_chunks, int32_t* idx,
                uint8_t* code);

/* Full compressor at chunk 4096, k 64: payload[n/4096][112], scales[n/4096].
 * nthreads <= 1 runs on the calling thread; more threads split the chunks. */
int orc_compress(const float* delta, float* ef, int64_t n, float beta,
                 uint8_t* payload, float* scales, int32_t nthreads);

/* Sum of n_peers decoded payloads into out[n] (overwritten), peer order
 * 0..n_peers-1 per coordinate, starting from +0.0.  n_peers may be 0. */
int orc_aggregate(const uint8_t* const* payloads, const float* const* scales,
                  int32_t n_peers, int64_t n, float* out, int32_t nthreads);

/* theta[i] <- theta[i] - out[i] / n_peers   (n_peers >= 1). */
int orc_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n);

/* Well-formedness of received payloads: indices strictly increasing, scale
 * finite and >= 0.  bad[c] = 0 for a well-formed chunk, else bit 0 = indices
 * not strictly increasing, bit 1 = scale not finite, bit 2 = scale negative.
 * Returns the number of bad chunks. */
int64_t orc_validate(const uint8_t* payload, const float* scales, int64_t n_chunks,
                     uint8_t* bad);

/* Statistics of one peer's n_chunks received records (reading R13):
 * counts[0] records that orc_validate flags, counts[1] records whose scale is
 * +0 or -0, counts[2] entries with code bit 0 (magnitude level), counts[3]
 * entries with code bit 1 (sign); *scale_max = the largest scale among records
 * whose scale is finite and not negative, +0 if there is none. */
void orc_peer_stats(const uint8_t* payload, const float* scales, int64_t n_chunks,
                    int64_t* counts, float* scale_max);

/* Pseudo-gradient: delta[i] = theta_pre[i] - theta_post[i]. */
void orc_pseudo_gradient(const float* theta_pre, const float* theta_post, int64_t n,
                         float* delta);

/* Decoded value of one 2-bit code at chunk scale s. */
float orc_decode(uint8_t code, float s);

#ifdef __cplusplus
}
#endif

#endif /* SPARSELOCO_ORACLE_H */
