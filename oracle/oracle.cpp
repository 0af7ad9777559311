/*
 * oracle.cpp -- CPU model of the SparseLoCo compressor and aggregator.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by tests, the smoke entry point
 * and the benchmark's CPU-baseline leg, never by the product.
 *
 * Built with plain g++ -O2 -ffp-contract=off (no fast-math, no SIMD intrinsics),
 * so every floating-point operation below is the single IEEE-754 binary32 or
 * binary64 operation it is written as, rounded to nearest-even, with denormals
 * kept.
 *
 * Step order follows the pages ([SF] = "The Sparse Frontier: SparseLoCo and the
 * Compression Math Behind Permissionless Pre-Training"):
 *   1. error feedback: acc = beta*ef + delta        [SF, "Why Extreme Sparsity
 *                                                    Doesn't Break Convergence",
 *                                                    error-feedback paragraph]
 *   2. non-overlapping chunks of 4,096 parameters    [SF, "Three Compression
 *   3. keep the top 64 by absolute magnitude           Levers", lever 1]
 *   4. per-chunk scale, four 2-bit levels             [SF, lever 2]
 *   5. 12-bit in-chunk index                          [SF, lever 3]
 *   6. 64 x (2 + 12) bits = 112 bytes per chunk       [SF, the per-chunk layout
 *                                                    formula after lever 3]
 *   7. residual back into ef                          [SF, error-feedback paragraph]
 *   8. receivers sum the union of peers' entries      [SF, sparse-aggregation
 *                                                    paragraph]
 *
 * Readings (the pages leave these open; each is stated where it is used):
 *   R1 beta is a parameter; beta = 1 is the pages' plain accumulation.
 *   R2 beta*ef + delta is one fused multiply-add (single rounding).
 *   R3 ranking is on acc (after the EF update), by |acc| via the 31-bit key
 *      bits(acc) & 0x7fffffff; ties at the cut go to the lower index.
 *   R4 the 64 kept entries are listed in ascending index order.
 *   R5 s = max |kept| (= max |acc| of the chunk); levels {-s, -s/3, +s/3, +s};
 *      magnitude bit set iff 3|v| > 2s exactly; s/3 correctly rounded in fp32.
 *   R6 code bit 0 = magnitude, bit 1 = IEEE sign bit of acc (-0 is negative).
 *   R7 payload = 96 bytes of 12-bit indices then 16 bytes of 2-bit codes, both
 *      LSB-first little-endian bit streams; the fp32 scale is stored apart.
 *   R8 ef <- acc - decoded at kept positions, acc elsewhere.
 *   R9 aggregation returns the sum, from +0.0, peers in ascending order.
 *   R10 outer update theta <- theta - sum / N (correctly rounded division).
 *   R11 pseudo-gradient delta = theta_pre - theta_post, one fp32 subtraction
 *       ([SF], "Why DiLoCo Alone Isn't Enough": the difference of the weights
 *       before and after the inner loop; the sign is the reading).
 *   R12 a well-formed record has strictly increasing indices and a finite,
 *       non-negative scale (-0 accepted).
 *   R13 per-peer statistics for anomaly screening ([SF], "What the Blockchain
 *       Does (and Doesn't Do)": a crafted sparse update stands out to anomaly
 *       detection): records flagged by the validator, records with a zero
 *       scale, entries at the magnitude level, entries with the sign bit, and
 *       the largest finite non-negative scale (-0 counts as +0).
 *
 * Parity status:
 *   orc_compress_unpacked  pinned (brute force over all inputs of tiny chunks,
 *                          exact-rational threshold checks, closed-form golden
 *                          chunks, symmetry and scaling invariants)
 *   orc_pack / orc_unpack  pinned (closed-form golden bytes, bitwise reader in
 *                          the tests); the layout itself is reading R7
 *   orc_compress           pinned (= unpacked + pack; page figures 112 B, 146.3x)
 *   orc_aggregate          pinned (N = 1 equals bitwise decode, exact dyadic
 *                          sums, scale doubling, support within the union);
 *                          the peer summation order is reading R9
 *   orc_apply_mean         pinned (closed form on exact inputs)
 *   orc_validate           pinned (hand-made malformed payloads, one per flag)
 *   orc_peer_stats         pinned (counts of constructed records, bitwise
 *                          reader of the code bytes, max over a numpy mask)
 *   orc_pseudo_gradient    pinned (exact small-integer weights)
 *   orc_decode             pinned (s/3 against exact-rational rounding)
 */
#include "oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

namespace {

const int32_t kChunk = 4096;     /* [SF, lever 1] */
const int32_t kTopK = 64;        /* [SF, lever 1] */
const int32_t kIndexBits = 12;   /* [SF, lever 3]: ceil(log2 4096) */
const int32_t kCodeBits = 2;     /* [SF, lever 2]: four levels */
const int32_t kIndexBytes = kTopK * kIndexBits / 8;          /* 96 */
const int32_t kPayloadBytes = kTopK * (kIndexBits + kCodeBits) / 8; /* 112 */

uint32_t bits_of(float v) {
    uint32_t b;
    std::memcpy(&b, &v, sizeof b);
    return b;
}

/* R3: the magnitude order used for ranking. */
uint32_t magnitude_key(float v) { return bits_of(v) & 0x7fffffffu; }

/* R6: IEEE sign bit. */
uint32_t sign_bit(float v) { return bits_of(v) >> 31; }

/* R5: one-third level, correctly rounded fp32 division. */
float third_of(float s) { return s / 3.0f; }

/* R5/R6: decoded value of a 2-bit code. */
float decode_value(uint8_t code, float s) {
    float mag = (code & 1u) ? s : third_of(s);
    return (code & 2u) ? -mag : mag;
}

/* One chunk: steps 1-5 and 7.  acc lives in a local copy. */
void compress_one_chunk(const float* delta, float* ef, int32_t chunk, int32_t k,
                        float beta, int32_t* out_idx, uint8_t* out_code,
                        float* out_scale) {
    std::vector<float> acc(chunk);
    for (int32_t i = 0; i < chunk; ++i) {
        acc[i] = std::fma(beta, ef[i], delta[i]);          /* R1, R2 */
    }

    /* Step 3: full sort of the chunk by (|acc| descending, index ascending);
     * the first k are kept (R3 tie rule). */
    std::vector<int32_t> order(chunk);
    for (int32_t i = 0; i < chunk; ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        uint32_t ka = magnitude_key(acc[a]);
        uint32_t kb = magnitude_key(acc[b]);
        if (ka != kb) return ka > kb;
        return a < b;
    });
    std::vector<int32_t> kept(order.begin(), order.begin() + k);
    std::sort(kept.begin(), kept.end());                   /* R4 */

    /* Step 4: scale and levels. */
    float s = std::fabs(acc[order[0]]);                    /* R5 */
    double two_s = 2.0 * (double)s;                        /* exact in binary64 */
    for (int32_t j = 0; j < k; ++j) {
        int32_t i = kept[j];
        float v = acc[i];
        uint32_t sign = sign_bit(v);
        /* 3|v| needs 26 significant bits: exact in binary64, so this is the
         * exact-real comparison 3|v| > 2s. */
        uint32_t mag = (3.0 * (double)std::fabs(v) > two_s) ? 1u : 0u;
        uint8_t code = (uint8_t)((sign << 1) | mag);
        out_idx[j] = i;
        out_code[j] = code;
        acc[i] = acc[i] - decode_value(code, s);           /* R8 */
    }
    *out_scale = s;
    for (int32_t i = 0; i < chunk; ++i) ef[i] = acc[i];    /* step 7 */
}

/* Step 6, R7: write value v of width w at bit position pos of a little-endian,
 * LSB-first byte stream. */
void put_bits(uint8_t* stream, int32_t pos, uint32_t v, int32_t w) {
    for (int32_t b = 0; b < w; ++b) {
        int32_t p = pos + b;
        if ((v >> b) & 1u) stream[p / 8] |= (uint8_t)(1u << (p % 8));
    }
}

uint32_t get_bits(const uint8_t* stream, int32_t pos, int32_t w) {
    uint32_t v = 0;
    for (int32_t b = 0; b < w; ++b) {
        int32_t p = pos + b;
        if ((stream[p / 8] >> (p % 8)) & 1u) v |= 1u << b;
    }
    return v;
}

void pack_one(const int32_t* idx, const uint8_t* code, uint8_t* out) {
    std::memset(out, 0, kPayloadBytes);
    for (int32_t j = 0; j < kTopK; ++j) {
        put_bits(out, j * kIndexBits, (uint32_t)idx[j], kIndexBits);
        put_bits(out + kIndexBytes, j * kCodeBits, code[j], kCodeBits);
    }
}

void unpack_one(const uint8_t* in, int32_t* idx, uint8_t* code) {
    for (int32_t j = 0; j < kTopK; ++j) {
        idx[j] = (int32_t)get_bits(in, j * kIndexBits, kIndexBits);
        code[j] = (uint8_t)get_bits(in + kIndexBytes, j * kCodeBits, kCodeBits);
    }
}

/* Run f(first_chunk, last_chunk) over [0, n_chunks) on nthreads threads. */
template <class F>
void for_chunks(int64_t n_chunks, int32_t nthreads, F f) {
    if (nthreads <= 1 || n_chunks < 2) {
        f((int64_t)0, n_chunks);
        return;
    }
    int64_t t = std::min<int64_t>(nthreads, n_chunks);
    std::vector<std::thread> pool;
    for (int64_t w = 0; w < t; ++w) {
        int64_t a = n_chunks * w / t;
        int64_t b = n_chunks * (w + 1) / t;
        pool.emplace_back([=] { f(a, b); });
    }
    for (auto& th : pool) th.join();
}

}  // namespace

extern "C" {

int orc_compress_unpacked(const float* delta, float* ef, int64_t n, int32_t chunk,
                          int32_t k, float beta, int32_t* idx, uint8_t* code,
                          float* scale) {
    if (chunk <= 0 || k <= 0 || k > chunk || n < 0 || n % chunk != 0) return -1;
    if (n > 0 && (!delta || !ef || !idx || !code || !scale)) return -1;
    int64_t n_chunks = n / chunk;
    for (int64_t c = 0; c < n_chunks; ++c) {
        compress_one_chunk(delta + c * chunk, ef + c * chunk, chunk, k, beta,
                           idx + c * k, code + c * k, scale + c);
    }
    return 0;
}

void orc_pack(const int32_t* idx, const uint8_t* code, int64_t n_chunks,
              uint8_t* payload) {
    for (int64_t c = 0; c < n_chunks; ++c) {
        pack_one(idx + c * kTopK, code + c * kTopK, payload + c * kPayloadBytes);
    }
}

void orc_unpack(const uint8_t* payload, int64_t n_chunks, int32_t* idx,
                uint8_t* code) {
    for (int64_t c = 0; c < n_chunks; ++c) {
        unpack_one(payload + c * kPayloadBytes, idx + c * kTopK, code + c * kTopK);
    }
}

int orc_compress(const float* delta, float* ef, int64_t n, float beta,
                 uint8_t* payload, float* scales, int32_t nthreads) {
    if (n < 0 || n % kChunk != 0) return -1;
    if (n > 0 && (!delta || !ef || !payload || !scales)) return -1;
    int64_t n_chunks = n / kChunk;
    for_chunks(n_chunks, nthreads, [&](int64_t a, int64_t b) {
        int32_t idx[kTopK];
        uint8_t code[kTopK];
        for (int64_t c = a; c < b; ++c) {
            compress_one_chunk(delta + c * kChunk, ef + c * kChunk, kChunk, kTopK,
                               beta, idx, code, scales + c);
            pack_one(idx, code, payload + c * kPayloadBytes);
        }
    });
    return 0;
}

int orc_aggregate(const uint8_t* const* payloads, const float* const* scales,
                  int32_t n_peers, int64_t n, float* out, int32_t nthreads) {
    if (n < 0 || n % kChunk != 0 || n_peers < 0) return -1;
    if (n > 0 && !out) return -1;
    if (n_peers > 0 && (!payloads || !scales)) return -1;
    int64_t n_chunks = n / kChunk;
    for_chunks(n_chunks, nthreads, [&](int64_t a, int64_t b) {
        int32_t idx[kTopK];
        uint8_t code[kTopK];
        for (int64_t c = a; c < b; ++c) {
            float* o = out + c * kChunk;
            for (int32_t i = 0; i < kChunk; ++i) o[i] = +0.0f;       /* R9 */
            for (int32_t p = 0; p < n_peers; ++p) {                  /* R9 order */
                unpack_one(payloads[p] + c * kPayloadBytes, idx, code);
                float s = scales[p][c];
                for (int32_t j = 0; j < kTopK; ++j) {
                    o[idx[j]] = o[idx[j]] + decode_value(code[j], s);
                }
            }
        }
    });
    return 0;
}

int orc_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n) {
    if (n_peers < 1 || n < 0) return -1;
    if (n > 0 && (!theta || !out)) return -1;
    float denom = (float)n_peers;
    for (int64_t i = 0; i < n; ++i) theta[i] = theta[i] - out[i] / denom;  /* R10 */
    return 0;
}

int64_t orc_validate(const uint8_t* payload, const float* scales, int64_t n_chunks,
                     uint8_t* bad) {
    /* R12, a well-formed record: strictly increasing indices, finite and
     * non-negative scale.  bad[c]: bit 0 order, bit 1 non-finite, bit 2 negative. */
    int64_t n_bad = 0;
    int32_t idx[kTopK];
    uint8_t code[kTopK];
    for (int64_t c = 0; c < n_chunks; ++c) {
        unpack_one(payload + c * kPayloadBytes, idx, code);
        uint8_t f = 0;
        for (int32_t j = 1; j < kTopK; ++j)
            if (!(idx[j] > idx[j - 1])) f |= 1;
        if (!std::isfinite(scales[c])) f |= 2;
        if (scales[c] < 0.0f) f |= 4;
        if (bad) bad[c] = f;
        if (f) ++n_bad;
    }
    return n_bad;
}

void orc_peer_stats(const uint8_t* payload, const float* scales, int64_t n_chunks,
                    int64_t* counts, float* scale_max) {
    /* R13.  Flags as in orc_validate; the code counts take every record as
     * received, well-formed or not. */
    int64_t bad = 0, zero_scale = 0, magnitude = 0, negative = 0;
    float top = 0.0f;
    int32_t idx[kTopK];
    uint8_t code[kTopK];
    for (int64_t c = 0; c < n_chunks; ++c) {
        uint8_t f = 0;
        orc_validate(payload + c * kPayloadBytes, scales + c, 1, &f);
        if (f) ++bad;
        const float s = scales[c];
        if (s == 0.0f) ++zero_scale;
        if ((f & 6u) == 0 && s > top) top = s;
        unpack_one(payload + c * kPayloadBytes, idx, code);
        for (int32_t j = 0; j < kTopK; ++j) {
            if (code[j] & 1u) ++magnitude;
            if (code[j] & 2u) ++negative;
        }
    }
    counts[0] = bad;
    counts[1] = zero_scale;
    counts[2] = magnitude;
    counts[3] = negative;
    *scale_max = top;
}

void orc_pseudo_gradient(const float* theta_pre, const float* theta_post, int64_t n,
                         float* delta) {
    /* [SF] "Why DiLoCo Alone Isn't Enough" (pseudo-gradient from the weights on
     * either side of the inner loop); R11 fixes the sign: pre - post. */
    for (int64_t i = 0; i < n; ++i) delta[i] = theta_pre[i] - theta_post[i];
}

float orc_decode(uint8_t code, float s) { return decode_value(code, s); }

}  // extern "C"
