// sparseloco.cpp -- the C ABI of libsparseloco.so (declared in
// include/sparseloco.h): host-side argument checks and kernel launches.  No
// synchronisation; the one allocation is sl_peer_stats's scratch (below).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <map>
#include <mutex>

#include "internal.h"
#include "sparseloco.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a);
    const uintptr_t y = reinterpret_cast<uintptr_t>(b);
    return na && nb && x < y + nb && y < x + na;
}

sl_status from_hip(hipError_t e) { return e == hipSuccess ? SL_OK : SL_ERR_HIP; }

// Argument checks of sl_peer_stats and sl_peer_stats_noalloc; fills the
// pointer table.  *noop is set when there is nothing to do (n_peers == 0).
sl_status peer_stats_args(const uint8_t* const* payloads, const float* const* scales, int32_t n_peers,
                          int64_t n_chunks, const uint8_t* flags, const int64_t* counts, const float* scale_max,
                          sl::PeerTable* table, bool* noop) {
    *noop = false;
    if (n_chunks < 0 || n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    if (n_peers < 0 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n_peers == 0) {
        *noop = true;
        return SL_OK;
    }
    if (!counts || !scale_max) return SL_ERR_INVALID_ARG;
    if (!aligned(counts, 8) || !aligned(scale_max, 4)) return SL_ERR_ALIGN;
    const size_t cbytes = (size_t)n_peers * 4 * sizeof(int64_t);
    const size_t mbytes = (size_t)n_peers * sizeof(float);
    const size_t fbytes = flags ? (size_t)n_peers * (size_t)n_chunks : 0;
    if (overlap(counts, cbytes, scale_max, mbytes) || overlap(flags, fbytes, counts, cbytes) ||
        overlap(flags, fbytes, scale_max, mbytes))
        return SL_ERR_INVALID_ARG;
    if (n_chunks > 0) {
        if (!payloads || !scales) return SL_ERR_INVALID_ARG;
        const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
        const size_t sbytes = (size_t)n_chunks * sizeof(float);
        for (int32_t p = 0; p < n_peers; ++p) {
            if (!payloads[p] || !scales[p]) return SL_ERR_INVALID_ARG;
            if (!aligned(payloads[p], 16) || !aligned(scales[p], 4)) return SL_ERR_ALIGN;
            const void* bufs[3] = {flags, counts, scale_max};
            const size_t lens[3] = {fbytes, cbytes, mbytes};
            for (int b = 0; b < 3; ++b)
                if (overlap(bufs[b], lens[b], payloads[p], pbytes) || overlap(bufs[b], lens[b], scales[p], sbytes))
                    return SL_ERR_INVALID_ARG;
            table->payload[p] = payloads[p];
            table->scales[p] = scales[p];
        }
    }
    return SL_OK;
}

// sl_peer_stats's scratch: one buffer per device, allocated and zeroed by the
// first call on the device and kept until the process ends.  That first call
// must not be made while its stream is being captured into a graph (it gets
// SL_ERR_HIP then); later calls allocate nothing and can be captured.
sl_status stats_scratch(void* stream, void** out) {
    static std::mutex mu;
    static std::map<int, void*> buffers;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SL_ERR_HIP;
    std::lock_guard<std::mutex> lock(mu);
    const auto it = buffers.find(dev);
    if (it != buffers.end()) {
        *out = it->second;
        return SL_OK;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return SL_ERR_HIP;
    void* p = nullptr;
    // sl_peer_stats's part, then sl_peer_stats_interleaved's.
    const size_t bytes = sl::peer_stats_scratch_bytes() + sl::interleaved_stats_scratch_bytes();
    if (hipMalloc(&p, bytes) != hipSuccess) return SL_ERR_HIP;
    // Zeroed before the first statistics kernel, which runs later on the same
    // stream.
    if (hipMemsetAsync(p, 0, bytes, s) != hipSuccess) {
        (void)hipFree(p);
        return SL_ERR_HIP;
    }
    buffers[dev] = p;
    *out = p;
    return SL_OK;
}

}  // namespace

extern "C" {

sl_status sl_compress(const float* delta, float* ef, float beta, uint8_t* payload,
                      float* scales, int64_t n, void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n == 0) return SL_OK;
    if (!delta || !ef || !payload || !scales) return SL_ERR_INVALID_ARG;
    if (!std::isfinite(beta)) return SL_ERR_INVALID_ARG;
    if (!aligned(delta, 16) || !aligned(ef, 16) || !aligned(payload, 16) || !aligned(scales, 4))
        return SL_ERR_ALIGN;
    const int64_t n_chunks = n / SL_CHUNK;
    if (n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    const size_t dense = (size_t)n * sizeof(float);
    const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * sizeof(float);
    if ((const void*)delta != (const void*)ef && overlap(delta, dense, ef, dense))
        return SL_ERR_INVALID_ARG;
    if (overlap(payload, pbytes, delta, dense) || overlap(payload, pbytes, ef, dense) ||
        overlap(scales, sbytes, delta, dense) || overlap(scales, sbytes, ef, dense) ||
        overlap(payload, pbytes, scales, sbytes))
        return SL_ERR_INVALID_ARG;
    return from_hip(sl::launch_compress(delta, ef, beta, payload, scales, n_chunks,
                                        static_cast<hipStream_t>(stream)));
}

sl_status sl_compress_weights(const float* theta_pre, const float* theta_post, float* ef,
                              float beta, uint8_t* payload, float* scales, int64_t n,
                              void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n == 0) return SL_OK;
    if (!theta_pre || !theta_post || !ef || !payload || !scales) return SL_ERR_INVALID_ARG;
    if (!std::isfinite(beta)) return SL_ERR_INVALID_ARG;
    if (!aligned(theta_pre, 16) || !aligned(theta_post, 16) || !aligned(ef, 16) ||
        !aligned(payload, 16) || !aligned(scales, 4))
        return SL_ERR_ALIGN;
    const int64_t n_chunks = n / SL_CHUNK;
    if (n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    const size_t dense = (size_t)n * sizeof(float);
    const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * sizeof(float);
    // theta_pre and theta_post are read only and may alias each other; every
    // written buffer must be disjoint from every other buffer.
    const void* in[2] = {theta_pre, theta_post};
    for (const void* p : in)
        if (overlap(ef, dense, p, dense) || overlap(payload, pbytes, p, dense) ||
            overlap(scales, sbytes, p, dense))
            return SL_ERR_INVALID_ARG;
    if (overlap(payload, pbytes, ef, dense) || overlap(scales, sbytes, ef, dense) ||
        overlap(payload, pbytes, scales, sbytes))
        return SL_ERR_INVALID_ARG;
    return from_hip(sl::launch_compress_weights(theta_pre, theta_post, ef, beta, payload, scales,
                                                n_chunks, static_cast<hipStream_t>(stream)));
}

sl_status sl_validate_payload(const uint8_t* payload, const float* scales, int64_t n_chunks,
                              uint8_t* flags, void* stream) {
    if (n_chunks < 0 || n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    if (n_chunks == 0) return SL_OK;
    if (!payload || !scales || !flags) return SL_ERR_INVALID_ARG;
    if (!aligned(payload, 16) || !aligned(scales, 4)) return SL_ERR_ALIGN;
    const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * sizeof(float);
    if (overlap(flags, (size_t)n_chunks, payload, pbytes) ||
        overlap(flags, (size_t)n_chunks, scales, sbytes))
        return SL_ERR_INVALID_ARG;
    sl::PeerTable table = {};
    table.payload[0] = payload;
    table.scales[0] = scales;
    return from_hip(sl::launch_validate(table, 1, n_chunks, flags, static_cast<hipStream_t>(stream)));
}

sl_status sl_validate_payloads(const uint8_t* const* payloads, const float* const* scales,
                               int32_t n_peers, int64_t n_chunks, uint8_t* flags, void* stream) {
    if (n_chunks < 0 || n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    if (n_peers < 0 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n_chunks == 0 || n_peers == 0) return SL_OK;
    if (!payloads || !scales || !flags) return SL_ERR_INVALID_ARG;
    const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * sizeof(float);
    const size_t fbytes = (size_t)n_peers * (size_t)n_chunks;
    sl::PeerTable table = {};
    for (int32_t p = 0; p < n_peers; ++p) {
        if (!payloads[p] || !scales[p]) return SL_ERR_INVALID_ARG;
        if (!aligned(payloads[p], 16) || !aligned(scales[p], 4)) return SL_ERR_ALIGN;
        if (overlap(flags, fbytes, payloads[p], pbytes) || overlap(flags, fbytes, scales[p], sbytes))
            return SL_ERR_INVALID_ARG;
        table.payload[p] = payloads[p];
        table.scales[p] = scales[p];
    }
    return from_hip(sl::launch_validate(table, n_peers, n_chunks, flags, static_cast<hipStream_t>(stream)));
}

sl_status sl_peer_stats(const uint8_t* const* payloads, const float* const* scales, int32_t n_peers,
                        int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max, void* stream) {
    sl::PeerTable table = {};
    bool noop = false;
    const sl_status st = peer_stats_args(payloads, scales, n_peers, n_chunks, flags, counts, scale_max, &table, &noop);
    if (st != SL_OK || noop) return st;
    void* scratch = nullptr;
    const sl_status ss = stats_scratch(stream, &scratch);
    if (ss != SL_OK) return ss;
    return from_hip(sl::launch_peer_stats(table, n_peers, n_chunks, flags, counts, scale_max, scratch,
                                          static_cast<hipStream_t>(stream)));
}

sl_status sl_peer_stats_interleaved(const uint8_t* records, const float* scales, int32_t n_peers, int64_t n_chunks,
                                   uint8_t* flags, int64_t* counts, float* scale_max, void* stream) {
    if (n_chunks < 0 || n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    if (n_peers < 0 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n_peers == 0) return SL_OK;
    if (!counts || !scale_max) return SL_ERR_INVALID_ARG;
    if (!aligned(counts, 8) || !aligned(scale_max, 4)) return SL_ERR_ALIGN;
    const size_t cbytes = (size_t)n_peers * 4 * sizeof(int64_t);
    const size_t mbytes = (size_t)n_peers * sizeof(float);
    const size_t fbytes = flags ? (size_t)n_peers * (size_t)n_chunks : 0;
    if (overlap(counts, cbytes, scale_max, mbytes) || overlap(flags, fbytes, counts, cbytes) ||
        overlap(flags, fbytes, scale_max, mbytes))
        return SL_ERR_INVALID_ARG;
    if (n_chunks > 0) {
        if (!records || !scales) return SL_ERR_INVALID_ARG;
        if (!aligned(records, 16) || !aligned(scales, 4)) return SL_ERR_ALIGN;
        const size_t rbytes = (size_t)n_chunks * (size_t)n_peers * SL_PAYLOAD_BYTES;
        const size_t sbytes = (size_t)n_chunks * (size_t)n_peers * sizeof(float);
        const void* bufs[3] = {flags, counts, scale_max};
        const size_t lens[3] = {fbytes, cbytes, mbytes};
        for (int b = 0; b < 3; ++b)
            if (overlap(bufs[b], lens[b], records, rbytes) || overlap(bufs[b], lens[b], scales, sbytes))
                return SL_ERR_INVALID_ARG;
    }
    void* scratch = nullptr;
    const sl_status ss = stats_scratch(stream, &scratch);
    if (ss != SL_OK) return ss;
    return from_hip(sl::launch_peer_stats_interleaved(records, scales, n_peers, n_chunks, flags, counts, scale_max,
                                                      static_cast<uint8_t*>(scratch) + sl::peer_stats_scratch_bytes(),
                                                      static_cast<hipStream_t>(stream)));
}

sl_status sl_peer_stats_noalloc(const uint8_t* const* payloads, const float* const* scales, int32_t n_peers,
                                int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                                void* stream) {
    sl::PeerTable table = {};
    bool noop = false;
    const sl_status st = peer_stats_args(payloads, scales, n_peers, n_chunks, flags, counts, scale_max, &table, &noop);
    if (st != SL_OK || noop) return st;
    void* scratch = nullptr;  // the library's static copy on the current device
    if (sl::peer_stats_static_scratch(&scratch) != hipSuccess) return SL_ERR_HIP;
    return from_hip(sl::launch_peer_stats(table, n_peers, n_chunks, flags, counts, scale_max, scratch,
                                          static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Validates the peer tables and fills the kernel's pointer table; `dst` (out or
// theta, float32[n]) must not overlap any record or scale buffer.
sl_status peer_table(const uint8_t* const* payloads, const float* const* scales, int32_t n_peers,
                     const float* dst, int64_t n, sl::PeerTable* table) {
    const int64_t n_chunks = n / SL_CHUNK;
    const size_t dense = (size_t)n * sizeof(float);
    const size_t pbytes = (size_t)n_chunks * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * sizeof(float);
    *table = {};
    if (n_peers > 0 && (!payloads || !scales)) return SL_ERR_INVALID_ARG;
    for (int32_t p = 0; p < n_peers; ++p) {
        if (!payloads[p] || !scales[p]) return SL_ERR_INVALID_ARG;
        if (!aligned(payloads[p], 16) || !aligned(scales[p], 4)) return SL_ERR_ALIGN;
        if (overlap(dst, dense, payloads[p], pbytes) || overlap(dst, dense, scales[p], sbytes))
            return SL_ERR_INVALID_ARG;
        table->payload[p] = payloads[p];
        table->scales[p] = scales[p];
    }
    return SL_OK;
}

}  // namespace

extern "C" {

sl_status sl_aggregate(const uint8_t* const* payloads, const float* const* scales,
                       int32_t n_peers, float* out, int64_t n, void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n_peers < 0 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n == 0) return SL_OK;
    if (!out) return SL_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return SL_ERR_ALIGN;
    if (n / SL_CHUNK > 0x7fffffff) return SL_ERR_SHAPE;
    sl::PeerTable table;
    const sl_status st = peer_table(payloads, scales, n_peers, out, n, &table);
    if (st != SL_OK) return st;
    return from_hip(sl::launch_aggregate(table, n_peers, out, n / SL_CHUNK,
                                         static_cast<hipStream_t>(stream)));
}

sl_status sl_aggregate_interleaved(const uint8_t* records, const float* scales, int32_t n_peers, float* out,
                                   int64_t n, void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n_peers < 0 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n == 0) return SL_OK;
    if (!out) return SL_ERR_INVALID_ARG;
    if (!aligned(out, 16)) return SL_ERR_ALIGN;
    const int64_t n_chunks = n / SL_CHUNK;
    if (n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    if (n_peers == 0) {
        const sl::PeerTable empty = {};
        return from_hip(sl::launch_aggregate(empty, 0, out, n_chunks, static_cast<hipStream_t>(stream)));
    }
    if (!records || !scales) return SL_ERR_INVALID_ARG;
    if (!aligned(records, 16) || !aligned(scales, 4)) return SL_ERR_ALIGN;
    const size_t dense = (size_t)n * sizeof(float);
    const size_t rbytes = (size_t)n_chunks * (size_t)n_peers * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * (size_t)n_peers * sizeof(float);
    if (overlap(out, dense, records, rbytes) || overlap(out, dense, scales, sbytes)) return SL_ERR_INVALID_ARG;
    return from_hip(sl::launch_aggregate_interleaved(records, scales, n_peers, out, n_chunks,
                                                     static_cast<hipStream_t>(stream)));
}

sl_status sl_aggregate_apply_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                         float* theta, int64_t n, void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n_peers < 1 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n == 0) return SL_OK;
    if (!theta || !records || !scales) return SL_ERR_INVALID_ARG;
    if (!aligned(theta, 16) || !aligned(records, 16) || !aligned(scales, 4)) return SL_ERR_ALIGN;
    const int64_t n_chunks = n / SL_CHUNK;
    if (n_chunks > 0x7fffffff) return SL_ERR_SHAPE;
    const size_t dense = (size_t)n * sizeof(float);
    const size_t rbytes = (size_t)n_chunks * (size_t)n_peers * SL_PAYLOAD_BYTES;
    const size_t sbytes = (size_t)n_chunks * (size_t)n_peers * sizeof(float);
    if (overlap(theta, dense, records, rbytes) || overlap(theta, dense, scales, sbytes)) return SL_ERR_INVALID_ARG;
    return from_hip(sl::launch_aggregate_apply_interleaved(records, scales, n_peers, theta, n_chunks,
                                                           static_cast<hipStream_t>(stream)));
}

sl_status sl_aggregate_apply(const uint8_t* const* payloads, const float* const* scales,
                             int32_t n_peers, float* theta, int64_t n, void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n_peers < 1 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n == 0) return SL_OK;
    if (!theta) return SL_ERR_INVALID_ARG;
    if (!aligned(theta, 16)) return SL_ERR_ALIGN;
    if (n / SL_CHUNK > 0x7fffffff) return SL_ERR_SHAPE;
    sl::PeerTable table;
    const sl_status st = peer_table(payloads, scales, n_peers, theta, n, &table);
    if (st != SL_OK) return st;
    return from_hip(sl::launch_aggregate_apply(table, n_peers, theta, n / SL_CHUNK,
                                               static_cast<hipStream_t>(stream)));
}

sl_status sl_apply_mean(float* theta, const float* out, int32_t n_peers, int64_t n,
                        void* stream) {
    if (n < 0 || n % SL_CHUNK != 0) return SL_ERR_SHAPE;
    if (n_peers < 1 || n_peers > SL_MAX_PEERS) return SL_ERR_TOO_MANY_PEERS;
    if (n == 0) return SL_OK;
    if (!theta || !out) return SL_ERR_INVALID_ARG;
    if (!aligned(theta, 16) || !aligned(out, 16)) return SL_ERR_ALIGN;
    const size_t dense = (size_t)n * sizeof(float);
    if (overlap(theta, dense, out, dense)) return SL_ERR_INVALID_ARG;
    return from_hip(sl::launch_apply_mean(theta, out, n_peers, n,
                                          static_cast<hipStream_t>(stream)));
}

sl_status sl_host_device_pointer(const void* host_ptr, void** device_ptr) {
    if (!host_ptr || !device_ptr) return SL_ERR_INVALID_ARG;
    *device_ptr = nullptr;
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(host_ptr), 0) != hipSuccess || !d) {
        (void)hipGetLastError();  // clear the error this query may leave behind
        return SL_ERR_INVALID_ARG;
    }
    *device_ptr = d;
    return SL_OK;
}

const char* sl_status_string(int status) {
    switch (status) {
        case SL_OK: return "SL_OK";
        case SL_ERR_INVALID_ARG: return "SL_ERR_INVALID_ARG: null pointer, non-finite beta or overlapping buffers";
        case SL_ERR_SHAPE: return "SL_ERR_SHAPE: n must be a non-negative multiple of 4096";
        case SL_ERR_ALIGN: return "SL_ERR_ALIGN: dense and payload buffers need 16-byte alignment, scales 4-byte";
        case SL_ERR_TOO_MANY_PEERS: return "SL_ERR_TOO_MANY_PEERS: n_peers outside the allowed range";
        case SL_ERR_HIP: return "SL_ERR_HIP: the HIP runtime reported a launch error";
        default: return "unknown sl_status";
    }
}

}  // extern "C"
