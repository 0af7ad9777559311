// internal.h -- launchers shared between the C-ABI layer and the kernel
// translation units.  Arguments are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sparseloco.h"

namespace sl {

// Chunks per kernel launch.  A launch's work-items along x must fit in 32
// bits, which at 256 lanes per workgroup allows fewer than 2^24 chunks; larger
// spans are therefore split into launches of at most 2^22 chunks (17.2e9
// parameters).  Every output depends on its own chunk only, so the split
// changes no result.
constexpr int64_t kLaunchChunks = int64_t(1) << 22;

// The streaming kernels (compress, compress from weights, apply_mean) and the
// chunk-major aggregate and fused update split a long call further, into equal
// launches of at most kStreamLaunchChunks chunks: one launch per call up to
// 8192 x 28672 parameters, four for a decoder block, 60 for the
// 16e9-parameter span.  Measured on lognormal values: the decoder block's
// compress, compress from weights and apply_mean
// ran at 0.777-0.784, 0.780-0.785 and 0.791-0.793 of HBM in one launch against
// 0.799-0.802, 0.799-0.802 and 0.818-0.826 in three to five; the 16e9 span at
// 0.742-0.752, 0.748-0.751 and 0.761 against 0.763-0.767, 0.761-0.764 and
// 0.786-0.790 in 48 to 80.  Much smaller launches lose to their tails (8192 x
// 28672 in four launches: 0.775 against 0.792).  These kernels take their
// chunks in linear order and the dispatcher deals workgroups to the XCDs
// round-robin; the loss in long launches fits the eight XCDs' fronts drifting
// apart, which a launch boundary undoes (giving each XCD its own range of
// chunks outright measured 4-6% slower still).  The per-peer aggregate kernels
// use such ranges on purpose and keep one launch: splitting them measured
// slower.
constexpr int64_t kStreamLaunchChunks = int64_t(1) << 16;

// Chunks per launch for a streaming kernel over n_chunks chunks.
inline int64_t stream_launch_chunks(int64_t n_chunks) {
    const int64_t parts = (n_chunks + kStreamLaunchChunks - 1) / kStreamLaunchChunks;
    return parts <= 1 ? n_chunks : (n_chunks + parts - 1) / parts;
}

// Pointer table passed by value in the kernel arguments (2 KiB).
struct PeerTable {
    const uint8_t* payload[SL_MAX_PEERS];
    const float* scales[SL_MAX_PEERS];
};

hipError_t launch_compress(const float* delta, float* ef, float beta, uint8_t* payload,
                           float* scales, int64_t n_chunks, hipStream_t stream);

hipError_t launch_aggregate(const PeerTable& peers, int32_t n_peers, float* out,
                            int64_t n_chunks, hipStream_t stream);

// Records laid out chunk-major across peers: chunk c's record from peer p at
// records + (c * n_peers + p) * 112, its scale at scales[c * n_peers + p];
// n_peers >= 1.
hipError_t launch_aggregate_interleaved(const uint8_t* records, const float* scales, int32_t n_peers, float* out,
                                        int64_t n_chunks, hipStream_t stream);

// The fused update theta <- theta - sum / n_peers on interleaved records
// (n_peers >= 1).
hipError_t launch_aggregate_apply_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                              float* theta, int64_t n_chunks, hipStream_t stream);

hipError_t launch_aggregate_apply(const PeerTable& peers, int32_t n_peers, float* theta,
                                  int64_t n_chunks, hipStream_t stream);

// flags[p * n_chunks + c] for peer p < n_peers and record c < n_chunks.
hipError_t launch_validate(const PeerTable& peers, int32_t n_peers, int64_t n_chunks, uint8_t* flags,
                           hipStream_t stream);

// Per-peer statistics (and, if flags is not null, the validation flags) of
// n_peers peers' n_chunks records in one launch, 1 <= n_peers <= SL_MAX_PEERS.
// counts: int64[n_peers][4], scale_max: float32[n_peers], both overwritten.
// scratch_ptr: device memory of peer_stats_scratch_bytes() bytes, all zero (as
// a completed call leaves it); calls that share a scratch must not overlap.
size_t peer_stats_scratch_bytes();
// The current device's copy of the library's static statistics scratch
// (peer_stats_scratch_bytes() bytes, zero at load).
hipError_t peer_stats_static_scratch(void** ptr);
hipError_t launch_peer_stats(const PeerTable& peers, int32_t n_peers, int64_t n_chunks, uint8_t* flags,
                             int64_t* counts, float* scale_max, void* scratch_ptr, hipStream_t stream);

// The same statistics and flags for records laid out chunk-major (chunk c's
// record from peer p at records + (c * n_peers + p) * 112, its scale at
// scales[c * n_peers + p]), 1 <= n_peers <= SL_MAX_PEERS.  scratch_ptr: device
// memory of interleaved_stats_scratch_bytes() bytes, zero before the first
// call (a completed call leaves it zero); calls that share it must not overlap.
size_t interleaved_stats_scratch_bytes();
hipError_t launch_peer_stats_interleaved(const uint8_t* records, const float* scales, int32_t n_peers,
                                         int64_t n_chunks, uint8_t* flags, int64_t* counts, float* scale_max,
                                         void* scratch_ptr, hipStream_t stream);

hipError_t launch_compress_weights(const float* theta_pre, const float* theta_post, float* ef,
                                   float beta, uint8_t* payload, float* scales, int64_t n_chunks,
                                   hipStream_t stream);

hipError_t launch_apply_mean(float* theta, const float* out, int32_t n_peers,
                             int64_t n, hipStream_t stream);

}  // namespace sl
