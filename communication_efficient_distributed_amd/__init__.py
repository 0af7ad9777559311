"""SparseLoCo pseudo-gradient compressor and aggregator for MI355X (gfx950).

The compute path is the HIP library libsparseloco.so (C ABI in
include/sparseloco.h).  The functions re-exported here marshal torch device
tensors into that library and do no arithmetic of their own; they raise if the
library is not built.
"""
from . import datagen  # noqa: F401  (distributions only)
from ._lib import (  # noqa: F401
    LIB_PATH,
    SL_CHUNK,
    SL_MAX_PEERS,
    SL_PAYLOAD_BYTES,
    SL_TOPK,
    LibraryMissing,
    PeerSet,
    SparseLoCoError,
    aggregate,
    apply_mean,
    compress,
    host_device_pointer,
    load,
    sl_aggregate,
    sl_aggregate_apply,
    sl_aggregate_apply_interleaved,
    sl_aggregate_interleaved,
    sl_apply_mean,
    sl_compress,
    sl_compress_host_ef,
    sl_compress_weights,
    sl_peer_stats,
    sl_peer_stats_interleaved,
    sl_status_string,
    sl_validate_payload,
    sl_validate_payloads,
)
