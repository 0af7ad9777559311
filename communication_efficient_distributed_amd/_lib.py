"""ctypes binding of libsparseloco.so (declared in include/sparseloco.h).

Marshalling only: every function here passes device pointers, sizes and the
current HIP stream to the library and raises on a non-OK status.  There is no
fallback: if the library is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparseloco.so")

SL_CHUNK = 4096
SL_TOPK = 64
SL_PAYLOAD_BYTES = 112
SL_MAX_PEERS = 128

STATUS = {
    0: "SL_OK",
    1: "SL_ERR_INVALID_ARG",
    2: "SL_ERR_SHAPE",
    3: "SL_ERR_ALIGN",
    4: "SL_ERR_TOO_MANY_PEERS",
    5: "SL_ERR_HIP",
}

EXPORTS = ("sl_compress", "sl_compress_weights", "sl_aggregate", "sl_aggregate_interleaved", "sl_aggregate_apply",
           "sl_aggregate_apply_interleaved",
           "sl_apply_mean", "sl_validate_payload", "sl_validate_payloads", "sl_peer_stats",
           "sl_peer_stats_interleaved", "sl_peer_stats_noalloc", "sl_host_device_pointer", "sl_status_string")


class SparseLoCoError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text}")
        self.status = status


class LibraryMissing(ImportError):
    pass


_handle = None


def load():
    """Load libsparseloco.so once; raise LibraryMissing if it is not built."""
    global _handle
    if _handle is not None:
        return _handle
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing(
            f"{LIB_PATH} is not built; run `python communication_efficient_distributed_amd/_build.py` "
            "(hipcc --offload-arch=gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.sl_compress.argtypes = [P, P, F32, P, P, I64, P]
    L.sl_compress.restype = ctypes.c_int
    L.sl_compress_weights.argtypes = [P, P, P, F32, P, P, I64, P]
    L.sl_compress_weights.restype = ctypes.c_int
    L.sl_validate_payload.argtypes = [P, P, I64, P, P]
    L.sl_validate_payload.restype = ctypes.c_int
    L.sl_validate_payloads.argtypes = [P, P, I32, I64, P, P]
    L.sl_validate_payloads.restype = ctypes.c_int
    L.sl_peer_stats.argtypes = [P, P, I32, I64, P, P, P, P]
    L.sl_peer_stats.restype = ctypes.c_int
    L.sl_peer_stats_interleaved.argtypes = [P, P, I32, I64, P, P, P, P]
    L.sl_peer_stats_interleaved.restype = ctypes.c_int
    L.sl_peer_stats_noalloc.argtypes = [P, P, I32, I64, P, P, P, P]
    L.sl_peer_stats_noalloc.restype = ctypes.c_int
    L.sl_host_device_pointer.argtypes = [P, ctypes.POINTER(ctypes.c_void_p)]
    L.sl_host_device_pointer.restype = ctypes.c_int
    L.sl_aggregate.argtypes = [P, P, I32, P, I64, P]
    L.sl_aggregate.restype = ctypes.c_int
    L.sl_aggregate_interleaved.argtypes = [P, P, I32, P, I64, P]
    L.sl_aggregate_interleaved.restype = ctypes.c_int
    L.sl_aggregate_apply_interleaved.argtypes = [P, P, I32, P, I64, P]
    L.sl_aggregate_apply_interleaved.restype = ctypes.c_int
    L.sl_aggregate_apply.argtypes = [P, P, I32, P, I64, P]
    L.sl_aggregate_apply.restype = ctypes.c_int
    L.sl_apply_mean.argtypes = [P, P, I32, I64, P]
    L.sl_apply_mean.restype = ctypes.c_int
    L.sl_status_string.argtypes = [ctypes.c_int]
    L.sl_status_string.restype = ctypes.c_char_p
    _handle = L
    return L


def sl_status_string(status: int) -> str:
    return load().sl_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise SparseLoCoError(fn, status, sl_status_string(status))


def _stream_of(t: torch.Tensor, stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream))
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def sl_compress(delta: torch.Tensor, ef: torch.Tensor, beta: float, payload: torch.Tensor,
                scales: torch.Tensor, stream=None) -> None:
    """One compression round: ef updated in place, payload [C,112] uint8 and
    scales [C] float32 written.  Asynchronous on `stream` (default: current)."""
    n = delta.numel()
    if ef.numel() != n:
        raise ValueError("delta and ef sizes differ")
    C = n // SL_CHUNK
    if payload.numel() != C * SL_PAYLOAD_BYTES or scales.numel() != C:
        raise ValueError("payload must hold n/4096*112 bytes and scales n/4096 floats")
    args = (_dev(delta, "delta", torch.float32), _dev(ef, "ef", torch.float32),
            ctypes.c_float(beta), _dev(payload, "payload", torch.uint8),
            _dev(scales, "scales", torch.float32), ctypes.c_int64(n), _stream_of(delta, stream))
    with torch.cuda.device(delta.device):
        _check("sl_compress", load().sl_compress(*args))


def sl_compress_weights(theta_pre: torch.Tensor, theta_post: torch.Tensor, ef: torch.Tensor,
                        beta: float, payload: torch.Tensor, scales: torch.Tensor,
                        stream=None) -> None:
    """sl_compress with delta = theta_pre - theta_post formed inside the kernel."""
    n = theta_pre.numel()
    if theta_post.numel() != n or ef.numel() != n:
        raise ValueError("theta_pre, theta_post and ef sizes differ")
    C = n // SL_CHUNK
    if payload.numel() != C * SL_PAYLOAD_BYTES or scales.numel() != C:
        raise ValueError("payload must hold n/4096*112 bytes and scales n/4096 floats")
    args = (_dev(theta_pre, "theta_pre", torch.float32), _dev(theta_post, "theta_post", torch.float32),
            _dev(ef, "ef", torch.float32), ctypes.c_float(beta),
            _dev(payload, "payload", torch.uint8), _dev(scales, "scales", torch.float32),
            ctypes.c_int64(n), _stream_of(theta_pre, stream))
    with torch.cuda.device(theta_pre.device):
        _check("sl_compress_weights", load().sl_compress_weights(*args))


def host_device_pointer(t: torch.Tensor) -> int:
    """GPU address of a pinned host tensor (raises if it is not pinned and mapped)."""
    if t.device.type != "cpu" or not t.is_pinned():
        raise ValueError("expected a pinned host tensor (torch.empty(..., pin_memory=True))")
    out = ctypes.c_void_p()
    _check("sl_host_device_pointer", load().sl_host_device_pointer(ctypes.c_void_p(t.data_ptr()),
                                                                   ctypes.byref(out)))
    return int(out.value)


def sl_compress_host_ef(delta: torch.Tensor, ef_host: torch.Tensor, beta: float,
                        payload: torch.Tensor, scales: torch.Tensor, stream=None) -> None:
    """sl_compress with the error-feedback buffer offloaded to pinned host memory:
    the kernel reads and writes it in place over the host link."""
    n = delta.numel()
    if ef_host.numel() != n or ef_host.dtype != torch.float32 or not ef_host.is_contiguous():
        raise ValueError("ef_host must be a contiguous float32 tensor of delta's size")
    C = n // SL_CHUNK
    if payload.numel() != C * SL_PAYLOAD_BYTES or scales.numel() != C:
        raise ValueError("payload must hold n/4096*112 bytes and scales n/4096 floats")
    ef_dev = host_device_pointer(ef_host)
    args = (_dev(delta, "delta", torch.float32), ctypes.c_void_p(ef_dev), ctypes.c_float(beta),
            _dev(payload, "payload", torch.uint8), _dev(scales, "scales", torch.float32),
            ctypes.c_int64(n), _stream_of(delta, stream))
    with torch.cuda.device(delta.device):
        _check("sl_compress", load().sl_compress(*args))


def sl_validate_payload(payload: torch.Tensor, scales: torch.Tensor, flags: torch.Tensor,
                        stream=None) -> None:
    """flags[c] = 0 for a well-formed record c, else bit 0 = indices not strictly
    increasing, bit 1 = scale not finite, bit 2 = scale negative."""
    C = scales.numel()
    if payload.numel() != C * SL_PAYLOAD_BYTES or flags.numel() != C:
        raise ValueError("payload must hold C*112 bytes and flags C bytes")
    args = (_dev(payload, "payload", torch.uint8), _dev(scales, "scales", torch.float32),
            ctypes.c_int64(C), _dev(flags, "flags", torch.uint8), _stream_of(payload, stream))
    with torch.cuda.device(payload.device):
        _check("sl_validate_payload", load().sl_validate_payload(*args))


def sl_validate_payloads(payloads, scales, flags: torch.Tensor, stream=None) -> None:
    """sl_validate_payload for every peer in one launch: flags is uint8
    [n_peers, n_chunks], row p for peer p."""
    N = len(payloads)
    if flags.dim() != 2 or flags.shape[0] != N:
        raise ValueError("flags must be a [n_peers, n_chunks] tensor")
    if isinstance(payloads, PeerSet) and payloads.device is not None and flags.device != payloads.device:
        raise ValueError("flags must be on the peers' device")
    C = flags.shape[1]
    N, pa, sa, _keep = _peer_arrays(payloads, scales, C)
    f = _dev(flags, "flags", torch.uint8)
    with torch.cuda.device(flags.device):
        _check("sl_validate_payloads", load().sl_validate_payloads(pa, sa, ctypes.c_int32(N),
                                                                   ctypes.c_int64(C), f,
                                                                   _stream_of(flags, stream)))


def sl_peer_stats(payloads, scales, counts: torch.Tensor, scale_max: torch.Tensor, flags=None,
                  n_chunks: int | None = None, stream=None, noalloc: bool = False) -> None:
    """Per-peer statistics of the received records, one pass.  counts is int64
    [n_peers, 4]: records flagged by validation, records with scale +-0,
    entries at the magnitude level, entries with the sign bit; scale_max is
    float32 [n_peers], the largest finite non-negative scale.  flags, if given,
    is uint8 [n_peers, n_chunks] and receives the validation flags.  n_chunks
    defaults to the peers' record count (peer 0's, or the PeerSet's).  With
    noalloc, sl_peer_stats_noalloc is called instead (the library's static
    scratch; nothing is allocated)."""
    N = len(payloads)
    if counts.dim() != 2 or tuple(counts.shape) != (N, 4):
        raise ValueError("counts must be a [n_peers, 4] tensor")
    if scale_max.numel() != N:
        raise ValueError("scale_max must hold n_peers floats")
    if n_chunks is None:
        if flags is not None:
            n_chunks = flags.shape[1] if flags.dim() == 2 else -1
        elif isinstance(payloads, PeerSet):
            n_chunks = payloads.n_chunks
        else:
            n_chunks = scales[0].numel() if N else 0
    if flags is not None and (flags.dim() != 2 or tuple(flags.shape) != (N, n_chunks)):
        raise ValueError("flags must be a [n_peers, n_chunks] tensor")
    N, pa, sa, _keep = _peer_arrays(payloads, scales, n_chunks)
    c = _dev(counts, "counts", torch.int64)
    m = _dev(scale_max, "scale_max", torch.float32)
    f = _dev(flags, "flags", torch.uint8) if flags is not None else ctypes.c_void_p(None)
    name = "sl_peer_stats_noalloc" if noalloc else "sl_peer_stats"
    with torch.cuda.device(counts.device):
        _check(name, getattr(load(), name)(pa, sa, ctypes.c_int32(N), ctypes.c_int64(n_chunks), f, c, m,
                                           _stream_of(counts, stream)))


def sl_peer_stats_interleaved(records: torch.Tensor, scales: torch.Tensor, counts: torch.Tensor,
                              scale_max: torch.Tensor, flags=None, stream=None) -> None:
    """sl_peer_stats on records laid out chunk-major across peers (records
    uint8 [n_chunks, n_peers, 112], scales float32 [n_chunks, n_peers]);
    counts, scale_max and flags ([n_peers, n_chunks]) per peer, as
    sl_peer_stats writes them."""
    if records.dim() != 3 or records.shape[2] != SL_PAYLOAD_BYTES:
        raise ValueError("records must be a [n_chunks, n_peers, 112] tensor")
    C, N = records.shape[0], records.shape[1]
    if scales.dim() != 2 or tuple(scales.shape) != (C, N):
        raise ValueError("scales must be a [n_chunks, n_peers] tensor")
    if counts.dim() != 2 or tuple(counts.shape) != (N, 4):
        raise ValueError("counts must be a [n_peers, 4] tensor")
    if scale_max.numel() != N:
        raise ValueError("scale_max must hold n_peers floats")
    if flags is not None and (flags.dim() != 2 or tuple(flags.shape) != (N, C)):
        raise ValueError("flags must be a [n_peers, n_chunks] tensor")
    if N and C:
        r, s = _dev(records, "records", torch.uint8), _dev(scales, "scales", torch.float32)
    else:
        r = s = ctypes.c_void_p(None)
    c = _dev(counts, "counts", torch.int64)
    m = _dev(scale_max, "scale_max", torch.float32)
    f = _dev(flags, "flags", torch.uint8) if flags is not None else ctypes.c_void_p(None)
    with torch.cuda.device(counts.device):
        _check("sl_peer_stats_interleaved", load().sl_peer_stats_interleaved(r, s, ctypes.c_int32(N), ctypes.c_int64(C),
                                                                             f, c, m, _stream_of(counts, stream)))


class PeerSet:
    """The peers' record and scale tensors, checked once, with the C pointer
    tables kept for repeated calls (receive buffers reused round after round).
    Pass it as `payloads` (with `scales=None`) to sl_aggregate,
    sl_aggregate_apply, aggregate, sl_validate_payloads and sl_peer_stats.  The tensors are
    held, so their storage stays alive; their contents may change between
    calls, their storage must not be replaced."""

    def __init__(self, payloads, scales):
        payloads, scales = list(payloads), list(scales)
        if len(payloads) != len(scales):
            raise ValueError("payloads and scales lists differ in length")
        if len(payloads) > SL_MAX_PEERS:
            raise ValueError(f"at most {SL_MAX_PEERS} peers")
        C = scales[0].numel() if scales else 0
        self.n_peers = len(payloads)
        self.n_chunks = C
        self.device = payloads[0].device if payloads else None
        pp = (ctypes.c_void_p * max(self.n_peers, 1))()
        sp = (ctypes.c_void_p * max(self.n_peers, 1))()
        for p in range(self.n_peers):
            if payloads[p].numel() != C * SL_PAYLOAD_BYTES or scales[p].numel() != C:
                raise ValueError(f"peer {p}: payload/scales sizes differ from peer 0's")
            pp[p] = _dev(payloads[p], f"payloads[{p}]", torch.uint8).value
            sp[p] = _dev(scales[p], f"scales[{p}]", torch.float32).value
        self._tensors = (payloads, scales)
        self._arrays = (pp, sp)
        self.pa = ctypes.cast(pp, ctypes.c_void_p)
        self.sa = ctypes.cast(sp, ctypes.c_void_p)

    def __len__(self):
        return self.n_peers


def _peer_arrays(payloads, scales, C):
    if isinstance(payloads, PeerSet):
        if payloads.n_peers and payloads.n_chunks != C:
            raise ValueError("peer records do not match the dense buffer")
        return payloads.n_peers, payloads.pa, payloads.sa, payloads
    if scales is None or len(payloads) != len(scales):
        raise ValueError("payloads and scales lists differ in length")
    N = len(payloads)
    pp = (ctypes.c_void_p * max(N, 1))()
    sp = (ctypes.c_void_p * max(N, 1))()
    for p in range(N):
        if payloads[p].numel() != C * SL_PAYLOAD_BYTES or scales[p].numel() != C:
            raise ValueError(f"peer {p}: payload/scales size does not match the dense buffer")
        pp[p] = _dev(payloads[p], f"payloads[{p}]", torch.uint8).value
        sp[p] = _dev(scales[p], f"scales[{p}]", torch.float32).value
    return N, ctypes.cast(pp, ctypes.c_void_p), ctypes.cast(sp, ctypes.c_void_p), (pp, sp)


def sl_aggregate(payloads, scales, out: torch.Tensor, stream=None) -> None:
    """out[n] = sum over peers (in list order) of the decoded payloads."""
    n = out.numel()
    N, pa, sa, _keep = _peer_arrays(payloads, scales, n // SL_CHUNK)
    o = _dev(out, "out", torch.float32)
    with torch.cuda.device(out.device):
        _check("sl_aggregate", load().sl_aggregate(pa, sa, ctypes.c_int32(N), o, ctypes.c_int64(n),
                                                   _stream_of(out, stream)))


def sl_aggregate_interleaved(records: torch.Tensor, scales: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    """sl_aggregate on records laid out chunk-major across peers: records is
    uint8 [n/4096, n_peers, 112] and scales float32 [n/4096, n_peers]; out is
    float32 [n].  The same sums as sl_aggregate on the per-peer buffers."""
    if records.dim() != 3 or records.shape[2] != SL_PAYLOAD_BYTES:
        raise ValueError("records must be a [n_chunks, n_peers, 112] tensor")
    C, N = records.shape[0], records.shape[1]
    if scales.dim() != 2 or tuple(scales.shape) != (C, N):
        raise ValueError("scales must be a [n_chunks, n_peers] tensor")
    n = out.numel()
    if n != C * SL_CHUNK:
        raise ValueError("out must hold n_chunks * 4096 floats")
    o = _dev(out, "out", torch.float32)
    if N:
        r, s = _dev(records, "records", torch.uint8), _dev(scales, "scales", torch.float32)
    else:
        r = s = ctypes.c_void_p(None)
    with torch.cuda.device(out.device):
        _check("sl_aggregate_interleaved", load().sl_aggregate_interleaved(r, s, ctypes.c_int32(N), o, ctypes.c_int64(n),
                                                                           _stream_of(out, stream)))


def sl_aggregate_apply_interleaved(records: torch.Tensor, scales: torch.Tensor, theta: torch.Tensor,
                                   stream=None) -> None:
    """sl_aggregate_apply on records laid out chunk-major across peers (records
    uint8 [n/4096, n_peers, 112], scales float32 [n/4096, n_peers]): theta <-
    theta - sum / n_peers in one pass."""
    if records.dim() != 3 or records.shape[2] != SL_PAYLOAD_BYTES:
        raise ValueError("records must be a [n_chunks, n_peers, 112] tensor")
    C, N = records.shape[0], records.shape[1]
    if scales.dim() != 2 or tuple(scales.shape) != (C, N):
        raise ValueError("scales must be a [n_chunks, n_peers] tensor")
    n = theta.numel()
    if n != C * SL_CHUNK:
        raise ValueError("theta must hold n_chunks * 4096 floats")
    t = _dev(theta, "theta", torch.float32)
    r, s = _dev(records, "records", torch.uint8), _dev(scales, "scales", torch.float32)
    with torch.cuda.device(theta.device):
        _check("sl_aggregate_apply_interleaved",
               load().sl_aggregate_apply_interleaved(r, s, ctypes.c_int32(N), t, ctypes.c_int64(n),
                                                     _stream_of(theta, stream)))


def sl_aggregate_apply(payloads, scales, theta: torch.Tensor, stream=None) -> None:
    """theta <- theta - (sum over peers of the decoded payloads) / n_peers."""
    n = theta.numel()
    N, pa, sa, _keep = _peer_arrays(payloads, scales, n // SL_CHUNK)
    t = _dev(theta, "theta", torch.float32)
    with torch.cuda.device(theta.device):
        _check("sl_aggregate_apply", load().sl_aggregate_apply(pa, sa, ctypes.c_int32(N), t,
                                                               ctypes.c_int64(n),
                                                               _stream_of(theta, stream)))


def sl_apply_mean(theta: torch.Tensor, out: torch.Tensor, n_peers: int, stream=None) -> None:
    """theta <- theta - out / n_peers (in place)."""
    n = theta.numel()
    if out.numel() != n:
        raise ValueError("theta and out sizes differ")
    args = (_dev(theta, "theta", torch.float32), _dev(out, "out", torch.float32),
            ctypes.c_int32(n_peers), ctypes.c_int64(n), _stream_of(theta, stream))
    with torch.cuda.device(theta.device):
        _check("sl_apply_mean", load().sl_apply_mean(*args))


# Convenience wrappers that allocate outputs with torch (device memory only).

def compress(delta: torch.Tensor, ef: torch.Tensor, beta: float = 0.95, stream=None):
    """sl_compress into freshly allocated outputs: returns (payload uint8
    [n/4096, 112], scales float32 [n/4096]); ef is updated in place."""
    C = delta.numel() // SL_CHUNK
    payload = torch.empty((C, SL_PAYLOAD_BYTES), dtype=torch.uint8, device=delta.device)
    scales = torch.empty(C, dtype=torch.float32, device=delta.device)
    sl_compress(delta, ef, beta, payload, scales, stream)
    return payload, scales


def aggregate(payloads, scales=None, n: int | None = None, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """sl_aggregate, allocating out (float32 [n]) unless it is given; n
    defaults to what the peers' records cover."""
    if out is None:
        if isinstance(payloads, PeerSet):
            if n is None:
                n = payloads.n_chunks * SL_CHUNK
            dev = payloads.device or torch.device("cuda")
        else:
            if n is None:
                n = payloads[0].numel() // SL_PAYLOAD_BYTES * SL_CHUNK
            dev = payloads[0].device if payloads else torch.device("cuda")
        out = torch.empty(n, dtype=torch.float32, device=dev)
    sl_aggregate(payloads, scales, out, stream)
    return out


def apply_mean(theta: torch.Tensor, out: torch.Tensor, n_peers: int, stream=None) -> torch.Tensor:
    """theta <- theta - out / n_peers in place (sl_apply_mean); returns theta."""
    sl_apply_mean(theta, out, n_peers, stream)
    return theta
