"""numpy front-end to the CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke entry point and by
the benchmark's CPU-baseline leg.  The product path never imports it.

Every function takes and returns numpy arrays; the arithmetic is all in
oracle.cpp.
"""
import ctypes
import os

import numpy as np

from .build import LIB, build_oracle

CHUNK = 4096
TOPK = 64
PAYLOAD_BYTES = 112

_lib = None


def lib():
    """Load liboracle.so, building it first if it is not there.  ORACLE_LIB
    names another build of oracle.cpp to load instead."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB", LIB)   # the mutation tests load planted variants
        if path == LIB and not os.path.exists(LIB):
            build_oracle()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        L.orc_compress_unpacked.argtypes = [P, P, i64, i32, i32, f32, P, P, P]
        L.orc_compress_unpacked.restype = ctypes.c_int
        L.orc_pack.argtypes = [P, P, i64, P]
        L.orc_pack.restype = None
        L.orc_unpack.argtypes = [P, i64, P, P]
        L.orc_unpack.restype = None
        L.orc_compress.argtypes = [P, P, i64, f32, P, P, i32]
        L.orc_compress.restype = ctypes.c_int
        L.orc_aggregate.argtypes = [P, P, i32, i64, P, i32]
        L.orc_aggregate.restype = ctypes.c_int
        L.orc_apply_mean.argtypes = [P, P, i32, i64]
        L.orc_apply_mean.restype = ctypes.c_int
        L.orc_validate.argtypes = [P, P, i64, P]
        L.orc_validate.restype = ctypes.c_int64
        L.orc_peer_stats.argtypes = [P, P, i64, P, P]
        L.orc_peer_stats.restype = None
        L.orc_pseudo_gradient.argtypes = [P, P, i64, P]
        L.orc_pseudo_gradient.restype = None
        L.orc_decode.argtypes = [ctypes.c_uint8, f32]
        L.orc_decode.restype = f32
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a


def compress_unpacked(delta, ef, chunk, k, beta):
    """Generic-chunk compressor.  Returns (idx[C,k] int32, code[C,k] uint8,
    scale[C] float32, new_ef float32); the input ef is not modified."""
    delta = _f32(delta)
    ef_new = _f32(ef).copy()
    n = delta.size
    assert ef_new.size == n and n % chunk == 0
    C = n // chunk
    idx = np.zeros((C, k), dtype=np.int32)
    code = np.zeros((C, k), dtype=np.uint8)
    scale = np.zeros(C, dtype=np.float32)
    rc = lib().orc_compress_unpacked(_ptr(delta), _ptr(ef_new), n, chunk, k,
                                     float(np.float32(beta)), _ptr(idx), _ptr(code),
                                     _ptr(scale))
    if rc != 0:
        raise ValueError("orc_compress_unpacked rejected its arguments")
    return idx, code, scale, ef_new


def pack(idx, code):
    idx = np.ascontiguousarray(idx, dtype=np.int32).reshape(-1, TOPK)
    code = np.ascontiguousarray(code, dtype=np.uint8).reshape(-1, TOPK)
    C = idx.shape[0]
    out = np.zeros((C, PAYLOAD_BYTES), dtype=np.uint8)
    lib().orc_pack(_ptr(idx), _ptr(code), C, _ptr(out))
    return out


def unpack(payload):
    payload = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1, PAYLOAD_BYTES)
    C = payload.shape[0]
    idx = np.zeros((C, TOPK), dtype=np.int32)
    code = np.zeros((C, TOPK), dtype=np.uint8)
    lib().orc_unpack(_ptr(payload), C, _ptr(idx), _ptr(code))
    return idx, code


def compress(delta, ef, beta=0.95, nthreads=1, inplace=False):
    """4096/64 compressor.  Returns (payload[C,112] uint8, scales[C] float32,
    new_ef).  With inplace=True, ef (a float32 contiguous array) is updated in
    place and returned as new_ef."""
    delta = _f32(delta).reshape(-1)
    if inplace:
        assert isinstance(ef, np.ndarray) and ef.dtype == np.float32 and ef.flags.c_contiguous
        ef_new = ef.reshape(-1)
    else:
        ef_new = _f32(ef).reshape(-1).copy()
    n = delta.size
    assert ef_new.size == n and n % CHUNK == 0
    C = n // CHUNK
    payload = np.zeros((C, PAYLOAD_BYTES), dtype=np.uint8)
    scales = np.zeros(C, dtype=np.float32)
    rc = lib().orc_compress(_ptr(delta), _ptr(ef_new), n, float(np.float32(beta)),
                            _ptr(payload), _ptr(scales), int(nthreads))
    if rc != 0:
        raise ValueError("orc_compress rejected its arguments")
    return payload, scales, ef_new


def aggregate(payloads, scales, n, nthreads=1):
    """Sum of the decoded payloads of len(payloads) peers into a float32[n]."""
    pl = [np.ascontiguousarray(p, dtype=np.uint8) for p in payloads]
    sc = [np.ascontiguousarray(s, dtype=np.float32) for s in scales]
    N = len(pl)
    assert len(sc) == N
    for p, s in zip(pl, sc):
        assert p.size == (n // CHUNK) * PAYLOAD_BYTES and s.size == n // CHUNK
    parr = (ctypes.c_void_p * max(N, 1))(*[p.ctypes.data for p in pl])
    sarr = (ctypes.c_void_p * max(N, 1))(*[s.ctypes.data for s in sc])
    out = np.empty(n, dtype=np.float32)
    rc = lib().orc_aggregate(ctypes.cast(parr, ctypes.c_void_p),
                             ctypes.cast(sarr, ctypes.c_void_p), N, n, _ptr(out),
                             int(nthreads))
    if rc != 0:
        raise ValueError("orc_aggregate rejected its arguments")
    return out


def apply_mean(theta, out, n_peers):
    th = _f32(theta).reshape(-1).copy()
    o = _f32(out).reshape(-1)
    assert th.size == o.size
    rc = lib().orc_apply_mean(_ptr(th), _ptr(o), int(n_peers), th.size)
    if rc != 0:
        raise ValueError("orc_apply_mean rejected its arguments")
    return th


def validate(payload, scales):
    payload = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1, PAYLOAD_BYTES)
    scales = _f32(scales).reshape(-1)
    C = payload.shape[0]
    assert scales.size == C
    bad = np.zeros(C, dtype=np.uint8)
    n_bad = lib().orc_validate(_ptr(payload), _ptr(scales), C, _ptr(bad))
    return int(n_bad), bad


def peer_stats(payload, scales):
    """Per-peer statistics of one peer's records: (counts int64[4], scale_max).
    counts = [records flagged by validate, records with scale +-0, entries at
    the magnitude level, entries with the sign bit]."""
    payload = np.ascontiguousarray(payload, dtype=np.uint8).reshape(-1, PAYLOAD_BYTES)
    scales = _f32(scales).reshape(-1)
    C = payload.shape[0]
    assert scales.size == C
    counts = np.zeros(4, dtype=np.int64)
    top = np.zeros(1, dtype=np.float32)
    lib().orc_peer_stats(_ptr(payload), _ptr(scales), C, _ptr(counts), _ptr(top))
    return counts, top[0]


def pseudo_gradient(theta_pre, theta_post):
    a = _f32(theta_pre).reshape(-1)
    b = _f32(theta_post).reshape(-1)
    assert a.size == b.size
    d = np.empty_like(a)
    lib().orc_pseudo_gradient(_ptr(a), _ptr(b), a.size, _ptr(d))
    return d


def decode(code, s):
    return np.float32(lib().orc_decode(int(code), float(np.float32(s))))
