"""Host-side tests of the C ABI (include/sparseloco.h): the library loads, exports
every declared entry point, and rejects bad arguments with the documented status
before anything reaches the GPU.  No compute call is made here.

Pointer arguments are fake addresses: argument checks never dereference them.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparseloco.h")

SL_OK, SL_ERR_INVALID_ARG, SL_ERR_SHAPE, SL_ERR_ALIGN, SL_ERR_TOO_MANY_PEERS, SL_ERR_HIP = range(6)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sl_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from communication_efficient_distributed_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from communication_efficient_distributed_amd import _build
        _build.build_library()
    return _lib.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("sl_compress", "sl_compress_weights", "sl_aggregate", "sl_aggregate_apply",
              "sl_apply_mean", "sl_validate_payload", "sl_validate_payloads", "sl_peer_stats",
              "sl_host_device_pointer", "sl_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (sl_\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_header_constants_match_pages():
    """The layout constants in the header: 4096-chunks, top 64, 12-bit indices,
    2-bit codes, 112-byte records (The Sparse Frontier, Three Compression
    Levers)."""
    text = open(HEADER).read()
    val = lambda k: int(re.search(rf"#define {k} (\d+)", text).group(1))
    assert val("SL_CHUNK") == 4096 and val("SL_TOPK") == 64
    assert val("SL_INDEX_BITS") == 12 and val("SL_CODE_BITS") == 2
    assert val("SL_PAYLOAD_BYTES") == 112 == val("SL_INDEX_BYTES") + val("SL_CODE_BYTES")
    assert val("SL_TOPK") * (val("SL_INDEX_BITS") + val("SL_CODE_BITS")) == 8 * val("SL_PAYLOAD_BYTES")


def test_status_strings(lib):
    for code, name in enumerate(["SL_OK", "SL_ERR_INVALID_ARG", "SL_ERR_SHAPE", "SL_ERR_ALIGN",
                                 "SL_ERR_TOO_MANY_PEERS", "SL_ERR_HIP"]):
        assert lib.sl_status_string(code).decode().startswith(name)
    assert lib.sl_status_string(99).decode() == "unknown sl_status"


A = 1 << 20  # fake, 16-byte aligned device addresses far apart
D, E, P, S, O, T = (A * k for k in (1, 200, 400, 600, 800, 1000))
N = 16 * 4096
beta = ctypes.c_float(0.95)


def comp(lib, d=D, e=E, b=beta, p=P, s=S, n=N):
    return lib.sl_compress(d, e, b, p, s, n, None)


def test_compress_argument_checks(lib):
    assert comp(lib, n=4095) == SL_ERR_SHAPE
    assert comp(lib, n=-4096) == SL_ERR_SHAPE
    assert comp(lib, n=0) == SL_OK                       # no-op, nothing enqueued
    assert comp(lib, d=None) == SL_ERR_INVALID_ARG
    assert comp(lib, e=None) == SL_ERR_INVALID_ARG
    assert comp(lib, p=None) == SL_ERR_INVALID_ARG
    assert comp(lib, s=None) == SL_ERR_INVALID_ARG
    assert comp(lib, b=ctypes.c_float(float("nan"))) == SL_ERR_INVALID_ARG
    assert comp(lib, b=ctypes.c_float(float("inf"))) == SL_ERR_INVALID_ARG
    assert comp(lib, d=D + 4) == SL_ERR_ALIGN
    assert comp(lib, e=E + 8) == SL_ERR_ALIGN
    assert comp(lib, p=P + 4) == SL_ERR_ALIGN
    assert comp(lib, s=S + 2) == SL_ERR_ALIGN
    # overlaps: ef inside delta (but not identical), payload or scales inside delta/ef
    assert comp(lib, e=D + 4096) == SL_ERR_INVALID_ARG
    assert comp(lib, p=D + 16) == SL_ERR_INVALID_ARG
    assert comp(lib, s=E + 64) == SL_ERR_INVALID_ARG
    assert comp(lib, s=P + 16) == SL_ERR_INVALID_ARG


def agg(lib, peers, scales, n_peers, out=O, n=N):
    pa = (ctypes.c_void_p * max(len(peers), 1))(*peers)
    sa = (ctypes.c_void_p * max(len(scales), 1))(*scales)
    return lib.sl_aggregate(ctypes.cast(pa, ctypes.c_void_p), ctypes.cast(sa, ctypes.c_void_p),
                            n_peers, out, n, None)


def test_aggregate_argument_checks(lib):
    pp = [P + k * A for k in range(3)]
    ss = [S + k * A for k in range(3)]
    assert agg(lib, pp, ss, 3, n=100) == SL_ERR_SHAPE
    assert agg(lib, pp, ss, -1) == SL_ERR_TOO_MANY_PEERS
    assert agg(lib, pp, ss, 129) == SL_ERR_TOO_MANY_PEERS
    assert agg(lib, pp, ss, 3, n=0) == SL_OK
    assert agg(lib, pp, ss, 3, out=None) == SL_ERR_INVALID_ARG
    assert agg(lib, pp, ss, 3, out=O + 4) == SL_ERR_ALIGN
    assert agg(lib, [pp[0], None, pp[2]], ss, 3) == SL_ERR_INVALID_ARG
    assert agg(lib, pp, [ss[0], ss[1], None], 3) == SL_ERR_INVALID_ARG
    assert agg(lib, [pp[0], pp[1] + 8, pp[2]], ss, 3) == SL_ERR_ALIGN
    assert agg(lib, pp, [ss[0], ss[1] + 1, ss[2]], 3) == SL_ERR_ALIGN
    assert agg(lib, [O + 4096] + pp[1:], ss, 3) == SL_ERR_INVALID_ARG      # out overlaps a record
    assert agg(lib, pp, [O + 64] + ss[1:], 3) == SL_ERR_INVALID_ARG        # out overlaps scales
    assert lib.sl_aggregate(None, None, 2, O, N, None) == SL_ERR_INVALID_ARG


def test_aggregate_interleaved_argument_checks(lib):
    """Every call here is rejected (or is a no-op) on the host, before any
    launch.  N = 16 chunks: records 3 x 16 x 112 bytes from R, scales from S."""
    R = P
    f = lib.sl_aggregate_interleaved
    assert f(R, S, 3, O, 100, None) == SL_ERR_SHAPE
    assert f(R, S, 3, O, -4096, None) == SL_ERR_SHAPE
    assert f(R, S, -1, O, N, None) == SL_ERR_TOO_MANY_PEERS
    assert f(R, S, 129, O, N, None) == SL_ERR_TOO_MANY_PEERS
    assert f(R, S, 3, O, 0, None) == SL_OK                              # no-op
    assert f(R, S, 3, None, N, None) == SL_ERR_INVALID_ARG
    assert f(R, S, 3, O + 4, N, None) == SL_ERR_ALIGN
    assert f(None, S, 3, O, N, None) == SL_ERR_INVALID_ARG
    assert f(R, None, 3, O, N, None) == SL_ERR_INVALID_ARG
    assert f(R + 8, S, 3, O, N, None) == SL_ERR_ALIGN
    assert f(R, S + 2, 3, O, N, None) == SL_ERR_ALIGN
    assert f(O + 4096, S, 3, O, N, None) == SL_ERR_INVALID_ARG          # records inside out
    assert f(R, O + 64, 3, O, N, None) == SL_ERR_INVALID_ARG            # scales inside out
    assert f(O - 3 * 16 * 112 + 16, S, 3, O, N, None) == SL_ERR_INVALID_ARG   # records reach out


def test_aggregate_apply_interleaved_argument_checks(lib):
    """Rejected on the host before any launch (theta at T, records at P, scales at S)."""
    f = lib.sl_aggregate_apply_interleaved
    assert f(P, S, 3, T, 100, None) == SL_ERR_SHAPE
    assert f(P, S, 0, T, N, None) == SL_ERR_TOO_MANY_PEERS
    assert f(P, S, 129, T, N, None) == SL_ERR_TOO_MANY_PEERS
    assert f(P, S, 3, T, 0, None) == SL_OK                              # no-op
    assert f(P, S, 3, None, N, None) == SL_ERR_INVALID_ARG
    assert f(None, S, 3, T, N, None) == SL_ERR_INVALID_ARG
    assert f(P, None, 3, T, N, None) == SL_ERR_INVALID_ARG
    assert f(P, S, 3, T + 4, N, None) == SL_ERR_ALIGN
    assert f(P + 8, S, 3, T, N, None) == SL_ERR_ALIGN
    assert f(P, S + 2, 3, T, N, None) == SL_ERR_ALIGN
    assert f(T + 4096, S, 3, T, N, None) == SL_ERR_INVALID_ARG          # records inside theta
    assert f(P, T + 64, 3, T, N, None) == SL_ERR_INVALID_ARG            # scales inside theta


def test_apply_mean_argument_checks(lib):
    assert lib.sl_apply_mean(T, O, 24, 4097, None) == SL_ERR_SHAPE
    assert lib.sl_apply_mean(T, O, 0, N, None) == SL_ERR_TOO_MANY_PEERS
    assert lib.sl_apply_mean(T, O, 129, N, None) == SL_ERR_TOO_MANY_PEERS
    assert lib.sl_apply_mean(T, O, 24, 0, None) == SL_OK
    assert lib.sl_apply_mean(None, O, 24, N, None) == SL_ERR_INVALID_ARG
    assert lib.sl_apply_mean(T, None, 24, N, None) == SL_ERR_INVALID_ARG
    assert lib.sl_apply_mean(T + 4, O, 24, N, None) == SL_ERR_ALIGN
    assert lib.sl_apply_mean(T, T + 16, 24, N, None) == SL_ERR_INVALID_ARG


def test_binding_rejects_host_tensors():
    import communication_efficient_distributed_amd as sl
    d = torch.zeros(4096)
    with pytest.raises((ValueError, TypeError)):
        sl.sl_compress(d, torch.zeros(4096), 0.95, torch.zeros((1, 112), dtype=torch.uint8),
                       torch.zeros(1))
    with pytest.raises((ValueError, TypeError)):
        sl.apply_mean(torch.zeros(4096), torch.zeros(4096), 3)


def test_binding_fails_loudly_without_library(tmp_path):
    """With the library missing, the product path raises; there is no fallback."""
    code = (
        "import communication_efficient_distributed_amd._lib as L\n"
        f"L.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "L._handle = None\n"
        "try:\n"
        "    L.load()\n"
        "except L.LibraryMissing as e:\n"
        "    print('raised', e)\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "raised" in r.stdout, r.stdout + r.stderr


def test_aggregate_apply_argument_checks(lib):
    pp = [P + k * A for k in range(3)]
    ss = [S + k * A for k in range(3)]

    def call(peers, scales, n_peers, theta=T, n=N):
        pa = (ctypes.c_void_p * max(len(peers), 1))(*peers)
        sa = (ctypes.c_void_p * max(len(scales), 1))(*scales)
        return lib.sl_aggregate_apply(ctypes.cast(pa, ctypes.c_void_p), ctypes.cast(sa, ctypes.c_void_p),
                                      n_peers, theta, n, None)

    assert call(pp, ss, 3, n=4096 + 1) == SL_ERR_SHAPE
    assert call(pp, ss, 0) == SL_ERR_TOO_MANY_PEERS          # the mean needs a peer
    assert call(pp, ss, 129) == SL_ERR_TOO_MANY_PEERS
    assert call(pp, ss, 3, n=0) == SL_OK
    assert call(pp, ss, 3, theta=None) == SL_ERR_INVALID_ARG
    assert call(pp, ss, 3, theta=T + 8) == SL_ERR_ALIGN
    assert call([pp[0], None, pp[2]], ss, 3) == SL_ERR_INVALID_ARG
    assert call([T + 4096] + pp[1:], ss, 3) == SL_ERR_INVALID_ARG    # theta overlaps a record


def test_compress_weights_argument_checks(lib):
    def call(a=D, b=D + 100 * A, e=E, bt=beta, p=P, s=S, n=N):
        return lib.sl_compress_weights(a, b, e, bt, p, s, n, None)
    assert call(n=4095) == SL_ERR_SHAPE
    assert call(n=0) == SL_OK
    assert call(a=None) == SL_ERR_INVALID_ARG
    assert call(b=None) == SL_ERR_INVALID_ARG
    assert call(bt=ctypes.c_float(float("nan"))) == SL_ERR_INVALID_ARG
    assert call(a=D + 4) == SL_ERR_ALIGN
    assert call(b=D + 100 * A + 8) == SL_ERR_ALIGN
    assert call(e=D + 4096) == SL_ERR_INVALID_ARG            # ef overlaps theta_pre
    assert call(p=D + 100 * A + 16) == SL_ERR_INVALID_ARG    # payload overlaps theta_post
    # theta_pre and theta_post may be the same buffer (read only): argument checks pass,
    # so only check that the aliasing itself is not what is rejected
    assert call(b=D, n=0) == SL_OK


def test_validate_argument_checks(lib):
    F = A * 1200
    assert lib.sl_validate_payload(P, S, -1, F, None) == SL_ERR_SHAPE
    assert lib.sl_validate_payload(P, S, 0, F, None) == SL_OK
    assert lib.sl_validate_payload(None, S, 16, F, None) == SL_ERR_INVALID_ARG
    assert lib.sl_validate_payload(P, None, 16, F, None) == SL_ERR_INVALID_ARG
    assert lib.sl_validate_payload(P, S, 16, None, None) == SL_ERR_INVALID_ARG
    assert lib.sl_validate_payload(P + 4, S, 16, F, None) == SL_ERR_ALIGN
    assert lib.sl_validate_payload(P, S + 2, 16, F, None) == SL_ERR_ALIGN
    assert lib.sl_validate_payload(P, S, 16, P + 100, None) == SL_ERR_INVALID_ARG   # flags overlap


def test_host_device_pointer_null_arguments(lib):
    out = ctypes.c_void_p(1)
    assert lib.sl_host_device_pointer(None, ctypes.byref(out)) == SL_ERR_INVALID_ARG
    assert lib.sl_host_device_pointer(A, None) == SL_ERR_INVALID_ARG


def test_validate_many_argument_checks(lib):
    F = A * 1200
    pp = [P + k * A for k in range(3)]
    ss = [S + k * A for k in range(3)]

    def call(peers, scales, n_peers, n_chunks=16, flags=F):
        pa = (ctypes.c_void_p * max(len(peers), 1))(*peers)
        sa = (ctypes.c_void_p * max(len(scales), 1))(*scales)
        return lib.sl_validate_payloads(ctypes.cast(pa, ctypes.c_void_p), ctypes.cast(sa, ctypes.c_void_p),
                                        n_peers, n_chunks, flags, None)

    assert call(pp, ss, 3, n_chunks=-1) == SL_ERR_SHAPE
    assert call(pp, ss, -1) == SL_ERR_TOO_MANY_PEERS
    assert call(pp, ss, 129) == SL_ERR_TOO_MANY_PEERS
    assert call(pp, ss, 0) == SL_OK                       # no-op
    assert call(pp, ss, 3, n_chunks=0) == SL_OK
    assert call(pp, ss, 3, flags=None) == SL_ERR_INVALID_ARG
    assert call([pp[0], None, pp[2]], ss, 3) == SL_ERR_INVALID_ARG
    assert call(pp, [ss[0], None, ss[2]], 3) == SL_ERR_INVALID_ARG
    assert call([pp[0], pp[1] + 8, pp[2]], ss, 3) == SL_ERR_ALIGN
    assert call(pp, [ss[0], ss[1] + 2, ss[2]], 3) == SL_ERR_ALIGN
    assert call(pp, ss, 3, flags=pp[1] + 16) == SL_ERR_INVALID_ARG      # flags overlap a record
    assert call(pp, ss, 3, flags=ss[2] - 8) == SL_ERR_INVALID_ARG       # flags (48 bytes) reach a scale buffer
    assert lib.sl_validate_payloads(None, None, 2, 16, F, None) == SL_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["sl_peer_stats", "sl_peer_stats_noalloc"])
def test_peer_stats_argument_checks(lib, name):
    """Every call here is rejected (or is a no-op) on the host, before any
    launch (and, for sl_peer_stats, before its scratch is allocated)."""
    fn = getattr(lib, name)
    F = A * 1200
    CNT = A * 1300
    MX = A * 1400
    pp = [P + k * A for k in range(3)]
    ss = [S + k * A for k in range(3)]

    def call(peers, scales, n_peers, n_chunks=16, flags=F, counts=CNT, smax=MX):
        pa = (ctypes.c_void_p * max(len(peers), 1))(*peers)
        sa = (ctypes.c_void_p * max(len(scales), 1))(*scales)
        return fn(ctypes.cast(pa, ctypes.c_void_p), ctypes.cast(sa, ctypes.c_void_p),
                  n_peers, n_chunks, flags, counts, smax, None)

    assert call(pp, ss, 3, n_chunks=-1) == SL_ERR_SHAPE
    assert call(pp, ss, 3, n_chunks=1 << 31) == SL_ERR_SHAPE
    assert call(pp, ss, -1) == SL_ERR_TOO_MANY_PEERS
    assert call(pp, ss, 129) == SL_ERR_TOO_MANY_PEERS
    assert call(pp, ss, 0) == SL_OK                                     # no-op
    assert call(pp, ss, 3, counts=None) == SL_ERR_INVALID_ARG
    assert call(pp, ss, 3, smax=None) == SL_ERR_INVALID_ARG
    assert call(pp, ss, 3, counts=CNT + 4) == SL_ERR_ALIGN
    assert call(pp, ss, 3, smax=MX + 2) == SL_ERR_ALIGN
    assert call([pp[0], None, pp[2]], ss, 3) == SL_ERR_INVALID_ARG
    assert call(pp, [ss[0], None, ss[2]], 3) == SL_ERR_INVALID_ARG
    assert call([pp[0], pp[1] + 8, pp[2]], ss, 3) == SL_ERR_ALIGN
    assert call(pp, [ss[0], ss[1] + 2, ss[2]], 3) == SL_ERR_ALIGN
    assert call(pp, ss, 3, counts=MX - 8) == SL_ERR_INVALID_ARG         # counts (96 bytes) reach scale_max
    assert call(pp, ss, 3, flags=CNT - 8) == SL_ERR_INVALID_ARG         # flags (48 bytes) reach counts
    assert call(pp, ss, 3, counts=pp[1] + 16) == SL_ERR_INVALID_ARG     # counts inside a record buffer
    assert call(pp, ss, 3, smax=ss[2]) == SL_ERR_INVALID_ARG            # scale_max on a scale buffer
    assert call(pp, ss, 3, flags=pp[0]) == SL_ERR_INVALID_ARG           # flags on a record buffer
    assert fn(None, None, 2, 16, None, CNT, MX, None) == SL_ERR_INVALID_ARG


def test_peer_stats_interleaved_argument_checks(lib):
    """Every call here is rejected (or is a no-op) on the host, before any
    launch and before the scratch is allocated.  3 peers x 16 chunks: records
    3 x 16 x 112 bytes from R, scales 3 x 16 x 4 bytes from S."""
    f = lib.sl_peer_stats_interleaved
    R = P
    F, CNT, MX = A * 1200, A * 1300, A * 1400
    assert f(R, S, 3, -1, F, CNT, MX, None) == SL_ERR_SHAPE
    assert f(R, S, 3, 1 << 31, F, CNT, MX, None) == SL_ERR_SHAPE
    assert f(R, S, -1, 16, F, CNT, MX, None) == SL_ERR_TOO_MANY_PEERS
    assert f(R, S, 129, 16, F, CNT, MX, None) == SL_ERR_TOO_MANY_PEERS
    assert f(R, S, 0, 16, F, CNT, MX, None) == SL_OK                         # no-op
    assert f(R, S, 3, 16, F, None, MX, None) == SL_ERR_INVALID_ARG
    assert f(R, S, 3, 16, F, CNT, None, None) == SL_ERR_INVALID_ARG
    assert f(R, S, 3, 16, F, CNT + 4, MX, None) == SL_ERR_ALIGN
    assert f(R, S, 3, 16, F, CNT, MX + 2, None) == SL_ERR_ALIGN
    assert f(None, S, 3, 16, F, CNT, MX, None) == SL_ERR_INVALID_ARG
    assert f(R, None, 3, 16, F, CNT, MX, None) == SL_ERR_INVALID_ARG
    assert f(R + 8, S, 3, 16, F, CNT, MX, None) == SL_ERR_ALIGN
    assert f(R, S + 2, 3, 16, F, CNT, MX, None) == SL_ERR_ALIGN
    assert f(R, S, 3, 16, F, MX - 8, MX, None) == SL_ERR_INVALID_ARG         # counts (96 bytes) reach scale_max
    assert f(R, S, 3, 16, CNT - 8, CNT, MX, None) == SL_ERR_INVALID_ARG      # flags (48 bytes) reach counts
    assert f(R, S, 3, 16, R + 3 * 16 * 112 - 8, CNT, MX, None) == SL_ERR_INVALID_ARG   # flags reach into the records
    assert f(R, S, 3, 16, F, S + 16, MX, None) == SL_ERR_INVALID_ARG         # counts on the scales
    assert f(R, S, 3, 16, F, CNT, S + 3 * 16 * 4 - 4, None) == SL_ERR_INVALID_ARG   # scale_max on the last scale


def test_peerset_checks_once_and_rejects_bad_tensors():
    import communication_efficient_distributed_amd as sl
    with pytest.raises(ValueError):
        sl.PeerSet([torch.zeros((4, 112), dtype=torch.uint8)], [torch.zeros(4)])      # host tensors
    with pytest.raises(ValueError):
        sl.PeerSet([torch.zeros((4, 112), dtype=torch.uint8)], [])                     # lengths differ
    empty = sl.PeerSet([], [])
    assert len(empty) == 0 and empty.n_chunks == 0


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "sparseloco.h"

/* A plain C99 caller: argument errors come back before any device work. */
int main(void) {
    float* fake = (float*)(unsigned long)0x10000;        /* never dereferenced */
    uint8_t* fake8 = (uint8_t*)(unsigned long)0x20000;
    const uint8_t* pp[1] = {fake8};
    const float* sp[1] = {fake};
    int bad = 0;
    bad |= sl_compress(fake, fake, 0.95f, fake8, fake, 4095, NULL) != SL_ERR_SHAPE;
    bad |= sl_compress(NULL, fake, 0.95f, fake8, fake, 4096, NULL) != SL_ERR_INVALID_ARG;
    bad |= sl_compress(fake, fake, 0.95f, fake8 + 1, fake, 4096, NULL) != SL_ERR_ALIGN;
    bad |= sl_compress(fake, fake, 0.95f, fake8, fake, 0, NULL) != SL_OK;
    bad |= sl_aggregate(pp, sp, SL_MAX_PEERS + 1, fake, 4096, NULL) != SL_ERR_TOO_MANY_PEERS;
    bad |= sl_aggregate_apply(pp, sp, 0, fake, 4096, NULL) != SL_ERR_TOO_MANY_PEERS;
    bad |= sl_apply_mean(fake, fake, 1, 4096, NULL) != SL_ERR_INVALID_ARG;      /* theta aliases out */
    bad |= sl_validate_payloads(pp, sp, 1, -1, fake8, NULL) != SL_ERR_SHAPE;
    bad |= strncmp(sl_status_string(SL_ERR_ALIGN), "SL_ERR_ALIGN", 12) != 0;
    printf("%s %d\n", bad ? "FAIL" : "OK", SL_PAYLOAD_BYTES);
    return bad;
}
"""


def test_header_compiles_as_c99_and_links(lib, tmp_path):
    """include/sparseloco.h is a plain C header: a C99 program includes it with
    warnings as errors, links libsparseloco.so without torch or Python, and gets
    the documented status codes for bad arguments."""
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(lib._name)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                    os.path.join(ROOT, "include"), str(src), "-L", libdir, "-lsparseloco",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.split() == ["OK", "112"], (out.stdout, out.stderr)


def test_c_roundtrip_program_compiles(lib, tmp_path):
    """The C host program of the C-boundary GPU test (tests/c/sl_c_roundtrip.c)
    builds as C99 with warnings as errors against the header, the library and
    the HIP runtime; run without arguments it prints its usage and exits 1
    before touching the GPU."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("sl_c_build", os.path.join(ROOT, "tests", "c", "build.py"))
    c_build = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(c_build)
    exe = c_build.build_c_roundtrip(out=str(tmp_path / "sl_c_roundtrip"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr, (r.returncode, r.stderr)
