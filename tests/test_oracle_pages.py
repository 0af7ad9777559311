"""Pins of the oracle against figures the pages print (tests/golden/pages_figures.txt).

The oracle's own outputs (payload stride, entries per chunk, bit widths) are
measured here and compared with the printed figures; nothing is taken from the
oracle's source constants.
"""
import ctypes
import os

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def load_figures():
    figs = {}
    with open(os.path.join(HERE, "golden", "pages_figures.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (t.strip() for t in line.split("="))
            figs[k] = float(v) if "." in v else int(v)
    return figs


FIG = load_figures()


def _raw_compress_into(orc, delta, guard_bytes=512):
    """Call orc_compress with an oversized payload buffer prefilled with 0xA5, so
    the bytes the oracle writes per chunk can be measured."""
    n = delta.size
    C = n // FIG["chunk_params"]
    buf = np.full(C * 200 + guard_bytes, 0xA5, dtype=np.uint8)
    scales = np.zeros(C, dtype=np.float32)
    ef = np.zeros(n, dtype=np.float32)
    rc = orc.lib().orc_compress(ctypes.c_void_p(delta.ctypes.data),
                                ctypes.c_void_p(ef.ctypes.data), n, ctypes.c_float(0.95),
                                ctypes.c_void_p(buf.ctypes.data),
                                ctypes.c_void_p(scales.ctypes.data), 1)
    assert rc == 0
    return buf, scales


def test_payload_size_and_ratio(orc):
    """[SF] layout formula: 64 entries of (2 + 12) bits make 896 bits, 112 bytes per chunk; the
    ratio 16,384 / 112 = 146.3x.  Measured from where the oracle stops writing."""
    rng = np.random.default_rng(1)
    C = 8
    delta = rng.standard_normal(C * FIG["chunk_params"]).astype(np.float32)
    buf, _ = _raw_compress_into(orc, delta)
    # The oracle writes a contiguous prefix; everything after it keeps the fill.
    # Random data makes a 0xA5 byte inside a payload unlikely but possible, so
    # measure with two different fills.
    written = None
    for fill in (0xA5, 0x5A):
        b2 = np.full_like(buf, fill)
        ef = np.zeros_like(delta)
        sc = np.zeros(C, np.float32)
        orc.lib().orc_compress(ctypes.c_void_p(delta.ctypes.data),
                               ctypes.c_void_p(ef.ctypes.data), delta.size,
                               ctypes.c_float(0.95), ctypes.c_void_p(b2.ctypes.data),
                               ctypes.c_void_p(sc.ctypes.data), 1)
        changed = np.nonzero(b2 != fill)[0]
        last = int(changed.max()) + 1
        written = last if written is None else max(written, last)
    per_chunk = written / C
    assert per_chunk == FIG["payload_bytes"]
    assert per_chunk * 8 == FIG["payload_bits"]
    assert FIG["topk"] * FIG["bits_per_entry"] == FIG["payload_bits"]
    assert FIG["value_bits"] + FIG["index_bits"] == FIG["bits_per_entry"]
    dense = FIG["chunk_params"] * 4
    assert dense == FIG["dense_chunk_bytes"] and dense * 8 == FIG["dense_chunk_bits"]
    assert round(dense / per_chunk, 1) == FIG["compression_ratio"]


def test_entries_per_chunk_and_density(orc):
    """[SF] lever 1: top-64 of 4,096 = 1.5625% density; 98.44% dropped."""
    rng = np.random.default_rng(2)
    delta = rng.standard_normal(4 * 4096).astype(np.float32)
    idx, code, scale, _ = orc.compress_unpacked(delta, np.zeros_like(delta), 4096, 64, 0.95)
    for c in range(4):
        kept = np.unique(idx[c])
        assert kept.size == FIG["topk"]
    density = 100.0 * idx.shape[1] / 4096
    assert density == FIG["density_percent"]
    assert round(density, 2) == FIG["density_percent_short"]
    assert round(100.0 - density, 2) == FIG["dropped_percent"]


def test_index_field_width_covers_chunk(orc):
    """[SF] lever 3: 12 bits = ceil(log2 4096).  Index 4095 (all twelve bits set)
    must survive a pack/unpack round trip, and the packed stream for index j
    starts at bit 12j."""
    assert int(np.ceil(np.log2(FIG["chunk_params"]))) == FIG["index_bits"]
    idx = np.arange(4096 - 64, 4096, dtype=np.int32).reshape(1, 64)
    code = np.zeros((1, 64), np.uint8)
    p = orc.pack(idx, code)
    i2, _ = orc.unpack(p)
    assert (i2 == idx).all()
    # bits 12*63 .. 12*64-1 hold 4095: the last 12 bits of the 96-byte region
    bitsarr = np.unpackbits(p[0, :96], bitorder="little")
    assert bitsarr[12 * 63: 12 * 64].all()


def test_model_level_figures():
    """[SF] ~2 GB per peer per sync, ~13 Mbps over 1,200 s, 290.8 GB dense,
    1.9 Gbps; [SA] 72,747,327,488 params; [CV] 94.5% utilisation."""
    P = FIG["model_params"]
    chunks, rem = divmod(P, FIG["chunk_params"])
    assert rem == 0 and chunks == 17_760_578
    payload = chunks * FIG["payload_bytes"]
    assert payload == 1_989_184_736
    assert round(payload / 1e9) == FIG["per_peer_sync_gb"]
    assert round(P * 4 / 1e9) == FIG["dense_sync_gb"]
    assert round(FIG["model_params_billions"] * 4, 1) == FIG["dense_sync_gb_exact"]
    assert round(payload * 8 / FIG["window_seconds"] / 1e6) == FIG["uplink_mbps_computed"]
    rate = FIG["dense_sync_gb_exact"] * 1e9 / FIG["window_seconds"]
    assert round(rate / 1e6) == FIG["dense_rate_mb_s"]
    assert round(rate * 8 / 1e9, 1) == FIG["dense_rate_gbps"]
    w = FIG["compute_minutes"] * 60
    assert round(100 * w / (w + FIG["comm_seconds"]), 1) == FIG["utilisation_percent"]
