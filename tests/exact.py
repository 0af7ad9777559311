"""Exact-rational helpers for pinning the oracle without reusing its arithmetic.

The oracle works in binary32/binary64 hardware arithmetic; these helpers work
in Python's ``fractions.Fraction`` (exact rationals) and choose the float32
result by the round-to-nearest-even definition directly.
"""
from fractions import Fraction

import numpy as np

F32 = np.float32


def frac(x) -> Fraction:
    """Exact rational value of a finite float32/float64."""
    return Fraction(float(x))


def round_f32(q: Fraction) -> np.float32:
    """float32 nearest to q, ties to even (q finite, within range)."""
    approx = F32(float(q))                  # at most a couple of ulps away
    cands = [approx]
    lo = approx
    hi = approx
    for _ in range(3):
        lo = np.nextafter(lo, F32(-np.inf), dtype=np.float32)
        hi = np.nextafter(hi, F32(np.inf), dtype=np.float32)
        cands += [lo, hi]
    cands = [c for c in cands if np.isfinite(c)]

    def dist(c):
        return abs(frac(c) - q)

    best = min(dist(c) for c in cands)
    ties = [c for c in cands if dist(c) == best]
    if len(ties) == 1:
        return ties[0]
    even = [c for c in ties if (int(np.array(c, dtype=np.float32).view(np.uint32)) & 1) == 0]
    assert len(even) == 1
    return even[0]


def bits(x) -> int:
    return int(np.array(x, dtype=np.float32).view(np.uint32))


def from_bits(b: int) -> np.float32:
    return np.array(b, dtype=np.uint32).view(np.float32)[()]


def read_bits_lsb_first(stream: np.ndarray, pos: int, width: int) -> int:
    """Read an unsigned field from a little-endian LSB-first byte stream, one
    bit at a time (independent of the oracle's reader)."""
    bitsarr = np.unpackbits(np.asarray(stream, dtype=np.uint8), bitorder="little")
    v = 0
    for b in range(width):
        v |= int(bitsarr[pos + b]) << b
    return v


def unpack_payload_bitwise(payload: np.ndarray):
    """Decode one 112-byte payload: 64 12-bit indices then 64 2-bit codes."""
    bitsarr = np.unpackbits(np.asarray(payload, dtype=np.uint8), bitorder="little")
    w_idx = 1 << np.arange(12)
    w_code = 1 << np.arange(2)
    idx = (bitsarr[: 64 * 12].reshape(64, 12) * w_idx).sum(1)
    code = (bitsarr[96 * 8: 96 * 8 + 128].reshape(64, 2) * w_code).sum(1)
    return idx.astype(np.int64), code.astype(np.int64)
