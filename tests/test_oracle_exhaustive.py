"""Brute-force pins of the oracle's selection, quantiser and residual on tiny
chunks, over every input drawn from a small value set.

Chunk selection is checked against an independent brute force (numpy argsort of
a unique integer score), the magnitude bit against exact integer arithmetic,
and the one-third level against exact-rational rounding.
"""
from fractions import Fraction

import numpy as np
import pytest

from exact import round_f32


def all_inputs(values, chunk):
    vals = np.array(values, dtype=np.float32)
    r = len(vals)
    code = np.arange(r ** chunk, dtype=np.int64)
    digits = (code[:, None] // (r ** np.arange(chunk, dtype=np.int64))[None, :]) % r
    return vals[digits]                        # [r**chunk, chunk], every input once


def brute_force_expectations(acc, k):
    """Expected (idx, code, scale, ef) from the definitions, per chunk."""
    n_in, chunk = acc.shape
    b = acc.view(np.uint32)
    key = (b & 0x7FFFFFFF).astype(np.int64)
    sign = (b >> 31).astype(np.int64)
    # unique score: larger key first, then lower index first
    score = key * chunk + (chunk - 1 - np.arange(chunk))[None, :]
    top = np.argsort(-score, axis=1, kind="stable")[:, :k]
    idx = np.sort(top, axis=1)
    s = np.abs(acc).max(axis=1)                 # max |acc|
    kept_vals = np.take_along_axis(acc, idx, axis=1)
    kept_abs = np.abs(kept_vals)
    # values are small integers: 3|v| > 2s is exact in float64 integer math
    mag = (3 * kept_abs.astype(np.int64) > 2 * s.astype(np.int64)[:, None]).astype(np.int64)
    kept_sign = np.take_along_axis(sign, idx, axis=1)
    code = (kept_sign << 1) | mag
    thirds = {float(v): round_f32(Fraction(float(v)) / 3) for v in np.unique(s)}
    s3 = np.array([thirds[float(v)] for v in s], dtype=np.float32)
    dec_abs = np.where(mag == 1, s[:, None], s3[:, None]).astype(np.float32)
    dec = np.where(kept_sign == 1, -dec_abs, dec_abs).astype(np.float32)
    ef = acc.copy()
    resid = (kept_vals - dec).astype(np.float32)
    np.put_along_axis(ef, idx, resid, axis=1)
    return idx, code, s, ef


@pytest.mark.parametrize("values,chunk,k", [
    # {+0, -0, +-1, +-2}: 6^8 = 1,679,616 chunks of 8, top-2
    ([0.0, -0.0, 1.0, -1.0, 2.0, -2.0], 8, 2),
    # {0, +-1, +-2, +-3}: 7^6 chunks of 6, top-3; puts |v| = 2 exactly on the
    # 2s/3 threshold when s = 3
    ([0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0], 6, 3),
])
def test_exhaustive_small_chunks(orc, values, chunk, k):
    delta = all_inputs(values, chunk)
    # ef carries the sign of a zero delta so that acc = fma(beta, ef, delta)
    # keeps -0.0 (fma(b, +0, -0) would give +0).
    ef0 = np.where(np.signbit(delta), np.float32(-0.0), np.float32(0.0)).astype(np.float32)
    acc = delta.copy()                          # beta * (+-0) + delta = delta exactly
    idx, code, scale, ef = orc.compress_unpacked(delta.reshape(-1), ef0.reshape(-1),
                                                 chunk, k, 0.95)
    e_idx, e_code, e_s, e_ef = brute_force_expectations(acc, k)
    assert np.array_equal(idx, e_idx)
    assert np.array_equal(code.astype(np.int64), e_code)
    assert np.array_equal(scale.view(np.uint32), e_s.view(np.uint32))
    assert np.array_equal(ef.reshape(acc.shape).view(np.uint32), e_ef.view(np.uint32))


def test_every_kept_beats_every_dropped(orc):
    """Property form of the selection on random chunks with heavy ties:
    for kept i and dropped j, key_i > key_j, or key_i == key_j and i < j."""
    rng = np.random.default_rng(7)
    chunk, k = 64, 16
    vals = rng.integers(-4, 5, size=(2000, chunk)).astype(np.float32)
    idx, code, scale, _ = orc.compress_unpacked(vals.reshape(-1), np.zeros(vals.size, np.float32),
                                                chunk, k, 1.0)
    key = vals.view(np.uint32) & 0x7FFFFFFF
    for c in range(vals.shape[0]):
        kept = np.zeros(chunk, bool)
        kept[idx[c]] = True
        assert np.all(np.diff(idx[c]) > 0)
        ki = key[c][kept]
        ii = np.nonzero(kept)[0]
        kj = key[c][~kept]
        jj = np.nonzero(~kept)[0]
        beats = (ki[:, None] > kj[None, :]) | ((ki[:, None] == kj[None, :]) & (ii[:, None] < jj[None, :]))
        assert beats.all()
