"""Pins of the oracle on the hand-derived special chunks E1..E4
(tests/golden/special_chunks.txt), plus the closed-form index-byte pattern of a
chunk whose kept indices are 0..63."""
import numpy as np
import pytest

import special_chunks as sc
from exact import unpack_payload_bitwise

GOLD = sc.load_golden()


@pytest.mark.parametrize("case", ["E1", "E2", "E3", "E4"])
def test_special_chunk_bytes(orc, case):
    d, e = sc.inputs(case)
    payload, scales, ef = orc.compress(d, e, beta=0.95)
    p = payload[0]
    for field, want in GOLD[case].items():
        if field == "scale":
            assert int(scales.view(np.uint32)[0]) == want
        else:
            a, b = sc.byte_range(field)
            assert p[a:b].tobytes() == want, (case, field, p[a:b].tobytes().hex())


@pytest.mark.parametrize("case", ["E1", "E2", "E3", "E4"])
def test_special_chunk_residual_and_indices(orc, case):
    d, e = sc.inputs(case)
    payload, scales, ef = orc.compress(d, e, beta=0.95)
    want = sc.expected_new_ef(case)
    assert np.array_equal(ef.view(np.uint32), want.view(np.uint32))
    idx, code = unpack_payload_bitwise(payload[0])
    assert np.array_equal(idx, sc.expected_kept(case))


def test_ascending_pair_closed_form(orc):
    """Kept indices 0..63 (all-zero chunk): pair (2m, 2m+1) packs to bytes
    [2m, ((2m+1) & 15) << 4, (2m+1) >> 4]."""
    d = np.zeros(4096, np.float32)
    payload, _, _ = orc.compress(d, np.zeros_like(d))
    want = []
    for m in range(32):
        a, b = 2 * m, 2 * m + 1
        want += [a & 0xFF, ((a >> 8) & 0xF) | ((b & 0xF) << 4), b >> 4]
    assert payload[0, :96].tolist() == want
    assert payload[0, 96:].tolist() == [0] * 16


def test_e1_ef_untouched_bitwise(orc):
    d, e = sc.inputs("E1")
    _, _, ef = orc.compress(d, e)
    assert np.array_equal(ef.view(np.uint32), np.zeros(4096, np.uint32))


def test_e4_negative_zero_residual(orc):
    """Kept -0.0 has code 2 and decodes to -s/3 = -1, so its residual is
    -0 - (-1) = +1 exactly."""
    d, e = sc.inputs("E4")
    payload, _, ef = orc.compress(d, e)
    idx, code = unpack_payload_bitwise(payload[0])
    assert code[3] == 2 and ef[3] == 1.0
