"""Builders for the hand-derived special chunks in tests/golden/special_chunks.txt
(inputs only; the expected bytes live in the fixture)."""
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def inputs(case):
    """(delta, ef) float32[4096] for special chunk E1..E4 (beta irrelevant:
    ef is +-0, so acc = delta)."""
    d = np.zeros(4096, np.float32)
    e = np.zeros(4096, np.float32)
    if case == "E1":
        pass
    elif case == "E2":
        d[4095] = 1.5
    elif case == "E3":
        d[10:1001:10] = -1.0
    elif case == "E4":
        d[0] = 3.0
        d[1] = 2.0
        d[2] = np.nextafter(np.float32(2.0), np.float32(3.0))
        d[3] = -0.0
        e[3] = -0.0            # fma(beta, -0, -0) = -0 keeps the negative zero
    else:
        raise KeyError(case)
    return d, e


def load_golden():
    """{case: {field: bytes-or-int}} from the fixture."""
    out = {}
    with open(os.path.join(HERE, "golden", "special_chunks.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            case, field, *vals = line.split()
            if field == "scale":
                out.setdefault(case, {})[field] = int(vals[0], 16)
            else:
                out.setdefault(case, {})[field] = bytes(int(v, 16) for v in vals)
    return out


def byte_range(field):
    """'bytes[a,b]' -> (a, b+1)."""
    a, b = field[len("bytes["):-1].split(",")
    return int(a), int(b) + 1


def expected_new_ef(case):
    """Hand-derived residual after one round (see the fixture comments)."""
    d, _ = inputs(case)
    ef = d.copy()
    if case == "E1":
        pass
    elif case == "E2":
        ef[0:63] = -0.5
        ef[4095] = 0.0
    elif case == "E3":
        ef[10:641:10] = 0.0
    elif case == "E4":
        ef[0] = 0.0
        ef[1] = 1.0
        ef[2] = np.float32(-1.0 + 2.0 ** -22)
        ef[3] = 1.0
        ef[4:64] = -1.0
    return ef


def expected_kept(case):
    if case in ("E1", "E4"):
        return np.arange(64)
    if case == "E2":
        return np.r_[np.arange(63), 4095]
    if case == "E3":
        return np.arange(10, 641, 10)
    raise KeyError(case)
