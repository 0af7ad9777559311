"""The boundary driven from C: tests/c/sl_c_roundtrip (built by
__graft_entry__.build()) is a plain C99 program that links libsparseloco.so and
the HIP runtime, with no Python or torch in its process.  It runs two rounds of
sl_compress from ef = 0, sl_aggregate over the two rounds' records and
sl_apply_mean on theta; every output is compared with the oracle bit for bit."""
import os
import subprocess

import numpy as np
import pytest

from communication_efficient_distributed_amd import datagen
from gpu_util import assert_bitwise, note

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "sl_c_roundtrip")


def test_c_program_round_trip(orc, tmp_path):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built: run __graft_entry__.build() first")
    C = 37
    n = C * 4096
    beta = np.float32(0.95)
    delta = datagen.lognormal(n, datagen.SMALL_1M, 9, 0).numpy()
    theta = datagen.theta0(n, datagen.SMALL_1M).numpy()
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    src.write_bytes(np.int64(n).tobytes() + beta.tobytes() + delta.tobytes() + theta.tobytes())
    note(f"C program: sl_compress x2, sl_aggregate (2 peers), sl_apply_mean, chunks={C}")
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.split() == ["OK", str(n)]
    raw = dst.read_bytes()
    pb, sb, db = C * 112, C * 4, n * 4
    assert len(raw) == 2 * (pb + sb) + 3 * db
    off = 0

    def take(nbytes, dtype):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=nbytes // np.dtype(dtype).itemsize, offset=off)
        off += nbytes
        return a

    p1, s1 = take(pb, np.uint8).reshape(C, 112), take(sb, np.float32)
    p2, s2 = take(pb, np.uint8).reshape(C, 112), take(sb, np.float32)
    ef, out, th = take(db, np.float32), take(db, np.float32), take(db, np.float32)
    op1, os1, ef1 = orc.compress(delta, np.zeros(n, np.float32), beta=float(beta))
    op2, os2, ef2 = orc.compress(delta, ef1, beta=float(beta))
    assert_bitwise(p1, op1, "round 1 records")
    assert_bitwise(s1, os1, "round 1 scales")
    assert_bitwise(p2, op2, "round 2 records")
    assert_bitwise(s2, os2, "round 2 scales")
    assert_bitwise(ef, ef2, "error feedback after two rounds")
    o = orc.aggregate([op1, op2], [os1, os2], n)
    assert_bitwise(out, o, "sum of the two rounds' records")
    assert_bitwise(th, orc.apply_mean(theta, o, 2), "theta - sum / 2")
