"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle.cpp is built a second time with -fsanitize=address,undefined and
-fno-sanitize-recover=all (g++, CPU only), and the oracle's pin files run
against that build through ORACLE_LIB, with the ASan runtime preloaded into
the child Python process.  Any out-of-bounds access, use after free, signed
overflow, invalid shift or misaligned access in the oracle then aborts the run.

Two controls show the sanitizers are live in this route: a planted one-past-
the-end read of the per-chunk accumulator and a planted over-wide shift in the
bit-stream reader must each abort the pin run with the sanitizer's report.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")
PIN_FILES = ["test_oracle_golden.py", "test_oracle_pages.py", "test_oracle_aggregate.py",
             "test_oracle_invariants.py", "test_oracle_exhaustive.py"]

FLAGS = ["-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off", "-fno-fast-math",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _libasan():
    if shutil.which("g++") is None:
        return None
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


LIBASAN = _libasan()
pytestmark = pytest.mark.skipif(LIBASAN is None, reason="g++ with the AddressSanitizer runtime is not available")


def build(text: str, tmp_path, name: str) -> str:
    cpp = tmp_path / f"{name}.cpp"
    cpp.write_text(text)
    so = str(tmp_path / f"{name}.so")
    subprocess.run(["g++", *FLAGS, "-I", os.path.join(ROOT, "oracle"), "-o", so, str(cpp)], check=True,
                   capture_output=True)
    return so


def run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_LIB=lib, LD_PRELOAD=LIBASAN,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    files = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                           *files], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def plant(old: str, new: str) -> str:
    src = open(SRC).read()
    assert src.count(old) == 1, f"plant site not unique or missing: {old!r}"
    return src.replace(old, new)


def test_pins_pass_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    r = run_pins(build(open(SRC).read(), tmp_path, "sanitized"))
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout


def test_planted_out_of_bounds_read_is_reported(tmp_path):
    text = plant("float s = std::fabs(acc[order[0]]);",
                 "float s = std::fabs(acc[order[0]]) + 0.0f * acc.data()[chunk];")
    r = run_pins(build(text, tmp_path, "oob"))
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]


def test_planted_invalid_shift_is_reported(tmp_path):
    text = plant("if ((stream[p / 8] >> (p % 8)) & 1u) v |= 1u << b;",
                 "if ((stream[p / 8] >> (p % 8)) & 1u) v |= 1u << (b + 32 * (w > 11));")
    r = run_pins(build(text, tmp_path, "shift"))
    assert r.returncode != 0
    assert "runtime error" in r.stderr and "shift" in r.stderr, r.stderr[-3000:]
