"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a temporary copy of oracle/oracle.cpp (on the
CPU; the file itself is untouched), builds it, and runs the oracle's pin tests
against the planted build.  Every plant must make at least one pin fail: that
shows the pins are tied to the pages and to mathematics, not to the oracle's own
code.  Mistakes are chosen where a reading of the pages could plausibly go
wrong: tie rule, threshold strictness, rounding of s/3 and of the error-feedback
update, entry order, code-bit and bit-stream layout, sign of zero, the scale,
the residual, the peer order, the outer update, the validator and the per-peer statistics.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")

# Fastest pin files first: a planted build stops at its first failing pin.
PIN_FILES = ["test_oracle_golden.py", "test_oracle_pages.py", "test_oracle_aggregate.py",
             "test_oracle_invariants.py", "test_oracle_exhaustive.py"]

# (name, [(text in oracle.cpp, planted replacement), ...])
MUTANTS = [
    ("tie: higher index wins", [("        return a < b;\n", "        return a > b;\n")]),
    ("ranking key keeps the sign bit",
     [("return bits_of(v) & 0x7fffffffu; }", "return bits_of(v); }")]),
    ("threshold not strict", [("> two_s) ? 1u : 0u", ">= two_s) ? 1u : 0u")]),
    ("s/3 by a rounded reciprocal", [("return s / 3.0f; }", "return s * (1.0f / 3.0f); }")]),
    ("ef update rounded twice",
     [("std::fma(beta, ef[i], delta[i])", "beta * ef[i] + delta[i]")]),
    ("beta ignored", [("std::fma(beta, ef[i], delta[i])", "ef[i] + delta[i]")]),
    ("entries left in rank order",
     [("    std::sort(kept.begin(), kept.end());                   /* R4 */", "")]),
    ("code bits swapped (consistently)",
     [("(uint8_t)((sign << 1) | mag)", "(uint8_t)((mag << 1) | sign)"),
      ("float mag = (code & 1u) ? s : third_of(s);", "float mag = (code & 2u) ? s : third_of(s);"),
      ("return (code & 2u) ? -mag : mag;", "return (code & 1u) ? -mag : mag;")]),
    ("sign from v < 0 (so -0 is positive)",
     [("uint32_t sign_bit(float v) { return bits_of(v) >> 31; }",
       "uint32_t sign_bit(float v) { return v < 0.0f ? 1u : 0u; }")]),
    ("scale from the lowest kept index",
     [("float s = std::fabs(acc[order[0]]);", "float s = std::fabs(acc[kept[0]]);")]),
    ("bit streams MSB-first within a byte",
     [("stream[p / 8] |= (uint8_t)(1u << (p % 8));", "stream[p / 8] |= (uint8_t)(1u << (7 - p % 8));"),
      ("if ((stream[p / 8] >> (p % 8)) & 1u) v |= 1u << b;",
       "if ((stream[p / 8] >> (7 - p % 8)) & 1u) v |= 1u << b;")]),
    ("residual sign flipped",
     [("acc[i] = acc[i] - decode_value(code, s);", "acc[i] = acc[i] + decode_value(code, s);")]),
    ("residual zeroed where sent",
     [("acc[i] = acc[i] - decode_value(code, s);", "acc[i] = 0.0f;")]),
    ("peers summed in descending order",
     [("for (int32_t p = 0; p < n_peers; ++p) {", "for (int32_t p = n_peers - 1; p >= 0; --p) {")]),
    ("sum starts from -0", [("o[i] = +0.0f;", "o[i] = -0.0f;")]),
    ("apply by a rounded reciprocal",
     [("theta[i] - out[i] / denom;", "theta[i] - out[i] * (1.0f / denom);")]),
    ("validator accepts repeated indices",
     [("if (!(idx[j] > idx[j - 1])) f |= 1;", "if (!(idx[j] >= idx[j - 1])) f |= 1;")]),
    ("statistics count the sign bit as magnitude",
     [("if (code[j] & 1u) ++magnitude;", "if (code[j] & 2u) ++magnitude;")]),
    ("statistics take the maximum over every scale",
     [("if ((f & 6u) == 0 && s > top) top = s;", "if (s > top) top = s;")]),
    ("statistics skip the code counts of flagged records",
     [("        unpack_one(payload + c * kPayloadBytes, idx, code);\n        for (int32_t j = 0; j < kTopK; ++j) {",
       "        unpack_one(payload + c * kPayloadBytes, idx, code);\n        if (f) continue;\n        for (int32_t j = 0; j < kTopK; ++j) {")]),
    ("pseudo-gradient sign flipped",
     [("delta[i] = theta_pre[i] - theta_post[i];", "delta[i] = theta_post[i] - theta_pre[i];")]),
]


def plant(src: str, edits) -> str:
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
        src = src.replace(old, new)
    return src


def build(path_cpp: str, path_so: str):
    cmd = ["g++", "-O2", "-std=c++17", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
           "-fno-fast-math", "-I", os.path.join(ROOT, "oracle"), "-o", path_so, path_cpp]
    subprocess.run(cmd, check=True, capture_output=True)


def run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, ORACLE_LIB=lib)
    files = [os.path.join(ROOT, "tests", f) for f in PIN_FILES]
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                           "-m", "not gpu", *files], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def test_mutation_sites_exist():
    src = open(SRC).read()
    for name, edits in MUTANTS:
        plant(src, edits)


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(SRC).read()
    libs = []
    for k, (name, edits) in enumerate(MUTANTS):
        cpp = tmp_path / f"m{k}.cpp"
        cpp.write_text(plant(src, edits))
        libs.append(str(tmp_path / f"m{k}.so"))
        build(str(cpp), libs[-1])
    with ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(run_pins, libs))
    survivors = [name for (name, _), r in zip(MUTANTS, results) if r.returncode == 0]
    for (name, _), r in zip(MUTANTS, results):
        assert r.returncode in (0, 1), f"{name}: pin run crashed\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}"
    assert not survivors, f"planted mistakes no pin caught: {survivors}"


def test_unplanted_copy_passes_the_pins(tmp_path):
    """Control: the same build route with nothing planted passes every pin."""
    cpp = tmp_path / "same.cpp"
    cpp.write_text(open(SRC).read())
    so = str(tmp_path / "same.so")
    build(str(cpp), so)
    r = run_pins(so)
    assert r.returncode == 0, r.stdout[-3000:]
