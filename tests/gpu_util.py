"""Shared helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import os
import sys

import numpy as np
import pytest
import torch


def note(msg: str):
    """Name the case before a GPU step, so a failing run says what it ran."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import communication_efficient_distributed_amd as sl
    sl.load()          # raises if the HIP library is not built: no fallback
    return sl


def oracle_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def assert_bitwise(a: np.ndarray, b: np.ndarray, what: str):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        av, bv = a.view(np.uint32), b.view(np.uint32)
    else:
        av, bv = a, b
    bad = np.nonzero(av.reshape(-1) != bv.reshape(-1))[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} mismatches, first at flat {i}: "
                             f"gpu={a.reshape(-1)[i]!r} oracle={b.reshape(-1)[i]!r}")


def assert_rel(gpu: np.ndarray, ref: np.ndarray, what: str, rel: float = 1e-6):
    """|g - r| <= rel * |r| elementwise (so r == 0 needs g == 0)."""
    g = gpu.astype(np.float64).reshape(-1)
    r = ref.astype(np.float64).reshape(-1)
    bad = np.nonzero(np.abs(g - r) > rel * np.abs(r))[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} outside {rel} rel, first at {i}: "
                             f"gpu={g[i]!r} oracle={r[i]!r}")
