"""The s/3 level for every non-negative finite fp32 scale, on the GPU, in both
kernels that form it.

"The Sparse Frontier", section "SparseLoCo: Three Compression Levers in One
Pass", lever 2: four levels per chunk around one scale s.  Reading: the inner
levels are +-fl(s/3) with fl correctly rounded (IEEE binary32 division, round
to nearest even, denormals kept).  A division that is only nearly correct
(a reciprocal, a flushed denormal) differs from it for some s, so every one of
the 0x7F800000 scales is checked:

- compress: a chunk [s, 0, ..., 0] with beta = 0 keeps s (magnitude level)
  and 63 zeros (lower index wins the tie), each zero at the +s/3 level, so
  its residual is fl(0 - fl(s/3)); the scale must be s and the record the one
  the oracle writes for such a chunk;
- aggregate: one peer whose records keep indices 0..63 at the +s/3 level
  gives out = fl(+0 + fl(s/3)) there and +0 elsewhere.

Expected values are IEEE binary32 divisions on the host (numpy), the record
bytes come from the oracle; the oracle's own s/3 is pinned against exact
rationals in the CPU tests.
"""
import numpy as np
import pytest
import torch

from gpu_util import note, require_gpu

CHUNK = 4096
N_SCALES = 0x7F800000          # bit patterns 0 .. 0x7F7FFFFF: +0 up to FLT_MAX
BATCH = 1 << 20                # chunks per call; N_SCALES is a whole number of batches
assert N_SCALES % BATCH == 0


def expected_third(start: int) -> np.ndarray:
    s = np.arange(start, start + BATCH, dtype=np.uint32).view(np.float32)
    return s / np.float32(3.0)


def check_columns(block: torch.Tensor, want: np.ndarray, start: int, what: str):
    """Every column of block [BATCH, k] equals want [BATCH] bit for bit."""
    w = torch.from_numpy(want.view(np.int32)).to(block.device)
    bad = block.view(torch.int32) != w[:, None]
    if bool(bad.any()):
        row = int(torch.nonzero(bad.any(dim=1))[0, 0])
        got = block[row].cpu().numpy()
        raise AssertionError(f"{what}: first bad s bits 0x{start + row:08x}: gpu row {got[:4]!r}... "
                             f"expected {want[row]!r}")


def check_zero(block: torch.Tensor, start: int, what: str):
    """block holds only +0.0."""
    assert not bool(block.view(torch.int32).any()), f"{what} must be +0, batch at 0x{start:08x}"


@pytest.mark.gpu
def test_compress_inner_level_for_every_scale(orc):
    sl = require_gpu()
    dev = torch.device("cuda:0")
    n = BATCH * CHUNK
    delta = torch.zeros(n, device=dev)
    ef = torch.zeros(n, device=dev)
    payload = torch.empty((BATCH, 112), dtype=torch.uint8, device=dev)
    scales = torch.empty(BATCH, device=dev)
    dv, ev = delta.view(BATCH, CHUNK), ef.view(BATCH, CHUNK)

    one = np.zeros(CHUNK, np.float32)
    one[0] = 1.0
    rec_pos = orc.compress(one, np.zeros(CHUNK, np.float32), beta=0.0)[0][0]
    rec_zero = orc.compress(np.zeros(CHUNK, np.float32), np.zeros(CHUNK, np.float32), beta=0.0)[0][0]
    want_rec = torch.from_numpy(np.tile(rec_pos, (BATCH, 1))).to(dev)

    for start in range(0, N_SCALES, BATCH):
        if start % (256 * BATCH) == 0:
            note(f"compress, scales 0x{start:08x}.. ({BATCH} chunks per call)")
        bits = torch.arange(start, start + BATCH, dtype=torch.int32, device=dev)
        dv[:, 0] = bits.view(torch.float32)
        # beta = 0: the previous batch's residuals in ef do not enter acc.
        sl.sl_compress(delta, ef, 0.0, payload, scales)
        assert torch.equal(scales.view(torch.int32), bits), f"scales, batch at 0x{start:08x}"
        if start == 0:
            want_rec[0] = torch.from_numpy(rec_zero).to(dev)
        assert torch.equal(payload, want_rec), f"records, batch at 0x{start:08x}"
        if start == 0:
            want_rec[0] = torch.from_numpy(rec_pos).to(dev)
        check_columns(ev[:, 1:64], np.float32(0.0) - expected_third(start), start, "ef at the kept zeros")
        check_zero(ev[:, :1], start, "ef at the kept maximum")
        check_zero(ev[:, 64:], start, "ef outside the kept set")


@pytest.mark.gpu
def test_aggregate_inner_level_for_every_scale(orc):
    sl = require_gpu()
    dev = torch.device("cuda:0")
    rec = orc.pack(np.arange(64, dtype=np.int32), np.zeros(64, np.uint8))[0]
    payload = torch.from_numpy(np.tile(rec, (BATCH, 1))).to(dev)
    out = torch.empty(BATCH * CHUNK, device=dev)
    ov = out.view(BATCH, CHUNK)

    for start in range(0, N_SCALES, BATCH):
        if start % (256 * BATCH) == 0:
            note(f"aggregate, scales 0x{start:08x}.. ({BATCH} chunks per call)")
        scales = torch.arange(start, start + BATCH, dtype=torch.int32, device=dev).view(torch.float32)
        sl.sl_aggregate([payload], [scales], out)
        check_columns(ov[:, :64], np.float32(0.0) + expected_third(start), start, "out at the kept indices")
        check_zero(ov[:, 64:], start, "out outside the record")
