"""Seeded synthetic pseudo-gradients shaped like the Covenant-72B layers.

This module holds distributions only: it draws random numbers and lays them out.
It contains none of the compressor's or aggregator's arithmetic, so the HIP path
and the CPU oracle can both consume what it produces.

Model shape (setupai.cc page "Covenant-72B: Largest Decentralized GPU Model",
Technical Deep Dive): width 8192, 64 query heads and 8 KV heads (head dim 128),
so Q/O are 8192x8192, K/V 8192x1024 and the MLP matrices 8192x28672.  The pages
publish no pseudo-gradient statistics; the distributions below are synthetic
stand-ins:

* ``lognormal``: z ~ N(0,1) times a per-1024-element group factor exp(N(0,1))
  (drawn once per (workload, peer) and held across rounds), times 20 for a
  Bernoulli(0.001) set of outlier entries drawn fresh each round.
* ``student_t3``: Student-t with 3 degrees of freedom, z / sqrt(chi2_3 / 3), and
  20% of the 4096-element chunks exactly zero (the same seeded set of chunks
  every round, a different set per peer).

Seeds: ``(workload << 32) | (peer << 16) | round``; peer 0 is the local
stream, aggregator peers are 1..N.  Group factors and the zero-chunk set use
round 0xFFFF.
"""
from __future__ import annotations

import math

import numpy as np
import torch

CHUNK = 4096          # parameters per chunk (input layout only)
GROUP = 1024          # elements per lognormal group
HELD = 0xFFFF         # "round" slot of per-peer quantities held across rounds

# Workload ids used in seeds.
SMALL_1M = 1          # 1,048,576 params, lognormal
ATTN_8192 = 2         # 8192 x 8192, lognormal
MLP_8192x28672 = 3    # 8192 x 28672, Student-t(3) with 20% zero chunks
DECODER_BLOCK = 4     # one decoder block, concatenated, lognormal
FLAT_16B = 5          # 16e9 flat span, lognormal

D_MODEL = 8192
D_KV = 1024
D_FF = 28672

# One decoder block, concatenation order Q, K, V, O, gate, up, down.
BLOCK_SHAPES = [
    ("q", (D_MODEL, D_MODEL)),
    ("k", (D_MODEL, D_KV)),
    ("v", (D_MODEL, D_KV)),
    ("o", (D_MODEL, D_MODEL)),
    ("gate", (D_MODEL, D_FF)),
    ("up", (D_MODEL, D_FF)),
    ("down", (D_MODEL, D_FF)),
]

WORKLOAD_PARAMS = {
    SMALL_1M: 1 << 20,
    ATTN_8192: D_MODEL * D_MODEL,
    MLP_8192x28672: D_MODEL * D_FF,
    DECODER_BLOCK: sum(a * b for _, (a, b) in BLOCK_SHAPES),
    FLAT_16B: 16_000_000_000,
}


def seed_of(workload: int, peer: int, rnd: int) -> int:
    return (int(workload) << 32) | ((int(peer) & 0xFFFF) << 16) | (int(rnd) & 0xFFFF)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def group_factors(n: int, workload: int, peer: int, device="cpu") -> torch.Tensor:
    """exp(N(0,1)) per contiguous 1024-element group, held across rounds."""
    n_groups = (n + GROUP - 1) // GROUP
    g = _gen(seed_of(workload, peer, HELD), device)
    return torch.randn(n_groups, generator=g, device=device, dtype=torch.float32).exp_()


def fill_lognormal_(out: torch.Tensor, workload: int, peer: int, rnd: int,
                    factors: torch.Tensor | None = None,
                    slice_elems: int = 1 << 28) -> torch.Tensor:
    """Fill a flat float32 tensor in place, slice by slice (bounded temporaries)."""
    assert out.dtype == torch.float32 and out.dim() == 1
    n = out.numel()
    dev = out.device
    if factors is None:
        factors = group_factors(n, workload, peer, dev)
    g = _gen(seed_of(workload, peer, rnd), dev)
    slice_elems = max(GROUP, (slice_elems // GROUP) * GROUP)
    for a in range(0, n, slice_elems):
        b = min(n, a + slice_elems)
        m = b - a
        z = torch.randn(m, generator=g, device=dev, dtype=torch.float32)
        ga = a // GROUP
        gb = (b + GROUP - 1) // GROUP
        f = factors[ga:gb].repeat_interleave(GROUP)[: m]
        u = torch.rand(m, generator=g, device=dev, dtype=torch.float32)
        z.mul_(f)
        z.mul_(torch.where(u < 0.001, torch.tensor(20.0, device=dev),
                           torch.tensor(1.0, device=dev)))
        out[a:b].copy_(z)
        del z, f, u
    return out


def lognormal(n: int, workload: int, peer: int, rnd: int, device="cpu",
              factors: torch.Tensor | None = None) -> torch.Tensor:
    out = torch.empty(n, dtype=torch.float32, device=device)
    return fill_lognormal_(out, workload, peer, rnd, factors)


def zero_chunk_ids(n_chunks: int, workload: int, peer: int, frac: float = 0.2,
                   device="cpu") -> torch.Tensor:
    """The first round(frac * n_chunks) chunks of a seeded permutation."""
    g = _gen(seed_of(workload, peer, HELD) ^ 0x5A5A5A5A, "cpu")
    perm = torch.randperm(n_chunks, generator=g)
    k = int(round(frac * n_chunks))
    return perm[:k].to(device)


def student_t3(n: int, workload: int, peer: int, rnd: int, device="cpu",
               zero_frac: float = 0.2, slice_elems: int = 1 << 26) -> torch.Tensor:
    """Student-t(3) values with a seeded set of exactly-zero 4096-chunks."""
    assert n % CHUNK == 0
    out = torch.empty(n, dtype=torch.float32, device=device)
    g = _gen(seed_of(workload, peer, rnd), device)
    slice_elems = max(CHUNK, (slice_elems // CHUNK) * CHUNK)
    for a in range(0, n, slice_elems):
        b = min(n, a + slice_elems)
        m = b - a
        z = torch.randn(m, generator=g, device=device, dtype=torch.float32)
        c = torch.randn(3, m, generator=g, device=device, dtype=torch.float32)
        chi2 = c.square_().sum(0)
        z.div_(chi2.div_(3.0).sqrt_())
        out[a:b].copy_(z)
        del z, c, chi2
    zc = zero_chunk_ids(n // CHUNK, workload, peer, zero_frac, device)
    out.view(-1, CHUNK)[zc] = 0.0
    return out


def workload_delta(workload: int, peer: int, rnd: int, device="cpu",
                   n: int | None = None) -> torch.Tensor:
    """Delta for one (workload, peer, round); n overrides the size (for tests
    that need the distribution at a smaller size)."""
    if n is None:
        n = WORKLOAD_PARAMS[workload]
    if workload == MLP_8192x28672:
        return student_t3(n, workload, peer, rnd, device)
    return lognormal(n, workload, peer, rnd, device)


def theta0(n: int, workload: int, device="cpu") -> torch.Tensor:
    """Initial parameters for the outer update: 0.02 * N(0,1)."""
    g = _gen(seed_of(workload, 0xFFFE, HELD), device)
    return torch.randn(n, generator=g, device=device, dtype=torch.float32).mul_(0.02)


def edge_crossing_layout():
    """Tensor sizes of a concatenated buffer whose chunk boundaries cross
    tensor edges: a 1000-element tensor, a 12,288-element tensor, then 3096
    elements of padding (16,384 = 4 chunks in all).  Chunk 0 holds the first
    tensor and the start of the second; chunk 3 holds the end of the second
    and the padding."""
    return [1000, 3 * CHUNK, 3096]


def random_entries(n_chunks: int, seed: int, k: int = 64, chunk: int = CHUNK,
                   scale_range=(1e-3, 10.0)):
    """Random well-formed chunk entries (not packed): strictly increasing
    indices, random 2-bit codes and positive finite scales.  numpy, host."""
    rng = np.random.default_rng(seed)
    idx = np.empty((n_chunks, k), dtype=np.int32)
    for c in range(n_chunks):
        idx[c] = np.sort(rng.choice(chunk, size=k, replace=False))
    code = rng.integers(0, 4, size=(n_chunks, k), dtype=np.uint8)
    lo, hi = scale_range
    scales = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n_chunks)).astype(np.float32)
    return idx, code, scales


def random_entries_bulk(n_chunks: int, seed: int, k: int = 64, chunk: int = CHUNK,
                        scale_range=(1e-3, 10.0)):
    """Like random_entries, vectorised for millions of chunks.  The k gaps
    before each kept index are 1 + floor of a random composition of the
    chunk - k spare positions over k + 1 parts, so indices are strictly
    increasing and start anywhere from 0; an eighth of the chunks are shifted
    to end exactly at chunk - 1."""
    rng = np.random.default_rng(seed)
    w = rng.random((n_chunks, k + 1))
    w *= (chunk - k) / w.sum(axis=1, keepdims=True)
    gaps = np.floor(w[:, :k]).astype(np.int32) + 1
    idx = np.cumsum(gaps, axis=1, dtype=np.int32) - 1
    right = rng.random(n_chunks) < 0.125           # an eighth end exactly at chunk - 1
    idx[right] += (chunk - 1 - idx[right, -1])[:, None]
    code = rng.integers(0, 4, size=(n_chunks, k), dtype=np.uint8)
    lo, hi = scale_range
    scales = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n_chunks)).astype(np.float32)
    return idx, code, scales
