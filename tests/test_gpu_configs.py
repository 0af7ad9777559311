"""GPU parity at the two largest workloads.

The decoder block is compared at every chunk for the compressor rounds and for
aggregate / apply on oracle-packed records, and on sampled chunks for the full
compress -> aggregate -> apply chain over 24 peers.  Every output of the
compressor and the aggregator depends only on its own chunk, so comparing the
GPU's full-size result with the oracle on a sample of chunks (plus the boundary
chunks) is exact, not statistical.  The oracle follows the
sampled chunks through every round from the same seeded inputs, and builds its
own peer records for them; nothing it consumes comes from the HIP path.
"""
import numpy as np
import pytest
import torch

from communication_efficient_distributed_amd import datagen
from gpu_util import assert_bitwise, assert_rel, note, oracle_threads, require_gpu

pytestmark = pytest.mark.gpu

CHUNK = 4096


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    """Chunks idx of a flat device tensor, as a host array [len(idx), 4096]."""
    i = torch.from_numpy(idx.astype(np.int64)).to(t.device)
    return t.view(-1, CHUNK).index_select(0, i).cpu().numpy()


def gather_rows(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    i = torch.from_numpy(idx.astype(np.int64)).to(t.device)
    return t.index_select(0, i).cpu().numpy()


def sample_chunks(n_chunks, extra, k, seed):
    rng = np.random.default_rng(seed)
    s = set(int(x) for x in rng.choice(n_chunks, size=min(k, n_chunks), replace=False))
    s |= {int(x) for x in extra if 0 <= x < n_chunks}
    return np.array(sorted(s), dtype=np.int64)


def block_chunk_edges(C):
    edges, off = [0, C - 1], 0
    for _, (a, b) in datagen.BLOCK_SHAPES:
        off += a * b
        edges += [off // CHUNK - 1, off // CHUNK]
    return edges


def test_decoder_block_two_rounds_full(orc):
    """One decoder block of a d=8192, 64-Q/8-KV-head transformer (Q, K, V, O,
    gate, up, down = 855,638,016 params) compressed as one flat buffer, two
    rounds from ef = 0: records, scales and ef compared at every chunk."""
    sl = require_gpu()
    W = datagen.DECODER_BLOCK
    n = datagen.WORKLOAD_PARAMS[W]
    T = oracle_threads()
    dev = torch.device("cuda:0")
    ef = torch.zeros(n, dtype=torch.float32, device=dev)
    ef_o = np.zeros(n, np.float32)
    factors = datagen.group_factors(n, W, 0, dev)
    for rnd in range(2):
        d = datagen.lognormal(n, W, 0, rnd, dev, factors=factors)
        note(f"decoder block round {rnd}: sl_compress n={n}")
        payload, scales = sl.compress(d, ef, 0.95)
        torch.cuda.synchronize()
        op, os_, ef_o = orc.compress(d.cpu().numpy(), ef_o, beta=0.95, nthreads=T, inplace=True)
        del d
        assert_bitwise(payload.cpu().numpy(), op, f"round {rnd} payload")
        assert_bitwise(scales.cpu().numpy(), os_, f"round {rnd} scales")
        assert_bitwise(ef.cpu().numpy(), ef_o, f"round {rnd} ef")
        del payload, scales


def test_decoder_block_peers_aggregate_apply_sampled(orc):
    """The chain at the decoder block: 24 peers' deltas compressed from ef = 0,
    their records aggregated, then theta <- theta - sum/24; compared on 2048
    sampled chunks plus the chunks on each side of every tensor edge.  The
    oracle builds its own peer records from the same seeded deltas."""
    sl = require_gpu()
    W = datagen.DECODER_BLOCK
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK
    T = oracle_threads()
    dev = torch.device("cuda:0")
    idx = sample_chunks(C, block_chunk_edges(C), 2048, seed=4)
    m = idx.size
    peer_p, peer_s, orc_p, orc_s = [], [], [], []
    scratch = torch.zeros(n, dtype=torch.float32, device=dev)
    for p in range(1, 25):
        d = datagen.lognormal(n, W, p, 0, dev)
        scratch.zero_()
        note(f"decoder block peer {p}: sl_compress")
        pl, s = sl.compress(d, scratch, 0.95)
        peer_p.append(pl)
        peer_s.append(s)
        op, os_, _ = orc.compress(gather(d, idx).reshape(-1), np.zeros(m * CHUNK, np.float32),
                                  beta=0.95, nthreads=T)
        orc_p.append(op)
        orc_s.append(os_)
        del d
    del scratch
    note("decoder block: sl_aggregate 24 peers")
    out = sl.aggregate(peer_p, peer_s, n)
    theta = datagen.theta0(n, W, dev)
    theta_s = gather(theta, idx).reshape(-1)
    note("decoder block: sl_apply_mean")
    sl.sl_apply_mean(theta, out, 24)
    torch.cuda.synchronize()
    o = orc.aggregate(orc_p, orc_s, m * CHUNK, nthreads=T)
    g = gather(out, idx).reshape(-1)
    assert_rel(g, o, "block aggregate")
    assert_bitwise(g, o, "block aggregate")
    assert_bitwise(gather(theta, idx).reshape(-1), orc.apply_mean(theta_s, o, 24), "block apply")


def test_decoder_block_aggregate_apply_full(orc):
    """Aggregate, apply and the fused aggregate-apply at the decoder block's
    full size, compared at every element: 24 peers of random well-formed
    records packed by the oracle (an eighth of the chunks end at index 4095)."""
    sl = require_gpu()
    W = datagen.DECODER_BLOCK
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK
    T = oracle_threads()
    dev = torch.device("cuda:0")
    orc_p, orc_s = [], []
    for p in range(1, 25):
        idx, code, sc = datagen.random_entries_bulk(C, (W << 32) | (p << 16) | 0xFFFD)
        orc_p.append(orc.pack(idx, code))
        orc_s.append(sc)
        del idx, code
    peer_p = [torch.from_numpy(x).to(dev) for x in orc_p]
    peer_s = [torch.from_numpy(x).to(dev) for x in orc_s]
    note("decoder block full: sl_aggregate 24 peers")
    out = sl.aggregate(peer_p, peer_s, n)
    theta = datagen.theta0(n, W, dev)
    theta_h = theta.cpu().numpy()
    fused = theta.clone()
    note("decoder block full: sl_apply_mean")
    sl.sl_apply_mean(theta, out, 24)
    note("decoder block full: sl_aggregate_apply 24 peers")
    sl.sl_aggregate_apply(peer_p, peer_s, fused)
    torch.cuda.synchronize()
    o = orc.aggregate(orc_p, orc_s, n, nthreads=T)
    assert_bitwise(out.cpu().numpy(), o, "block aggregate (full)")
    del out
    want = orc.apply_mean(theta_h, o, 24)
    assert_bitwise(theta.cpu().numpy(), want, "block apply (full)")
    assert_bitwise(fused.cpu().numpy(), want, "block fused aggregate-apply (full)")


def _free_gpu_bytes():
    free, _ = torch.cuda.mem_get_info()
    return free


def test_flat_16b_span_sampled(orc):
    """A 16e9-parameter flat span (64 GB delta + 64 GB ef resident; ef then holds
    the 64 GB dense update),
    per-1024 lognormal scales, 10 consecutive rounds, then 24 peers aggregated.
    Sampled parity includes the chunks at element offsets 2^31 and 2^32 and at
    byte offset 2^32, where 32-bit indexing would break."""
    sl = require_gpu()
    W = datagen.FLAT_16B
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK
    need = 2 * 4 * n + 25 * C * 116 + (8 << 30)   # delta, ef (reused as out), records, slack
    if _free_gpu_bytes() < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory")
    T = oracle_threads()
    dev = torch.device("cuda:0")
    special = [0, C - 1, (1 << 31) // CHUNK - 1, (1 << 31) // CHUNK, (1 << 32) // CHUNK - 1,
               (1 << 32) // CHUNK, (1 << 32) // (4 * CHUNK), (1 << 32) // (4 * CHUNK) - 1]
    per = -(-C // -(-C // (1 << 16)))    # chunks per streaming launch (60 launches)
    special += [per - 1, per, 59 * per - 1, 59 * per]
    idx = sample_chunks(C, special, 4096, seed=5)
    m = idx.size

    delta = torch.empty(n, dtype=torch.float32, device=dev)
    ef = torch.zeros(n, dtype=torch.float32, device=dev)
    ef_o = np.zeros(m * CHUNK, np.float32)
    factors = datagen.group_factors(n, W, 0, dev)
    for rnd in range(10):
        datagen.fill_lognormal_(delta, W, 0, rnd, factors=factors)
        note(f"16B span round {rnd}: sl_compress n={n}")
        payload, scales = sl.compress(delta, ef, 0.95)
        torch.cuda.synchronize()
        op, os_, ef_o = orc.compress(gather(delta, idx).reshape(-1), ef_o, beta=0.95, nthreads=T,
                                     inplace=True)
        assert_bitwise(gather_rows(payload, idx), op, f"round {rnd} payload")
        assert_bitwise(gather_rows(scales, idx), os_, f"round {rnd} scales")
        assert_bitwise(gather(ef, idx).reshape(-1), ef_o, f"round {rnd} ef")
        del payload, scales
    del factors

    # Peers: delta_p generated into `delta`, compressed against a zeroed `ef`
    # (the local ef is no longer needed); the records stay resident.
    peer_p, peer_s, orc_p, orc_s = [], [], [], []
    for p in range(1, 25):
        fac = datagen.group_factors(n, W, p, dev)
        datagen.fill_lognormal_(delta, W, p, 0, factors=fac)
        del fac
        ef.zero_()
        note(f"16B span peer {p}: sl_compress")
        pl, s = sl.compress(delta, ef, 0.95)
        peer_p.append(pl)
        peer_s.append(s)
        op, os_, _ = orc.compress(gather(delta, idx).reshape(-1), np.zeros(m * CHUNK, np.float32),
                                  beta=0.95, nthreads=T)
        orc_p.append(op)
        orc_s.append(os_)
    del delta
    out = ef  # reuse the 64 GB buffer for the dense update
    note("16B span: sl_aggregate 24 peers")
    sl.sl_aggregate(peer_p, peer_s, out)
    torch.cuda.synchronize()
    o = orc.aggregate(orc_p, orc_s, m * CHUNK, nthreads=T)
    g = gather(out, idx).reshape(-1)
    assert_rel(g, o, "16B aggregate")
    assert_bitwise(g, o, "16B aggregate")


def test_span_split_over_launches_sampled(orc):
    """A span of 2^22 + 3 chunks (17.2e9 parameters), past where the library
    splits an aggregate call into two kernel launches (2^22 chunks each at
    most; the streaming kernels, compress and apply_mean, split long calls
    into equal launches of at most 2^16 chunks, here 65 of 64,528): compress
    (two rounds), compress from weights, 2-peer aggregate, fused
    aggregate-apply and apply_mean, then the aggregate and the fused update on
    the same records laid out chunk-major, compared with the oracle on sampled
    chunks that include both sides of the 2^22 split and of the first and last
    streaming-launch boundaries."""
    sl = require_gpu()
    W = datagen.FLAT_16B
    K = 1 << 22
    C = K + 3
    n = C * CHUNK
    need = 2 * 4 * n + 5 * C * 116 + (8 << 30)   # two dense buffers, records (both layouts), slack
    if _free_gpu_bytes() < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory")
    T = oracle_threads()
    dev = torch.device("cuda:0")
    parts = -(-C // (1 << 16))
    per = -(-C // parts)                 # chunks per streaming launch
    last = (parts - 1) * per
    idx = sample_chunks(C, [0, 1, per - 1, per, last - 1, last, K - 2, K - 1, K, K + 1, K + 2], 512, seed=7)
    m = idx.size

    a = torch.empty(n, dtype=torch.float32, device=dev)
    ef = torch.zeros(n, dtype=torch.float32, device=dev)
    ef_o = np.zeros(m * CHUNK, np.float32)
    factors = datagen.group_factors(n, W, 0, dev)
    for rnd in range(2):
        datagen.fill_lognormal_(a, W, 0, 0x100 + rnd, factors=factors)
        note(f"split span round {rnd}: sl_compress n={n}")
        payload, scales = sl.compress(a, ef, 0.95)
        torch.cuda.synchronize()
        op, os_, ef_o = orc.compress(gather(a, idx).reshape(-1), ef_o, beta=0.95, nthreads=T, inplace=True)
        assert_bitwise(gather_rows(payload, idx), op, f"round {rnd} payload")
        assert_bitwise(gather_rows(scales, idx), os_, f"round {rnd} scales")
        assert_bitwise(gather(ef, idx).reshape(-1), ef_o, f"round {rnd} ef")

    # Weights variant with theta_pre and theta_post the same buffer: delta is 0
    # at every chunk only if both are sliced alike for every launch.
    datagen.fill_lognormal_(a, W, 0, 0x102, factors=factors)
    note("split span: sl_compress_weights (theta_pre aliases theta_post)")
    sl.sl_compress_weights(a, a, ef, 0.95, payload, scales)
    torch.cuda.synchronize()
    th = gather(a, idx).reshape(-1)
    op, os_, ef_o = orc.compress(orc.pseudo_gradient(th, th), ef_o, beta=0.95, nthreads=T, inplace=True)
    assert_bitwise(gather_rows(payload, idx), op, "weights payload")
    assert_bitwise(gather_rows(scales, idx), os_, "weights scales")
    assert_bitwise(gather(ef, idx).reshape(-1), ef_o, "weights ef")
    del payload, scales, factors

    peer_p, peer_s, orc_p, orc_s = [], [], [], []
    for p in (1, 2):
        datagen.fill_lognormal_(a, W, p, 0x100)
        ef.zero_()
        note(f"split span peer {p}: sl_compress")
        pl, s = sl.compress(a, ef, 0.95)
        peer_p.append(pl)
        peer_s.append(s)
        op, os_, _ = orc.compress(gather(a, idx).reshape(-1), np.zeros(m * CHUNK, np.float32),
                                  beta=0.95, nthreads=T)
        orc_p.append(op)
        orc_s.append(os_)

    out = ef
    note("split span: sl_aggregate 2 peers")
    sl.sl_aggregate(peer_p, peer_s, out)
    torch.cuda.synchronize()
    o = orc.aggregate(orc_p, orc_s, m * CHUNK, nthreads=T)
    assert_bitwise(gather(out, idx).reshape(-1), o, "split aggregate")

    theta = a
    datagen.fill_lognormal_(theta, W, 0, 0x103)
    th0 = gather(theta, idx).reshape(-1)
    note("split span: sl_aggregate_apply 2 peers")
    sl.sl_aggregate_apply(peer_p, peer_s, theta)
    torch.cuda.synchronize()
    th1 = orc.apply_mean(th0, o, 2)
    assert_bitwise(gather(theta, idx).reshape(-1), th1, "split aggregate_apply")

    note("split span: sl_apply_mean")
    sl.sl_apply_mean(theta, out, 2)
    torch.cuda.synchronize()
    assert_bitwise(gather(theta, idx).reshape(-1), orc.apply_mean(th1, o, 2), "split apply_mean")

    # The same two peers' records laid out chunk-major: each launch of the
    # split must start at its own chunk's records (offset c0 * 2 * 112).
    rec = torch.empty((C, 2, 112), dtype=torch.uint8, device=dev)
    sc = torch.empty((C, 2), dtype=torch.float32, device=dev)
    for k in range(2):
        rec[:, k, :] = peer_p[k]
        sc[:, k] = peer_s[k]
    del peer_p, peer_s
    note("split span: sl_aggregate_interleaved 2 peers")
    out.fill_(float("nan"))
    sl.sl_aggregate_interleaved(rec, sc, out)
    torch.cuda.synchronize()
    assert_bitwise(gather(out, idx).reshape(-1), o, "split aggregate, chunk-major")
    datagen.fill_lognormal_(theta, W, 0, 0x103)
    note("split span: sl_aggregate_apply_interleaved 2 peers")
    sl.sl_aggregate_apply_interleaved(rec, sc, theta)
    torch.cuda.synchronize()
    assert_bitwise(gather(theta, idx).reshape(-1), th1, "split aggregate_apply, chunk-major")
