"""A whole round captured in a HIP graph, through the C ABI.

The round is: validate each peer's records, take the per-peer statistics of
all of them in one pass, then the fused aggregate + outer update of theta,
then compress the next pseudo-gradient.  The library issues
no allocation and no memset, so the captured kernels replay exactly as
launched.  Every replay runs with eager work (input resets, host copies)
between replays, and is compared with the oracle.
"""
import numpy as np
import pytest
import torch

from communication_efficient_distributed_amd import datagen
from gpu_util import assert_bitwise, note, require_gpu

pytestmark = pytest.mark.gpu


def test_round_replayed_from_a_graph(orc):
    sl = require_gpu()
    dev = torch.device("cuda:0")
    C, N = 64, 5
    n = C * 4096
    W = datagen.SMALL_1M

    # Oracle-made peer records (one with a malformed chunk, flagged but still summed).
    peers_p, peers_s = [], []
    for p in range(1, N + 1):
        d = datagen.lognormal(n, W, p, 3).numpy()
        pl, s, _ = orc.compress(d, np.zeros(n, np.float32), beta=0.95)
        peers_p.append(pl)
        peers_s.append(s)
    peers_s[2] = peers_s[2].copy()
    peers_s[2][7] = -1.0                           # negative scale: flag bit 2
    theta0 = datagen.theta0(n, W).numpy()
    delta0 = datagen.lognormal(n, W, 0, 4).numpy()
    ef0 = (datagen.lognormal(n, W, 0, 5).numpy() * np.float32(0.1)).astype(np.float32)

    # What the round must produce.
    want_flags = [orc.validate(pl, s)[1] for pl, s in zip(peers_p, peers_s)]
    want_stats = [orc.peer_stats(pl, s) for pl, s in zip(peers_p, peers_s)]
    want_theta = orc.apply_mean(theta0, orc.aggregate(peers_p, peers_s, n), N)
    want_payload, want_scales, want_ef = orc.compress(delta0, ef0, beta=0.95)

    # Static device buffers the graph reads and writes.
    dp = [torch.from_numpy(x).to(dev) for x in peers_p]
    ds = [torch.from_numpy(x).to(dev) for x in peers_s]
    theta = torch.empty(n, dtype=torch.float32, device=dev)
    delta = torch.empty(n, dtype=torch.float32, device=dev)
    ef = torch.empty(n, dtype=torch.float32, device=dev)
    payload = torch.empty((C, 112), dtype=torch.uint8, device=dev)
    scales = torch.empty(C, dtype=torch.float32, device=dev)
    flags = torch.empty((N, C), dtype=torch.uint8, device=dev)
    counts = torch.empty((N, 4), dtype=torch.int64, device=dev)
    smax = torch.empty(N, dtype=torch.float32, device=dev)
    src = {k: torch.from_numpy(v).to(dev) for k, v in
           (("theta", theta0), ("delta", delta0), ("ef", ef0))}

    def reset():
        theta.copy_(src["theta"])
        delta.copy_(src["delta"])
        ef.copy_(src["ef"])
        payload.zero_()
        scales.zero_()
        flags.fill_(0xFF)
        counts.fill_(-1)                       # the statistics pass must clear its outputs itself
        smax.fill_(-1.0)

    def round_():
        for p in range(N):
            sl.sl_validate_payload(dp[p], ds[p], flags[p])
        sl.sl_peer_stats(dp, ds, counts, smax)
        sl.sl_aggregate_apply(dp, ds, theta)
        sl.sl_compress(delta, ef, 0.95, payload, scales)

    def check(what):
        torch.cuda.synchronize()
        for p in range(N):
            assert_bitwise(flags[p].cpu().numpy(), want_flags[p], f"{what}: flags of peer {p}")
            assert counts[p].cpu().tolist() == want_stats[p][0].tolist(), f"{what}: counts of peer {p}"
            assert_bitwise(smax[p:p + 1].cpu().numpy(), np.float32([want_stats[p][1]]), f"{what}: scale_max of peer {p}")
        assert_bitwise(theta.cpu().numpy(), want_theta, f"{what}: theta")
        assert_bitwise(payload.cpu().numpy(), want_payload, f"{what}: payload")
        assert_bitwise(scales.cpu().numpy(), want_scales, f"{what}: scales")
        assert_bitwise(ef.cpu().numpy(), want_ef, f"{what}: ef")

    # Eager reference run (also the warm-up torch asks for before capture).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        note("graph test: eager round")
        round_()
    torch.cuda.current_stream().wait_stream(side)
    check("eager")
    assert int((flags[2].cpu().numpy() != 0).sum()) == 1

    graph = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    note("graph test: capture")
    with torch.cuda.graph(graph):
        round_()
    for rep in range(3):
        reset()                                   # eager work between replays
        torch.cuda.synchronize()
        note(f"graph test: replay {rep}")
        graph.replay()
        check(f"replay {rep}")
        _ = theta.sum().item()                    # more eager work on the same stream
