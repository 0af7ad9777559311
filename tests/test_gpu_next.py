"""GPU parity of the rows after the core path: the pseudo-gradient formed inside
the compressor, payload validation for untrusted peers, and error feedback
offloaded to pinned host memory."""
import numpy as np
import pytest
import torch

from communication_efficient_distributed_amd import datagen
from gpu_util import assert_bitwise, note, oracle_threads, require_gpu

pytestmark = pytest.mark.gpu


def weights_pair(n, seed):
    """theta_pre ~ 0.02 N(0,1) and theta_post = theta_pre - a lognormal step."""
    g = torch.Generator().manual_seed(seed)
    pre = torch.randn(n, generator=g) * 0.02
    step = datagen.lognormal(n, datagen.SMALL_1M, 7, seed) * 1e-3
    return pre.numpy().astype(np.float32), (pre - step).numpy().astype(np.float32)


@pytest.mark.parametrize("n", [256 * 4096, datagen.WORKLOAD_PARAMS[datagen.MLP_8192x28672]])
def test_compress_weights(orc, n):
    sl = require_gpu()
    T = oracle_threads()
    ef_o = np.zeros(n, np.float32)
    ef_g = torch.zeros(n, dtype=torch.float32, device="cuda")
    for rnd in range(2):
        pre, post = weights_pair(n, 10 + rnd)
        note(f"sl_compress_weights n={n} round {rnd}")
        C = n // 4096
        payload = torch.empty((C, 112), dtype=torch.uint8, device="cuda")
        scales = torch.empty(C, dtype=torch.float32, device="cuda")
        sl.sl_compress_weights(torch.from_numpy(pre).cuda(), torch.from_numpy(post).cuda(), ef_g,
                               0.95, payload, scales)
        torch.cuda.synchronize()
        delta = orc.pseudo_gradient(pre, post)
        op, os_, ef_o = orc.compress(delta, ef_o, beta=0.95, nthreads=T, inplace=True)
        assert_bitwise(payload.cpu().numpy(), op, "payload")
        assert_bitwise(scales.cpu().numpy(), os_, "scales")
        assert_bitwise(ef_g.cpu().numpy(), ef_o, "ef")


def test_validate_payload_flags(orc):
    sl = require_gpu()
    C = 512
    idx, code, sc = datagen.random_entries(C, 321)
    rng = np.random.default_rng(3)
    bad_rows = rng.choice(C, 60, replace=False)
    for k, c in enumerate(bad_rows):
        kind = k % 6
        if kind == 0:
            j = rng.integers(1, 64)
            idx[c, [j - 1, j]] = idx[c, [j, j - 1]]        # swapped neighbours
        elif kind == 1:
            j = rng.integers(1, 64)
            idx[c, j] = idx[c, j - 1]                      # duplicate
        elif kind == 2:
            sc[c] = np.nan
        elif kind == 3:
            sc[c] = -np.float32(rng.random() + 0.1)        # negative
        elif kind == 4:
            sc[c] = -np.inf
        else:
            idx[c] = idx[c][::-1]                          # descending
            sc[c] = np.inf
    payload = orc.pack(idx, code)
    _, want = orc.validate(payload, sc)
    assert (want != 0).sum() == 60
    flags = torch.full((C,), 255, dtype=torch.uint8, device="cuda")
    note("sl_validate_payload planted defects")
    sl.sl_validate_payload(torch.from_numpy(payload).cuda(), torch.from_numpy(sc).cuda(), flags)
    torch.cuda.synchronize()
    assert_bitwise(flags.cpu().numpy(), want, "flags")


def defective_peers(orc, N, C, seed):
    """N peers of C records each; every third peer gets 40 defects (order,
    duplicates, NaN of either sign, -inf, negative denormal scale, -0 which is
    allowed, reversed indices)."""
    rng = np.random.default_rng(seed)
    payloads, scales = [], []
    for p in range(N):
        idx, code, sc = datagen.random_entries_bulk(C, 900 + p)
        if p % 3 == 1:
            rows = rng.choice(C, 40, replace=False)
            for k, c in enumerate(rows):
                kind = k % 8
                if kind == 0:
                    j = rng.integers(1, 64)
                    idx[c, [j - 1, j]] = idx[c, [j, j - 1]]
                elif kind == 1:
                    j = rng.integers(1, 64)
                    idx[c, j] = idx[c, j - 1]
                elif kind == 2:
                    sc[c] = np.nan
                elif kind == 3:
                    sc[c] = np.uint32(0xFFC00001).view(np.float32)    # NaN with the sign bit
                elif kind == 4:
                    sc[c] = -np.inf
                elif kind == 5:
                    sc[c] = np.uint32(0x80000001).view(np.float32)    # -smallest denormal
                elif kind == 6:
                    sc[c] = -0.0                                      # allowed
                else:
                    idx[c] = idx[c][::-1]
        if p % 4 == 2:
            code[rng.choice(C, 9, replace=False)] = 1                 # crafted: all entries at +s
            sc[rng.choice(C, 5, replace=False)] = 0.0                 # empty chunks
        if p == 5:
            sc[3] = np.inf                                            # flagged, above every finite scale
            sc[4] = np.float32(3e38)                                  # the largest valid scale
        payloads.append(orc.pack(idx, code))
        scales.append(sc)
    return payloads, scales


def test_validate_many_peers_in_one_launch(orc):
    """sl_validate_payloads over 24 peers and a ragged 1000 records each, with
    defects planted in some peers, row by row against the oracle."""
    sl = require_gpu()
    N, C = 24, 1000
    payloads, scales = defective_peers(orc, N, C, 17)
    want = [orc.validate(pl, sc)[1] for pl, sc in zip(payloads, scales)]
    assert sum(int((w != 0).sum()) for w in want) >= 8 * 34      # defects planted (a few may be overwritten)
    flags = torch.full((N, C), 255, dtype=torch.uint8, device="cuda")
    note("sl_validate_payloads 24 peers x 1000 records")
    sl.sl_validate_payloads([torch.from_numpy(x).cuda() for x in payloads],
                            [torch.from_numpy(x).cuda() for x in scales], flags)
    torch.cuda.synchronize()
    got = flags.cpu().numpy()
    for p in range(N):
        assert_bitwise(got[p], want[p], f"flags of peer {p}")


def check_peer_stats(sl, orc, payloads, scales, with_flags=True):
    N, C = len(payloads), scales[0].size
    counts = torch.full((N, 4), -1, dtype=torch.int64, device="cuda")
    smax = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    flags = torch.full((N, C), 255, dtype=torch.uint8, device="cuda") if with_flags else None
    peers = sl.PeerSet([torch.from_numpy(x).cuda() for x in payloads], [torch.from_numpy(x).cuda() for x in scales])
    note(f"sl_peer_stats {N} peers x {C} records, flags={with_flags}")
    sl.sl_peer_stats(peers, None, counts, smax, flags=flags)
    torch.cuda.synchronize()
    got_c, got_m = counts.cpu().numpy(), smax.cpu().numpy()
    for p in range(N):
        wc, wm = orc.peer_stats(payloads[p], scales[p])
        assert got_c[p].tolist() == wc.tolist(), f"counts of peer {p}"
        assert_bitwise(got_m[p:p + 1], np.float32([wm]), f"scale_max of peer {p}")
    if with_flags:
        got_f = flags.cpu().numpy()
        for p in range(N):
            assert_bitwise(got_f[p], orc.validate(payloads[p], scales[p])[1], f"flags of peer {p}")
    return got_c, got_m


@pytest.mark.parametrize("N,C", [(5, 1025), (24, 7687), (128, 2049), (1, 70000), (3, 4096)])
def test_peer_stats_super_block_edges(orc, N, C):
    """sl_peer_stats where a peer's last super-block of 1024 records holds one
    record (5 x 1025, 128 x 2049), where the grid of 512 workgroups takes
    several super-blocks each and neighbouring super-blocks belong to
    different peers (24 x 7687, 128 x 2049), one peer spread over 69
    super-blocks (1 x 70000) and whole super-blocks only (3 x 4096), against
    the oracle."""
    sl = require_gpu()
    payloads, scales = defective_peers(orc, N, C, 500 + N)
    check_peer_stats(sl, orc, payloads, scales, with_flags=True)


def test_peer_stats_against_the_oracle(orc):
    """sl_peer_stats over 24 peers x 1000 records with planted defects,
    crafted all-magnitude chunks, zero scales and an infinite scale; counts,
    maxima and flags against the oracle; without flags the statistics are the
    same."""
    sl = require_gpu()
    payloads, scales = defective_peers(orc, 24, 1000, 17)
    a = check_peer_stats(sl, orc, payloads, scales, with_flags=True)
    b = check_peer_stats(sl, orc, payloads, scales, with_flags=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert a[1][5] == np.float32(3e38)


@pytest.mark.parametrize("N,C", [(1, 1), (3, 63), (128, 257), (24, 57344)])
def test_peer_stats_shapes(orc, N, C):
    """One record, ragged counts, the most peers, and the full 8192 x 28672
    shape with 24 peers."""
    sl = require_gpu()
    payloads, scales = [], []
    for p in range(N):
        idx, code, sc = datagen.random_entries_bulk(C, 3100 + p)
        payloads.append(orc.pack(idx, code))
        scales.append(sc)
    check_peer_stats(sl, orc, payloads, scales, with_flags=(N * C <= 200000))


def test_peer_stats_calls_in_a_row(orc):
    """Twenty calls on one stream alternating two shapes (24 peers x 3000
    records, 128 x 40): every call leaves the scratch's arrival counters at
    zero for the next, and every result matches the oracle."""
    sl = require_gpu()
    shapes = []
    for N, C, seed in ((24, 3000, 61), (128, 40, 62)):
        payloads, scales = [], []
        for p in range(N):
            idx, code, sc = datagen.random_entries_bulk(C, seed * 1000 + p)
            sc = sc.copy()
            sc[p % C] = 0.0
            payloads.append(orc.pack(idx, code))
            scales.append(sc.astype(np.float32))
        want = [orc.peer_stats(pl, sc) for pl, sc in zip(payloads, scales)]
        peers = sl.PeerSet([torch.from_numpy(x).cuda() for x in payloads],
                           [torch.from_numpy(x).cuda() for x in scales])
        shapes.append((N, peers, want))
    for k in range(20):
        N, peers, want = shapes[k % 2]
        counts = torch.full((N, 4), -1, dtype=torch.int64, device="cuda")
        smax = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
        note(f"sl_peer_stats call {k}: {N} peers")
        sl.sl_peer_stats(peers, None, counts, smax)
        torch.cuda.synchronize()
        got_c, got_m = counts.cpu().numpy(), smax.cpu().numpy()
        for p in range(N):
            assert got_c[p].tolist() == want[p][0].tolist(), f"call {k}: counts of peer {p}"
            assert_bitwise(got_m[p:p + 1], np.float32([want[p][1]]), f"call {k}: scale_max of peer {p}")


def test_peer_stats_without_records():
    """n_chunks = 0: the statistics are still written, all zero."""
    sl = require_gpu()
    counts = torch.full((3, 4), 7, dtype=torch.int64, device="cuda")
    smax = torch.full((3,), 7.0, dtype=torch.float32, device="cuda")
    e = [torch.empty(0, dtype=torch.uint8, device="cuda")] * 3
    s = [torch.empty(0, dtype=torch.float32, device="cuda")] * 3
    note("sl_peer_stats n_chunks=0")
    sl.sl_peer_stats(e, s, counts, smax)
    torch.cuda.synchronize()
    assert not counts.any() and smax.view(torch.int32).eq(0).all()


def test_compressor_output_is_well_formed():
    """Every record the compressor writes passes validation (full MLP shape,
    including its all-zero chunks)."""
    sl = require_gpu()
    W = datagen.MLP_8192x28672
    n = datagen.WORKLOAD_PARAMS[W]
    d = datagen.student_t3(n, W, 0, 0, torch.device("cuda"))
    payload, scales = sl.compress(d, torch.zeros_like(d), 0.95)
    flags = torch.full((n // 4096,), 255, dtype=torch.uint8, device="cuda")
    note("sl_validate_payload on compressor output")
    sl.sl_validate_payload(payload, scales, flags)
    torch.cuda.synchronize()
    assert int(flags.count_nonzero()) == 0


def test_ef_offloaded_to_host(orc):
    """ef in pinned host memory, read and written by the kernel in place:
    identical to device-resident ef and to the oracle over three rounds."""
    sl = require_gpu()
    n = 1 << 22
    ef_host = torch.zeros(n, dtype=torch.float32, pin_memory=True)
    ef_dev = torch.zeros(n, dtype=torch.float32, device="cuda")
    ef_o = np.zeros(n, np.float32)
    C = n // 4096
    for rnd in range(3):
        d = datagen.lognormal(n, datagen.SMALL_1M, 0, rnd).cuda()
        p1 = torch.empty((C, 112), dtype=torch.uint8, device="cuda")
        s1 = torch.empty(C, dtype=torch.float32, device="cuda")
        note(f"sl_compress with host ef, round {rnd}")
        sl.sl_compress_host_ef(d, ef_host, 0.95, p1, s1)
        p2, s2 = sl.compress(d, ef_dev, 0.95)
        torch.cuda.synchronize()
        op, os_, ef_o = orc.compress(d.cpu().numpy(), ef_o, beta=0.95, nthreads=oracle_threads(),
                                     inplace=True)
        assert_bitwise(p1.cpu().numpy(), op, "payload")
        assert_bitwise(s1.cpu().numpy(), os_, "scales")
        assert_bitwise(ef_host.numpy(), ef_o, "host ef")
        assert_bitwise(ef_dev.cpu().numpy(), ef_o, "device ef")
        assert_bitwise(p2.cpu().numpy(), op, "device-ef payload")


def test_outer_loop_rounds(orc):
    """Three outer rounds of five peers, composed as the pages' round runs.
    Each peer p has its own error feedback. It takes theta, runs a synthetic
    inner loop (theta_post = theta - step_p) and compresses its
    pseudo-gradient straight from the weights (sl_compress_weights). The
    round's records are screened (sl_peer_stats) and applied to theta with
    the fused update (sl_aggregate_apply), and the next round starts from
    that theta. Everything is compared with the oracle doing the same,
    bitwise, every round."""
    sl = require_gpu()
    N, C = 5, 48
    n = C * 4096
    W = datagen.SMALL_1M
    theta_o = datagen.theta0(n, W).numpy()
    theta_g = torch.from_numpy(theta_o).cuda()
    ef_o = [np.zeros(n, np.float32) for _ in range(N)]
    ef_g = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(N)]
    pay_g = [torch.empty((C, 112), dtype=torch.uint8, device="cuda") for _ in range(N)]
    sc_g = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(N)]
    counts = torch.empty((N, 4), dtype=torch.int64, device="cuda")
    smax = torch.empty(N, dtype=torch.float32, device="cuda")
    for rnd in range(3):
        pay_o, sc_o = [], []
        for p in range(N):
            step = (datagen.lognormal(n, W, p + 1, 50 + rnd).numpy() * np.float32(1e-3)).astype(np.float32)
            post_o = (theta_o - step).astype(np.float32)
            pl, s, ef_o[p] = orc.compress(orc.pseudo_gradient(theta_o, post_o), ef_o[p], beta=0.95)
            pay_o.append(pl)
            sc_o.append(s)
            note(f"outer loop round {rnd} peer {p}: sl_compress_weights")
            sl.sl_compress_weights(theta_g, torch.from_numpy(post_o).cuda(), ef_g[p], 0.95, pay_g[p], sc_g[p])
        note(f"outer loop round {rnd}: sl_peer_stats + sl_aggregate_apply")
        sl.sl_peer_stats(pay_g, sc_g, counts, smax)
        sl.sl_aggregate_apply(pay_g, sc_g, theta_g)
        theta_o = orc.apply_mean(theta_o, orc.aggregate(pay_o, sc_o, n), N)
        torch.cuda.synchronize()
        for p in range(N):
            assert_bitwise(pay_g[p].cpu().numpy(), pay_o[p], f"round {rnd} peer {p} records")
            assert_bitwise(sc_g[p].cpu().numpy(), sc_o[p], f"round {rnd} peer {p} scales")
            assert_bitwise(ef_g[p].cpu().numpy(), ef_o[p], f"round {rnd} peer {p} ef")
            wc, wm = orc.peer_stats(pay_o[p], sc_o[p])
            assert counts[p].cpu().tolist() == wc.tolist(), f"round {rnd} peer {p} counts"
            assert wc[0] == 0                         # the compressor's records are well formed
        assert_bitwise(theta_g.cpu().numpy(), theta_o, f"round {rnd} theta")


def test_rounds_with_changing_participation_and_ef_resume(orc):
    """Five outer rounds in which participation changes, as the pages' open
    network allows: a peer that sits a round out runs no compressor, so its
    error feedback is untouched; a peer whose records do not arrive (lost, or
    filtered out by the validator) has still updated its own error feedback,
    but the update sums only what arrived. The third round delivers nothing:
    the sum is +0 everywhere and theta is left as it is. Before the fourth
    round every peer's error feedback is saved to host memory, the device
    buffers are freed, and the run continues from fresh buffers restored from
    the saved copies; the error feedback is the compressor's only state, so
    the continuation must match the oracle, which never stopped, bit for bit.
    The last two rounds deliver chunk-major records (one peer, then all),
    applied through sl_aggregate_apply_interleaved and through
    sl_aggregate_interleaved + sl_apply_mean."""
    sl = require_gpu()
    N, C = 6, 37
    n = C * 4096
    W = datagen.SMALL_1M
    # (peers that compress, peers whose records arrive) per round
    rounds = [(range(6), range(6)),
              ((0, 1, 2, 4, 5), (0, 2, 5)),
              ((1, 3), ()),
              (range(6), (3,)),
              (range(6), range(6))]
    theta_o = datagen.theta0(n, W).numpy()
    theta_g = torch.from_numpy(theta_o).cuda()
    ef_o = [np.zeros(n, np.float32) for _ in range(N)]
    ef_g = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(N)]
    pay_g = [torch.empty((C, 112), dtype=torch.uint8, device="cuda") for _ in range(N)]
    sc_g = [torch.empty(C, dtype=torch.float32, device="cuda") for _ in range(N)]
    for rnd, (active, arrived) in enumerate(rounds):
        if rnd == 3:
            note("saving every peer's error feedback to host and restoring it into new buffers")
            saved = [e.cpu().numpy().copy() for e in ef_g]
            del ef_g
            torch.cuda.synchronize()
            ef_g = [torch.from_numpy(s).cuda() for s in saved]
        pay_o, sc_o = {}, {}
        for p in active:
            step = (datagen.lognormal(n, W, p + 11, 90 + rnd).numpy() * np.float32(1e-3)).astype(np.float32)
            post_o = (theta_o - step).astype(np.float32)
            pay_o[p], sc_o[p], ef_o[p] = orc.compress(orc.pseudo_gradient(theta_o, post_o), ef_o[p], beta=0.95)
            note(f"participation round {rnd} peer {p}: sl_compress_weights")
            sl.sl_compress_weights(theta_g, torch.from_numpy(post_o).cuda(), ef_g[p], 0.95, pay_g[p], sc_g[p])
        got = [p for p in arrived]
        sum_o = orc.aggregate([pay_o[p] for p in got], [sc_o[p] for p in got], n)
        if not got:
            out = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
            note(f"participation round {rnd}: sl_aggregate over no peers")
            sl.sl_aggregate([], [], out)
            torch.cuda.synchronize()
            assert_bitwise(out.cpu().numpy(), sum_o, f"round {rnd} empty sum")
            assert not np.signbit(sum_o).any() and not sum_o.any()
        elif rnd == 3:
            rec = torch.stack([pay_g[p] for p in got], dim=1).contiguous()
            sc = torch.stack([sc_g[p] for p in got], dim=1).contiguous()
            note(f"participation round {rnd}: sl_aggregate_apply_interleaved, {len(got)} peer(s)")
            sl.sl_aggregate_apply_interleaved(rec, sc, theta_g)
            theta_o = orc.apply_mean(theta_o, sum_o, len(got))
        elif rnd == 4:
            rec = torch.stack([pay_g[p] for p in got], dim=1).contiguous()
            sc = torch.stack([sc_g[p] for p in got], dim=1).contiguous()
            out = torch.empty(n, dtype=torch.float32, device="cuda")
            note(f"participation round {rnd}: sl_aggregate_interleaved + sl_apply_mean, {len(got)} peers")
            sl.sl_aggregate_interleaved(rec, sc, out)
            sl.sl_apply_mean(theta_g, out, len(got))
            theta_o = orc.apply_mean(theta_o, sum_o, len(got))
        else:
            note(f"participation round {rnd}: sl_aggregate_apply over peers {got}")
            sl.sl_aggregate_apply([pay_g[p] for p in got], [sc_g[p] for p in got], theta_g)
            theta_o = orc.apply_mean(theta_o, sum_o, len(got))
        torch.cuda.synchronize()
        for p in active:
            assert_bitwise(pay_g[p].cpu().numpy(), pay_o[p], f"round {rnd} peer {p} records")
            assert_bitwise(sc_g[p].cpu().numpy(), sc_o[p], f"round {rnd} peer {p} scales")
        for p in range(N):
            assert_bitwise(ef_g[p].cpu().numpy(), ef_o[p], f"round {rnd} peer {p} ef")
        assert_bitwise(theta_g.cpu().numpy(), theta_o, f"round {rnd} theta")


def test_validate_chunk_major_records(orc):
    """Records laid out chunk-major across peers (the layout of
    sl_aggregate_interleaved) are validated by sl_validate_payload over the
    buffer viewed as C * N records: every record is checked on its own, so the
    flags come back chunk-major, flag [c, p] for peer p's record of chunk c.
    24 peers of a ragged 1000 records with planted defects, against the
    oracle's per-peer flags."""
    sl = require_gpu()
    N, C = 24, 1000
    payloads, scales = defective_peers(orc, N, C, 77)
    rec = np.ascontiguousarray(np.stack(payloads, axis=1))       # [C, N, 112]
    sc = np.ascontiguousarray(np.stack(scales, axis=1))          # [C, N]
    want = np.stack([orc.validate(payloads[p], scales[p])[1] for p in range(N)], axis=1)
    assert (want != 0).sum() > 0
    flags = torch.full((C * N,), 255, dtype=torch.uint8, device="cuda")
    note("sl_validate_payload over chunk-major records, 24 peers x 1000")
    sl.sl_validate_payload(torch.from_numpy(rec.reshape(C * N, 112)).cuda(),
                           torch.from_numpy(sc.reshape(C * N)).cuda(), flags)
    torch.cuda.synchronize()
    assert_bitwise(flags.cpu().numpy().reshape(C, N), want, "chunk-major flags")


def check_peer_stats_interleaved(sl, orc, payloads, scales, with_flags=True):
    """sl_peer_stats_interleaved on the peers' records laid out chunk-major,
    against the oracle's per-peer statistics and flags."""
    N, C = len(payloads), scales[0].size if payloads else 0
    rec = np.ascontiguousarray(np.stack(payloads, axis=1)) if N else np.zeros((C, 0, 112), np.uint8)
    sc = np.ascontiguousarray(np.stack(scales, axis=1)) if N else np.zeros((C, 0), np.float32)
    counts = torch.full((N, 4), -1, dtype=torch.int64, device="cuda")
    smax = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    flags = torch.full((N, C), 255, dtype=torch.uint8, device="cuda") if with_flags else None
    note(f"sl_peer_stats_interleaved {N} peers x {C} records, flags={with_flags}")
    sl.sl_peer_stats_interleaved(torch.from_numpy(rec).cuda(), torch.from_numpy(sc).cuda(), counts, smax, flags=flags)
    torch.cuda.synchronize()
    got_c, got_m = counts.cpu().numpy(), smax.cpu().numpy()
    for p in range(N):
        wc, wm = orc.peer_stats(payloads[p], scales[p])
        assert got_c[p].tolist() == wc.tolist(), f"counts of peer {p}"
        assert_bitwise(got_m[p:p + 1], np.float32([wm]), f"scale_max of peer {p}")
        if with_flags:
            assert_bitwise(flags[p].cpu().numpy(), orc.validate(payloads[p], scales[p])[1], f"flags of peer {p}")


def test_peer_stats_chunk_major_records(orc):
    """sl_peer_stats_interleaved: the same statistics and flags as sl_peer_stats
    for the peers' records laid out chunk-major (24 peers x 1000 records with
    planted defects, with and without flags), then one record, ragged counts
    and the most peers."""
    sl = require_gpu()
    payloads, scales = defective_peers(orc, 24, 1000, 17)
    check_peer_stats_interleaved(sl, orc, payloads, scales, with_flags=True)
    check_peer_stats_interleaved(sl, orc, payloads, scales, with_flags=False)
    for N, C in ((1, 1), (3, 63), (128, 257)):
        p_, s_ = defective_peers(orc, N, C, 100 + N)
        check_peer_stats_interleaved(sl, orc, p_, s_, with_flags=True)


@pytest.mark.parametrize("N,C", [(85, 77), (100, 333), (24, 7687), (1, 70000), (128, 2049), (24, 57344)])
def test_peer_stats_chunk_major_block_edges(orc, N, C):
    """sl_peer_stats_interleaved where a workgroup's block of whole chunks
    leaves lanes idle (85 and 100 peers: 255 and 200 of 256 lanes), where a
    workgroup takes several blocks and the last workgroup a partial one
    (24 x 7687, 1 x 70000, 128 x 2049), and at the full 8192 x 28672 shape
    with 24 peers (eleven or twelve blocks per workgroup, as the bench times
    it), against the oracle."""
    sl = require_gpu()
    payloads, scales = defective_peers(orc, N, C, 300 + N)
    check_peer_stats_interleaved(sl, orc, payloads, scales, with_flags=True)


def test_peer_stats_chunk_major_repeated_calls(orc):
    """Consecutive sl_peer_stats_interleaved calls, each of which must start
    from zero totals (the previous call leaves them so), with sl_peer_stats
    (whose part of the same scratch allocation is separate) in between, then a
    call with no records: zero counts and a +0 scale maximum."""
    sl = require_gpu()
    a = defective_peers(orc, 24, 1000, 41)
    b = defective_peers(orc, 5, 300, 42)
    check_peer_stats_interleaved(sl, orc, *a, with_flags=True)
    check_peer_stats_interleaved(sl, orc, *b, with_flags=False)
    pays = [torch.from_numpy(pl).cuda() for pl in a[0]]
    scs = [torch.from_numpy(sc).cuda() for sc in a[1]]
    counts = torch.full((24, 4), -1, dtype=torch.int64, device="cuda")
    smax = torch.full((24,), -1.0, dtype=torch.float32, device="cuda")
    note("sl_peer_stats 24 x 1000 between chunk-major calls")
    sl.sl_peer_stats(pays, scs, counts, smax)
    torch.cuda.synchronize()
    for p in range(24):
        wc, _ = orc.peer_stats(a[0][p], a[1][p])
        assert counts[p].cpu().tolist() == wc.tolist(), f"sl_peer_stats counts of peer {p}"
    check_peer_stats_interleaved(sl, orc, *a, with_flags=True)
    counts = torch.full((3, 4), -1, dtype=torch.int64, device="cuda")
    smax = torch.full((3,), -1.0, dtype=torch.float32, device="cuda")
    note("sl_peer_stats_interleaved 3 peers x 0 records")
    sl.sl_peer_stats_interleaved(torch.empty((0, 3, 112), dtype=torch.uint8, device="cuda"),
                                 torch.empty((0, 3), dtype=torch.float32, device="cuda"), counts, smax)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [[0, 0, 0, 0]] * 3
    assert_bitwise(smax.cpu().numpy(), np.zeros(3, np.float32), "scale_max with no records")
    check_peer_stats_interleaved(sl, orc, *b, with_flags=True)


@pytest.mark.parametrize("N,C", [(24, 777), (81, 131)])
def test_repeated_calls_are_bit_identical(orc, N, C):
    """Every aggregation, validation and statistics entry point, called twice
    on the same inputs, gives bit-identical outputs; the chunk-major entry
    points give the same bits as the per-peer ones on the same records.  The
    aggregates take well-formed records packed by the oracle (the one-chunk
    kernels with three and with nine record loads per lane), validation and
    statistics the same peers with planted defects."""
    sl = require_gpu()
    n = C * 4096

    def layouts(payloads, scales):
        pays = [torch.from_numpy(x).cuda() for x in payloads]
        scs = [torch.from_numpy(x).cuda() for x in scales]
        rec = torch.stack([p.view(C, 112) for p in pays], dim=1).contiguous()
        return sl.PeerSet(pays, scs), rec, torch.stack(scs, dim=1).contiguous()

    clean = [datagen.random_entries_bulk(C, 900 + p) for p in range(N)]
    peers, rec, scm = layouts([orc.pack(i, c) for i, c, _ in clean], [s for _, _, s in clean])
    bad_peers, bad_rec, bad_scm = layouts(*defective_peers(orc, N, C, 900 + N))
    theta0 = torch.randn(n, generator=torch.Generator().manual_seed(N)).cuda()

    def outputs():
        note(f"repeated calls: {N} peers x {C} chunks")
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        sl.sl_aggregate(peers, None, out)
        out_il = torch.empty_like(out)
        sl.sl_aggregate_interleaved(rec, scm, out_il)
        th = theta0.clone()
        sl.sl_aggregate_apply(peers, None, th)
        th_il = theta0.clone()
        sl.sl_aggregate_apply_interleaved(rec, scm, th_il)
        flags = torch.empty((N, C), dtype=torch.uint8, device="cuda")
        sl.sl_validate_payloads(bad_peers, None, flags)
        counts = torch.empty((N, 4), dtype=torch.int64, device="cuda")
        smax = torch.empty(N, dtype=torch.float32, device="cuda")
        sl.sl_peer_stats(bad_peers, None, counts, smax)
        counts_il = torch.empty_like(counts)
        smax_il = torch.empty_like(smax)
        sl.sl_peer_stats_interleaved(bad_rec, bad_scm, counts_il, smax_il)
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in dict(out=out, out_il=out_il, th=th, th_il=th_il, flags=flags,
                                                     counts=counts, smax=smax, counts_il=counts_il,
                                                     smax_il=smax_il).items()}

    a, b = outputs(), outputs()
    for k in a:
        assert_bitwise(a[k], b[k], f"{k}, second call")
    assert_bitwise(a["out"], a["out_il"], "aggregate: per-peer against chunk-major")
    assert_bitwise(a["th"], a["th_il"], "fused update: per-peer against chunk-major")
    assert_bitwise(a["counts"], a["counts_il"], "statistics: per-peer against chunk-major")
    assert_bitwise(a["smax"], a["smax_il"], "scale maxima: per-peer against chunk-major")
