"""Benchmark of the SparseLoCo hot path on one MI355X.

A step is one pass of the path over one synthetic 8192 x 28672 fp32
pseudo-gradient (Student-t(3) values, 20% exactly-zero chunks), as the MLP
workload defines it:
  sl_compress     error feedback + top-64/4096 + 2-bit codes + 12-bit pack
  sl_aggregate    decode and sum 24 peers' records into a dense fp32 update
The outer update theta <- theta - sum / 24 (sl_apply_mean, part of the
decoder-block workload) is timed separately on the same sizes, and the
fused aggregate + update and the other entry points under "next_rows".
Inputs are resident in HBM before timing starts.  Prints one JSON line.

Besides the step, it times the same aggregate over rotating record sets whose
total exceeds the 256 MB last-level cache ("aggregate_cold": every call reads
its records from HBM, as a round's freshly received records are), the
compressor's warmup calls, and the entry points of the NEXT rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --summarize-profile DIR   (rocprofv3 CSV output -> profiles/*.txt)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X published HBM3E bandwidth
N_PEERS = 24
BETA = 0.95
CHUNK = 4096
PAYLOAD = 112                    # record bytes per chunk (12-bit indices, 2-bit codes)
RECORD = PAYLOAD + 4             # payload bytes + fp32 scale per chunk

# Algorithmic bytes per parameter (what the method must move).
BYTES_COMPRESS = 4 + 4 + 4 + RECORD / CHUNK           # read delta, ef; write ef; record
BYTES_AGGREGATE = 4 + N_PEERS * RECORD / CHUNK        # write out; read 24 records
BYTES_APPLY = 4 + 4 + 4                               # read theta, out; write theta

METRIC = "compressed Gparams/s and % of HBM roofline (compress + 24-peer aggregate)"
PROFILE = os.path.join(ROOT, "profiles", "compress_mlp_8192x28672_counters.txt")
CSRC = os.path.join(ROOT, "communication_efficient_distributed_amd", "csrc")
# The compressor's device code: its source and every header it includes.
KERNEL_SOURCES = [os.path.join(CSRC, f) for f in ("compress.hip", "wave.h", "residency.h", "internal.h")] + \
    [os.path.join(ROOT, "include", "sparseloco.h")]


def code_digest(paths) -> str:
    """SHA-256 (16 hex digits) of the given C++ sources with comments removed
    and whitespace collapsed: a comment edit leaves it unchanged, a code edit
    does not."""
    h = hashlib.sha256()
    for path in paths:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def traffic_from_profile(n_params: int):
    """HBM bytes per compress launch from the committed counter summary, or None
    if there is none or it was taken on different compressor code."""
    if not os.path.exists(PROFILE):
        return None
    txt = open(PROFILE).read()
    m = re.search(r"compress_code_sha256_16:\s*([0-9a-f]{16})", txt)
    if not m or m.group(1) != code_digest(KERNEL_SOURCES):
        return None
    f = re.search(r"compress_hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    p = re.search(r"params_per_launch:\s*(\d+)", txt)
    if not f or not p or int(p.group(1)) != n_params:
        return None
    return float(f.group(1))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # After the GPU idles, the first ~25 compressor calls run up to 30% slower
    # while the device settles under load.  Setup ends with the peers'
    # compressions, leading straight into the warmup; 30 warmup steps (about
    # 20 ms) add margin.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip timing the entry points beyond the three-step path")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip timing compress and aggregate at the other workload shapes")
    ap.add_argument("--cpu-sample-chunks", type=int, default=57344)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a torch copy of 1 GiB (for counter calibration)")
    ap.add_argument("--cold-sets", type=int, default=4,
                    help="independent 24-peer record sets the cold aggregate rotates through")
    ap.add_argument("--workload-shapes", default="small_1m,attn_8192x8192,decoder_block,flat_16b,mlp_many_peers",
                    help="comma-separated shapes the workloads section times")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="write profiles/*.txt from the rocprofv3 CSV output under DIR and exit")
    ap.add_argument("--progress", action="store_true",
                    help="print a line to stderr as each stage of the run ends")
    ap.add_argument("--profile-out", metavar="DIR", default=os.path.join(ROOT, "profiles"),
                    help="where --summarize-profile writes (default: profiles/)")
    return ap.parse_args()


def stage(args, what):
    if args.progress:
        print(f"[bench] {time.strftime('%H:%M:%S')} {what}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.profile_out)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the compressor and aggregator are chunk-local, "
              "and a multi-GPU run would shard chunk ranges and all-gather the records, which "
              "is not implemented here; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import communication_efficient_distributed_amd as sl
    from communication_efficient_distributed_amd import datagen

    sl.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # Three device copies of exactly 1 GiB, before any other kernel of the
        # run, so that a counter summary finds them as the run's first dispatches.
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    W = datagen.MLP_8192x28672
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK

    # Resident inputs.
    delta = datagen.student_t3(n, W, 0, 0, dev)
    ef = torch.zeros(n, dtype=torch.float32, device=dev)
    payload = torch.empty((C, 112), dtype=torch.uint8, device=dev)
    scales = torch.empty(C, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    theta = datagen.theta0(n, W, dev)
    # Host copy for the CPU baseline, taken before the peer records are made
    # so that the GPU goes from that work straight into the warmup steps.
    ef0_host = ef.cpu().numpy()
    peer_p, peer_s = [], []
    scratch_ef = torch.zeros(n, dtype=torch.float32, device=dev)
    for p in range(1, N_PEERS + 1):
        d = datagen.student_t3(n, W, p, 0, dev)
        scratch_ef.zero_()
        pl, s = sl.compress(d, scratch_ef, BETA)
        peer_p.append(pl)
        peer_s.append(s)
        del d
    # Further independent record sets (peers 25, 26, ...) for the cold
    # aggregate: 4 sets x 160 MB exceed the last-level cache, so each call's
    # records come from HBM.
    cold_sets = [sl.PeerSet(peer_p, peer_s)]
    cold_lists = [(peer_p, peer_s)]
    for k in range(1, max(1, args.cold_sets)):
        cp, cs = [], []
        for p in range(k * N_PEERS + 1, (k + 1) * N_PEERS + 1):
            d = datagen.student_t3(n, W, p, 0, dev)
            scratch_ef.zero_()
            pl, s = sl.compress(d, scratch_ef, BETA)
            cp.append(pl)
            cs.append(s)
            del d
        cold_sets.append(sl.PeerSet(cp, cs))
        cold_lists.append((cp, cs))
    del scratch_ef
    torch.cuda.synchronize()
    stage(args, f"setup: {len(cold_sets)} record sets of {N_PEERS} peers")

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        sl.sl_compress(delta, ef, BETA, payload, scales)
        if ev is not None:
            ev[1].record(stream)
        sl.sl_aggregate(peer_p, peer_s, out)
        if ev is not None:
            ev[2].record(stream)

    # Warmup steps, each compress call timed, so the line shows whether the
    # timed steps start in the steady state.
    wevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.warmup)]
    for k in range(args.warmup):
        step(wevs[k])
    torch.cuda.synchronize()
    t_warm = [e[0].elapsed_time(e[1]) for e in wevs]
    stage(args, f"{args.warmup} warmup steps")

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    t_c = [e[0].elapsed_time(e[1]) for e in evs]
    t_a = [e[1].elapsed_time(e[2]) for e in evs]
    span_ms = evs[0][0].elapsed_time(evs[-1][2])
    ms_per_step = span_ms / K

    # The same step with the aggregate's records read from HBM: each step
    # takes the next of the rotating record sets.
    def step_cold(k, ev):
        ev[0].record(stream)
        sl.sl_compress(delta, ef, BETA, payload, scales)
        ev[1].record(stream)
        sl.sl_aggregate(cold_sets[k % len(cold_sets)], None, out)
        ev[2].record(stream)

    for k in range(len(cold_sets)):
        step_cold(k, [torch.cuda.Event(enable_timing=True) for _ in range(3)])
    cevs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for k in range(K):
        step_cold(k, cevs[k])
    torch.cuda.synchronize()
    t_cc = [e[0].elapsed_time(e[1]) for e in cevs]
    t_ac = [e[1].elapsed_time(e[2]) for e in cevs]
    ms_per_step_cold = cevs[0][0].elapsed_time(cevs[-1][2]) / K

    # Once more with the same record sets laid out chunk-major across peers
    # (sl_aggregate_interleaved), copied into that layout here.
    il_sets = [interleaved_records(torch, p_, s_) for p_, s_ in cold_lists]

    def step_cold_il(k, ev):
        ev[0].record(stream)
        sl.sl_compress(delta, ef, BETA, payload, scales)
        ev[1].record(stream)
        r_, s_ = il_sets[k % len(il_sets)]
        sl.sl_aggregate_interleaved(r_, s_, out)
        ev[2].record(stream)

    for k in range(len(il_sets)):
        step_cold_il(k, [torch.cuda.Event(enable_timing=True) for _ in range(3)])
    ievs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    for k in range(K):
        step_cold_il(k, ievs[k])
    torch.cuda.synchronize()
    t_ai = [e[1].elapsed_time(e[2]) for e in ievs]
    t_ci = [e[0].elapsed_time(e[1]) for e in ievs]
    ms_per_step_cold_il = ievs[0][0].elapsed_time(ievs[-1][2]) / K
    del il_sets
    stage(args, f"{K} timed steps, cached and cold records (per peer and chunk-major)")

    # The outer update, outside the step: same K, one event pair per call.
    for _ in range(args.warmup):
        sl.sl_apply_mean(theta, out, N_PEERS)
    mevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for k in range(K):
        mevs[k][0].record(stream)
        sl.sl_apply_mean(theta, out, N_PEERS)
        mevs[k][1].record(stream)
    torch.cuda.synchronize()
    t_m = [e[0].elapsed_time(e[1]) for e in mevs]
    avg = lambda xs: float(sum(xs) / len(xs))
    tc, ta, tm = avg(t_c), avg(t_a), avg(t_m)

    def kstats(t_ms, bpp, samples=None):
        gps = n / (t_ms * 1e-3) / 1e9
        gbs = bpp * n / (t_ms * 1e-3) / 1e9
        r = {"ms": round(t_ms, 5), "gparams_per_s": round(gps, 2), "gb_per_s": round(gbs, 1),
             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_param": round(bpp, 4)}
        if samples:
            r["ms_median"] = round(statistics.median(samples), 5)
            r["ms_min"] = round(min(samples), 5)
        return r

    value = n / (ms_per_step * 1e-3) / 1e9
    comp = kstats(tc, BYTES_COMPRESS, t_c)
    comp["first_timed_ms"] = round(t_c[0], 5)
    comp["last_timed_ms"] = round(t_c[-1], 5)
    agg_cold = kstats(avg(t_ac), BYTES_AGGREGATE, t_ac)
    agg_cold.update({"record_sets": len(cold_sets),
                     "record_bytes_per_set": N_PEERS * C * RECORD,
                     "note": "each call aggregates the next of the record sets, whose total exceeds the "
                             "256 MB last-level cache: the records come from HBM"})
    step_cold_stats = kstats(ms_per_step_cold, BYTES_COMPRESS + BYTES_AGGREGATE)
    step_cold_stats["compress_ms"] = round(avg(t_cc), 5)
    agg_cold_il = kstats(avg(t_ai), BYTES_AGGREGATE, t_ai)
    agg_cold_il.update({"record_sets": len(cold_sets),
                        "note": "the same record sets laid out chunk-major across peers "
                                "(sl_aggregate_interleaved): one contiguous span of records per chunk"})
    step_cold_il_stats = kstats(ms_per_step_cold_il, BYTES_COMPRESS + BYTES_AGGREGATE)
    step_cold_il_stats["compress_ms"] = round(avg(t_ci), 5)
    traffic = traffic_from_profile(n)
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "mlp_8192x28672_student_t3_zero20",
            "params": n,
            "chunks": C,
            "peers": N_PEERS,
            "beta": BETA,
            "step": "sl_compress + sl_aggregate(24 peers)",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "compress_kernel",
            "achieved": comp["gb_per_s"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": comp["hbm_frac"],
            "traffic": traffic,
            "algorithmic_bytes_per_launch": round(BYTES_COMPRESS * n),
        },
        "kernels": {
            "compress": comp,
            "aggregate": kstats(ta, BYTES_AGGREGATE, t_a),
            "apply_mean": kstats(tm, BYTES_APPLY, t_m),
            "compress_plus_aggregate": kstats(tc + ta, BYTES_COMPRESS + BYTES_AGGREGATE),
            "aggregate_cold": agg_cold,
            "step_cold": step_cold_stats,
            "aggregate_cold_interleaved": agg_cold_il,
            "step_cold_interleaved": step_cold_il_stats,
        },
        "warmup_trace": {
            "steps": args.warmup,
            "compress_ms_first": round(t_warm[0], 5) if t_warm else None,
            "compress_ms_last": round(t_warm[-1], 5) if t_warm else None,
            "compress_ms_max": round(max(t_warm), 5) if t_warm else None,
            "timed_compress_ms_first": round(t_c[0], 5),
            "timed_compress_ms_last": round(t_c[-1], 5),
            "timed_compress_ms_max": round(max(t_c), 5),
        },
        "wall_s_timed": round(wall, 4),
        "device": device_props(torch, dev),
    }

    if not args.no_next_rows:
        result["next_rows"] = next_rows(sl, delta, ef, payload, scales, peer_p, peer_s, theta, n,
                                        stream, kstats)
        stage(args, "next rows")

    if not args.no_workloads:
        del out, cold_sets
        result["workloads"] = workloads(sl, dev, args.workload_shapes.split(","), lambda w: stage(args, w))

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, delta, ef0_host, peer_p, peer_s, theta, n)
        stage(args, "cpu baseline")

    print(json.dumps(result), flush=True)


# Calls per next_rows row timed with add_back_to_back(timed(...)): NEXT_WARM
# warm-up calls and NEXT_REPS timed ones, then one warm-up and NEXT_REPS calls
# back to back (the trace summary counts dispatches with these).
NEXT_REPS = 20
NEXT_WARM = 3
NEXT_ROW_CALLS = NEXT_WARM + NEXT_REPS + 1 + NEXT_REPS


def next_rows(sl, delta, ef, payload, scales, peer_p, peer_s, theta, n, stream, kstats, reps=NEXT_REPS):
    """The entry points beyond the compress + aggregate step, on the same
    workload (not part of `value`): fused aggregate + outer update, compression
    straight from pre/post weights, error feedback in pinned host memory, record
    validation for one peer and for all 24 in one launch."""
    import torch

    def timed(fn, k=reps, warm=NEXT_WARM):
        # Each call is timed on its own, queued behind a short spin kernel so
        # that the host-side argument marshalling (pointer tables of 24 peers)
        # is done before the GPU reaches it: the events see the kernel only.
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(k)]
        for e0, e1 in evs:
            torch.cuda._sleep(200000)
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ts = [e0.elapsed_time(e1) for e0, e1 in evs]
        timed.samples = ts
        return sum(ts) / k

    def back_to_back(fn, k=reps):
        # k calls between one pair of events, queued behind a spin kernel: for
        # kernels of a few tens of microseconds the per-call events above add
        # a few microseconds each; this is the per-call rate when calls follow
        # one another (arguments prepared once, as PeerSet does).
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000000)
        e0.record(stream)
        for _ in range(k):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / k

    def add_back_to_back(st, fn, bpp):
        t2 = back_to_back(fn)
        b2 = kstats(t2, bpp)
        st["ms_back_to_back"] = b2["ms"]
        st["hbm_frac_back_to_back"] = b2["hbm_frac"]
        return st

    res = {}
    # The 24-peer rows take the peers as a PeerSet: its pointer tables are built
    # once, so no host-side marshalling can hold a call back.
    peers = sl.PeerSet(peer_p, peer_s)
    t = timed(lambda: sl.sl_aggregate_apply(peers, None, theta))
    res["aggregate_apply_fused"] = kstats(t, 8 + N_PEERS * RECORD / CHUNK, timed.samples)
    pre = theta
    post = theta - delta               # so that pre - post carries the workload's values
    t = timed(lambda: sl.sl_compress_weights(pre, post, ef, BETA, payload, scales))
    res["compress_weights"] = kstats(t, 16 + RECORD / CHUNK, timed.samples)
    del post
    ef_host = torch.zeros(n, dtype=torch.float32, pin_memory=True)
    t = timed(lambda: sl.sl_compress_host_ef(delta, ef_host, BETA, payload, scales), k=5, warm=1)
    st = kstats(t, 4 + RECORD / CHUNK)       # HBM bytes only; ef moves over the host link
    link = 8 * n / (t * 1e-3) / 1e9          # ef read and written over the host link
    dma = host_link_dma(torch, ef_host, delta.device, stream)
    st["host_link_gb_per_s"] = round(link, 1)
    st["host_link_peak_gb_per_s"] = dma["bidirectional_gb_per_s"]
    st["host_link_frac"] = round(link / dma["bidirectional_gb_per_s"], 4)
    st["host_link_dma"] = dma
    st["host_link_note"] = ("peak = concurrent host-to-device and device-to-host copies of the same "
                            "4 bytes per parameter each way, measured in this run; PCIe 5.0 x16 "
                            "signals 64 GB/s per direction")
    res["compress_host_ef"] = st
    del ef_host
    flags = torch.empty(n // CHUNK, dtype=torch.uint8, device=delta.device)
    one = lambda: sl.sl_validate_payload(peer_p[0], peer_s[0], flags)
    t = timed(one)
    res["validate_one_peer"] = add_back_to_back(kstats(t, (RECORD + 1) / CHUNK, timed.samples), one,
                                                (RECORD + 1) / CHUNK)
    flags_all = torch.empty((N_PEERS, n // CHUNK), dtype=torch.uint8, device=delta.device)
    bpp = N_PEERS * (RECORD + 1) / CHUNK
    val = lambda: sl.sl_validate_payloads(peers, None, flags_all)
    t = timed(val)
    res["validate_24_peers"] = add_back_to_back(kstats(t, bpp, timed.samples), val, bpp)
    counts = torch.empty((N_PEERS, 4), dtype=torch.int64, device=delta.device)
    smax = torch.empty(N_PEERS, dtype=torch.float32, device=delta.device)
    stats = lambda: sl.sl_peer_stats(peers, None, counts, smax, flags=flags_all)
    t = timed(stats)
    res["peer_stats_24_peers"] = add_back_to_back(kstats(t, bpp, timed.samples), stats, bpp)
    # the same statistics on the records laid out chunk-major across peers
    il_r, il_s = interleaved_records(torch, peer_p, peer_s)
    stats_il = lambda: sl.sl_peer_stats_interleaved(il_r, il_s, counts, smax, flags=flags_all)
    t = timed(stats_il)
    res["peer_stats_24_peers_chunk_major"] = add_back_to_back(kstats(t, bpp, timed.samples), stats_il, bpp)
    # The rows above re-read one set of records, which then sits in the
    # last-level cache.  The same passes with records from HBM: four sets
    # (about 640 MB in each layout), taken in turn.
    pp_sets = [peers] + [sl.PeerSet([x.clone() for x in peer_p], [x.clone() for x in peer_s]) for _ in range(3)]
    il_sets = [(il_r, il_s)] + [(il_r.clone(), il_s.clone()) for _ in range(3)]
    turn = [0]

    def rotate(sets):
        turn[0] += 1
        return sets[turn[0] % len(sets)]

    cold = {
        "validate_24_peers_cold": lambda: sl.sl_validate_payloads(rotate(pp_sets), None, flags_all),
        "peer_stats_24_peers_cold": lambda: sl.sl_peer_stats(rotate(pp_sets), None, counts, smax, flags=flags_all),
        "peer_stats_24_peers_chunk_major_cold": lambda: sl.sl_peer_stats_interleaved(*rotate(il_sets), counts, smax,
                                                                                     flags=flags_all),
    }
    for name, fn in cold.items():
        t = timed(fn)
        res[name] = add_back_to_back(kstats(t, bpp, timed.samples), fn, bpp)
        res[name]["record_sets"] = len(pp_sets)
    # A round's receive path on records from HBM: the statistics pass (with the
    # validation flags) and then the aggregate of the same records, per-peer and
    # chunk-major.  The second pass may find records the first left cached.
    dense = torch.empty(n, dtype=torch.float32, device=delta.device)

    def receive(sets, stats_fn, agg_fn):
        def fn():
            st = rotate(sets)
            stats_fn(st)
            agg_fn(st)
        return fn

    bpr = bpp + 4 + N_PEERS * RECORD / CHUNK
    for name, fn in (
            ("receive_24_peers_cold", receive(
                pp_sets, lambda st: sl.sl_peer_stats(st, None, counts, smax, flags=flags_all),
                lambda st: sl.sl_aggregate(st, None, dense))),
            ("receive_24_peers_chunk_major_cold", receive(
                il_sets, lambda st: sl.sl_peer_stats_interleaved(*st, counts, smax, flags=flags_all),
                lambda st: sl.sl_aggregate_interleaved(*st, dense)))):
        t = timed(fn)
        res[name] = add_back_to_back(kstats(t, bpr, timed.samples), fn, bpr)
        res[name].update({"record_sets": len(pp_sets),
                          "note": "per-peer statistics with validation flags, then the 24-peer aggregate of "
                                  "the same records; bytes are the two passes' algorithmic bytes"})
    del il_r, il_s, il_sets, pp_sets, dense
    # The 24-peer aggregate with records from HBM, the peers' records and
    # scales packed as a receiver would allocate its receive buffers: one
    # [N, C, 112] record buffer and one [N, C] scale buffer per set (same
    # per-peer entry point), four sets taken in turn.
    C_ = n // CHUNK
    packed = []
    for k in range(4):
        rec = torch.empty((N_PEERS, C_, PAYLOAD), dtype=torch.uint8, device=delta.device)
        sc = torch.empty((N_PEERS, C_), dtype=torch.float32, device=delta.device)
        for q in range(N_PEERS):
            rec[q].copy_(peer_p[q].view(C_, PAYLOAD))
            sc[q].copy_(peer_s[q])
        packed.append((rec, sc, sl.PeerSet([rec[q] for q in range(N_PEERS)], [sc[q] for q in range(N_PEERS)])))
    dense = torch.empty(n, dtype=torch.float32, device=delta.device)
    agg_p = lambda: sl.sl_aggregate(rotate([x[2] for x in packed]), None, dense)
    bpa = 4 + N_PEERS * RECORD / CHUNK
    t = timed(agg_p)
    res["aggregate_cold_packed"] = add_back_to_back(kstats(t, bpa, timed.samples), agg_p, bpa)
    res["aggregate_cold_packed"].update({"record_sets": len(packed),
                                         "note": "sl_aggregate on records from HBM, each set's records in one "
                                                 "[N, C, 112] buffer and its scales in one [N, C] buffer"})
    del packed, dense
    res["small_round_1m"] = small_round(sl, delta.device)
    return res


def host_link_dma(torch, host_a, dev, stream, reps=3):
    """Rates of the host link as the copy engines see it, on the bytes the
    host-resident EF round moves: host-to-device and device-to-host copies of
    the same size alone, then both at once on two streams (pinned memory)."""
    nbytes = host_a.numel() * host_a.element_size()
    host_b = torch.empty_like(host_a, pin_memory=True)
    d_a = torch.empty(host_a.numel(), dtype=host_a.dtype, device=dev)
    d_b = torch.empty_like(d_a)
    s1, s2 = torch.cuda.Stream(device=dev), torch.cuda.Stream(device=dev)

    def run(h2d, d2h):
        best = None
        for _ in range(reps):
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            s1.wait_stream(stream)
            s2.wait_stream(stream)
            if h2d:
                with torch.cuda.stream(s1):
                    d_a.copy_(host_a, non_blocking=True)
            if d2h:
                with torch.cuda.stream(s2):
                    host_b.copy_(d_b, non_blocking=True)
            stream.wait_stream(s1)
            stream.wait_stream(s2)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return round((int(h2d) + int(d2h)) * nbytes / (best * 1e-3) / 1e9, 1)

    r = {"bytes_each_way": nbytes, "h2d_gb_per_s": run(True, False), "d2h_gb_per_s": run(False, True),
         "bidirectional_gb_per_s": run(True, True)}
    del host_b, d_a, d_b
    return r


def interleaved_records(torch, payloads, scales):
    """The peers' per-peer records and scales copied into the chunk-major layout
    of sl_aggregate_interleaved: uint8 [C, P, 112] and float32 [C, P]."""
    C, P = scales[0].numel(), len(payloads)
    rec = torch.empty((C, P, PAYLOAD), dtype=torch.uint8, device=scales[0].device)
    sc = torch.empty((C, P), dtype=torch.float32, device=scales[0].device)
    for k in range(P):
        rec[:, k, :].copy_(payloads[k].view(C, PAYLOAD))
        sc[:, k].copy_(scales[k])
    return rec, sc


def timed_calls(torch, stream, fn, k=20, warm=3):
    """Mean and per-call times (ms) of fn, each call timed on its own behind a
    short spin kernel, so that host-side argument marshalling (pointer tables
    of 24 peers) is finished before the GPU reaches it: the events see the
    kernels only."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(k)]
    for e0, e1 in evs:
        torch.cuda._sleep(200000)
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    t = [e0.elapsed_time(e1) for e0, e1 in evs]
    return sum(t) / k, t


def workloads(sl, dev, shapes, done=lambda what: None, reps=10):
    """Compress and the 24-peer aggregate at the other workload shapes: the
    1,048,576-parameter case (cache-resident), one 8192 x 8192 projection, one
    decoder block (also the fused aggregate + update and apply_mean), and the
    16e9-parameter flat span (skipped when the device lacks the 203 GB it
    needs).  Every buffer is resident; 24 peers' records come from compressing
    24 independently seeded pseudo-gradients from ef = 0."""
    import torch

    from communication_efficient_distributed_amd import datagen

    stream = torch.cuda.current_stream(dev)

    def st(n, t_ms, bpp, samples):
        gbs = bpp * n / (t_ms * 1e-3) / 1e9
        return {"ms": round(t_ms, 5), "ms_min": round(min(samples), 5),
                "gparams_per_s": round(n / (t_ms * 1e-3) / 1e9, 2), "gb_per_s": round(gbs, 1),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_param": round(bpp, 4)}

    res = {}
    for name, W in (("small_1m", datagen.SMALL_1M), ("attn_8192x8192", datagen.ATTN_8192),
                    ("decoder_block", datagen.DECODER_BLOCK), ("flat_16b", datagen.FLAT_16B)):
        if name not in shapes:
            continue
        n = datagen.WORKLOAD_PARAMS[W]
        C = n // CHUNK
        need = 3 * 4 * n + N_PEERS * C * RECORD + (4 << 30)
        free, _ = torch.cuda.mem_get_info(dev)
        if free < need:
            res[name] = {"params": n, "skipped": f"needs {need / 1e9:.0f} GB of free device memory, "
                                                 f"{free / 1e9:.0f} GB free"}
            continue
        a = torch.empty(n, dtype=torch.float32, device=dev)
        ef = torch.empty(n, dtype=torch.float32, device=dev)
        pp, ps = [], []
        for p in range(1, N_PEERS + 1):
            datagen.fill_lognormal_(a, W, p, 0)
            ef.zero_()
            pl, sc = sl.compress(a, ef, BETA)
            pp.append(pl)
            ps.append(sc)
        peers = sl.PeerSet(pp, ps)
        datagen.fill_lognormal_(a, W, 0, 0)
        ef.zero_()
        payload = torch.empty((C, 112), dtype=torch.uint8, device=dev)
        scales = torch.empty(C, dtype=torch.float32, device=dev)
        out = torch.empty(n, dtype=torch.float32, device=dev)
        r = {"params": n, "chunks": C, "peers": N_PEERS}
        t, ts = timed_calls(torch, stream, lambda: sl.sl_compress(a, ef, BETA, payload, scales), k=reps)
        r["compress"] = st(n, t, BYTES_COMPRESS, ts)
        t, ts = timed_calls(torch, stream, lambda: sl.sl_aggregate(peers, None, out), k=reps)
        r["aggregate"] = st(n, t, BYTES_AGGREGATE, ts)
        if W == datagen.FLAT_16B:
            # The same records laid out chunk-major, when the device has room
            # for a second copy of them (10.9 GB).
            free, _ = torch.cuda.mem_get_info(dev)
            if free > N_PEERS * C * RECORD + (2 << 30):
                il_r, il_s = interleaved_records(torch, pp, ps)
                t, ts = timed_calls(torch, stream, lambda: sl.sl_aggregate_interleaved(il_r, il_s, out), k=reps)
                r["aggregate_interleaved"] = st(n, t, BYTES_AGGREGATE, ts)
                del il_r, il_s
        if W == datagen.DECODER_BLOCK:
            # One 581 MB record set read call after call stays partly in the
            # 256 MB last-level cache; a second set, alternated with the first,
            # makes every call read its records from HBM.
            pp2, ps2 = [], []
            for p in range(N_PEERS + 1, 2 * N_PEERS + 1):
                datagen.fill_lognormal_(a, W, p, 0)
                ef.zero_()
                pl, sc = sl.compress(a, ef, BETA)
                pp2.append(pl)
                ps2.append(sc)
            sets = [peers, sl.PeerSet(pp2, ps2)]
            turn = [0]

            def cold_call():
                turn[0] += 1
                sl.sl_aggregate(sets[turn[0] % 2], None, out)

            t, ts = timed_calls(torch, stream, cold_call, k=reps)
            r["aggregate_cold"] = dict(st(n, t, BYTES_AGGREGATE, ts), record_sets=2,
                                       note="two 24-peer record sets alternated, each call's records from HBM; "
                                            "'aggregate' re-reads one set, which stays partly cache-resident")
            il = [interleaved_records(torch, pp, ps), interleaved_records(torch, pp2, ps2)]

            def cold_il_call():
                turn[0] += 1
                r_, s_ = il[turn[0] % 2]
                sl.sl_aggregate_interleaved(r_, s_, out)

            t, ts = timed_calls(torch, stream, cold_il_call, k=reps)
            r["aggregate_cold_interleaved"] = dict(st(n, t, BYTES_AGGREGATE, ts), record_sets=2,
                                                   note="the same two sets laid out chunk-major across peers")
            datagen.fill_lognormal_(a, W, 0, 0)
            ef.zero_()
            theta = ef
            theta.copy_(a).mul_(0.02)
            t, ts = timed_calls(torch, stream, lambda: sl.sl_aggregate_apply(peers, None, theta), k=reps)
            r["aggregate_apply_fused"] = st(n, t, 8 + N_PEERS * RECORD / CHUNK, ts)

            def fused_cold():
                turn[0] += 1
                sl.sl_aggregate_apply(sets[turn[0] % 2], None, theta)

            def fused_cold_il():
                turn[0] += 1
                r_, s_ = il[turn[0] % 2]
                sl.sl_aggregate_apply_interleaved(r_, s_, theta)

            t, ts = timed_calls(torch, stream, fused_cold, k=reps)
            r["aggregate_apply_fused_cold"] = dict(st(n, t, 8 + N_PEERS * RECORD / CHUNK, ts), record_sets=2)
            t, ts = timed_calls(torch, stream, fused_cold_il, k=reps)
            r["aggregate_apply_fused_cold_interleaved"] = dict(st(n, t, 8 + N_PEERS * RECORD / CHUNK, ts),
                                                               record_sets=2)
            del sets, pp2, ps2, il
            t, ts = timed_calls(torch, stream, lambda: sl.sl_apply_mean(theta, out, N_PEERS), k=reps)
            r["apply_mean"] = st(n, t, BYTES_APPLY, ts)
        res[name] = r
        done(f"workload {name}")
        del a, ef, out, payload, scales, pp, ps, peers
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    if "mlp_many_peers" in shapes:
        res["mlp_many_peers"] = many_peers(sl, dev, reps)
        done("workload mlp_many_peers")
    return res


MANY_PEERS = (36, 48, 55, 64, 81, 128)


def many_peers(sl, dev, reps):
    """The aggregate at 8192 x 28672 with more peers than the step's 24: 36 to
    128 distinct peers' records (240 to 850 MB per set), each count timed back
    to back over two independent record sets taken in turn, so that every call
    reads its records from HBM (one set re-read would stay partly in the
    256 MB last-level cache)."""
    import torch

    from communication_efficient_distributed_amd import datagen

    W = datagen.MLP_8192x28672
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK
    stream = torch.cuda.current_stream(dev)
    ef = torch.empty(n, dtype=torch.float32, device=dev)
    M = max(MANY_PEERS)
    pp, ps = [], []
    for p in range(1, 2 * M + 1):   # set 0: peers 1..M, set 1: peers M+1..2M
        d = datagen.student_t3(n, W, p, 0, dev)
        ef.zero_()
        x, y = sl.compress(d, ef, BETA)
        pp.append(x)
        ps.append(y)
        del d
    del ef
    out = torch.empty(n, dtype=torch.float32, device=dev)
    res = {"params": n, "chunks": C, "record_sets": 2,
           "note": "per count, two independent record sets taken in turn: every call reads its records from HBM"}
    for P in MANY_PEERS:
        sets = [sl.PeerSet(pp[:P], ps[:P]), sl.PeerSet(pp[M:M + P], ps[M:M + P])]
        for k in range(3):
            sl.sl_aggregate(sets[k % 2], None, out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(reps):
            sl.sl_aggregate(sets[k % 2], None, out)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps
        bpp = 4 + P * RECORD / CHUNK
        gbs = bpp * n / (t * 1e-3) / 1e9
        res[str(P)] = {"ms": round(t, 5), "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                       "bytes_per_param": round(bpp, 4), "record_mb": round(P * C * RECORD / 1e6, 1)}
    # The same records laid out chunk-major across peers (sl_aggregate_interleaved).
    il = {}
    for P in MANY_PEERS:
        ils = [interleaved_records(torch, pp[:P], ps[:P]), interleaved_records(torch, pp[M:M + P], ps[M:M + P])]
        for k in range(3):
            sl.sl_aggregate_interleaved(*ils[k % 2], out)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(reps):
            sl.sl_aggregate_interleaved(*ils[k % 2], out)
        e1.record(stream)
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / reps
        bpp = 4 + P * RECORD / CHUNK
        gbs = bpp * n / (t * 1e-3) / 1e9
        il[str(P)] = {"ms": round(t, 5), "gb_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del ils
    res["interleaved"] = il
    del pp, ps, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def small_round(sl, dev, reps=50):
    """A whole round at the 1,048,576-parameter shape (256 chunks), where
    launches dominate: validate 24 peers, fused aggregate + update, compress.
    Timed eagerly (back to back, as a caller would issue it), eagerly with
    the peers' pointer tables prepared once (PeerSet), and as one HIP graph
    replay."""
    import torch

    from communication_efficient_distributed_amd import datagen

    W = datagen.SMALL_1M
    n = datagen.WORKLOAD_PARAMS[W]
    C = n // CHUNK
    scratch = torch.zeros(n, dtype=torch.float32, device=dev)
    pp, ps = [], []
    for p in range(1, N_PEERS + 1):
        scratch.zero_()
        a, b = sl.compress(datagen.lognormal(n, W, p, 0, dev), scratch, BETA)
        pp.append(a)
        ps.append(b)
    delta = datagen.lognormal(n, W, 0, 0, dev)
    ef = torch.zeros(n, dtype=torch.float32, device=dev)
    theta = datagen.theta0(n, W, dev)
    payload = torch.empty((C, 112), dtype=torch.uint8, device=dev)
    scales = torch.empty(C, dtype=torch.float32, device=dev)
    flags = torch.empty((N_PEERS, C), dtype=torch.uint8, device=dev)

    def round_():
        sl.sl_validate_payloads(pp, ps, flags)
        sl.sl_aggregate_apply(pp, ps, theta)
        sl.sl_compress(delta, ef, BETA, payload, scales)

    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(3):
            round_()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        round_()
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) / reps * 1e3
    peers = sl.PeerSet(pp, ps)                   # pointer tables checked and built once

    def round_peerset():
        sl.sl_validate_payloads(peers, None, flags)
        sl.sl_aggregate_apply(peers, None, theta)
        sl.sl_compress(delta, ef, BETA, payload, scales)

    for _ in range(3):
        round_peerset()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        round_peerset()
    e1.record()
    torch.cuda.synchronize()
    peerset_us = e0.elapsed_time(e1) / reps * 1e3
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) / reps * 1e3
    return {"params": n, "peers": N_PEERS, "kernels_per_round": 3,
            "eager_us_per_round": round(eager_us, 2),
            "eager_peerset_us_per_round": round(peerset_us, 2),
            "graph_us_per_round": round(graph_us, 2)}


def device_props(torch, dev) -> dict:
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None),
            "compute_units": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1)}


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_per_workload(T, sample_chunks=2048):
    """The oracle's compress and 24-peer aggregate rates on a 2048-chunk
    sample of each workload's own distribution (host-generated inputs, peers
    compressed by the oracle from ef = 0), plus the time the whole of each
    workload would take at that rate (extrapolated, per chunk)."""
    import numpy as np

    import oracle
    from communication_efficient_distributed_amd import datagen

    m = sample_chunks * CHUNK
    res = {}
    for name, W in (("small_1m", datagen.SMALL_1M), ("attn_8192", datagen.ATTN_8192),
                    ("mlp_8192x28672", datagen.MLP_8192x28672),
                    ("decoder_block", datagen.DECODER_BLOCK), ("flat_16b", datagen.FLAT_16B)):
        full = datagen.WORKLOAD_PARAMS[W]
        k = min(m, full)
        d = datagen.workload_delta(W, 0, 0, n=k).numpy()
        peers = [oracle.compress(datagen.workload_delta(W, p, 0, n=k).numpy(), np.zeros(k, np.float32),
                                 beta=BETA, nthreads=T)[:2] for p in range(1, 4)]
        pp = [peers[i % 3][0] for i in range(N_PEERS)]
        ps = [peers[i % 3][1] for i in range(N_PEERS)]
        t0 = time.perf_counter()
        oracle.compress(d, np.zeros(k, np.float32), beta=BETA, nthreads=T)
        t1 = time.perf_counter()
        oracle.aggregate(pp, ps, k, nthreads=T)
        t2 = time.perf_counter()
        res[name] = {"sample_params": k, "compress_gparams_per_s": round(k / (t1 - t0) / 1e9, 5),
                     "aggregate_gparams_per_s": round(k / (t2 - t1) / 1e9, 5),
                     "full_workload_seconds_extrapolated": round(full / k * (t2 - t0), 2)}
    return res


def cpu_baseline(args, delta, ef0_host, peer_p, peer_s, theta, n):
    """The CPU oracle on the first S chunks of the same workload, the same step
    (compress + 24-peer aggregate), on up to 16 host threads (and on one
    thread for a smaller sample).
    Reported as a baseline, not a target."""
    import numpy as np

    import oracle

    def run(S, T):
        m = S * CHUNK
        d = delta[:m].cpu().numpy()
        e = ef0_host[:m].copy()
        pp = [p[:S].cpu().numpy() for p in peer_p]
        ps = [s[:S].cpu().numpy() for s in peer_s]
        t0 = time.perf_counter()
        oracle.compress(d, e, beta=BETA, nthreads=T, inplace=True)
        t1 = time.perf_counter()
        oracle.aggregate(pp, ps, m, nthreads=T)
        t2 = time.perf_counter()
        return m, t2 - t0, t1 - t0, t2 - t1

    S = min(args.cpu_sample_chunks, n // CHUNK)
    T = max(1, min(16, os.cpu_count() or 1))
    m, dt, dc, da = run(S, T)
    S1 = min(4096, S)
    m1, dt1, dc1, da1 = run(S1, 1)
    g = lambda params, sec: round(params / sec / 1e9, 5)
    per_workload = oracle_per_workload(T)
    return {"value": g(m, dt), "unit": "Gparams/s", "cores": T, "kind": "oracle",
            "per_workload_sample": per_workload,
            "sample": f"first {S} chunks ({m} params) of the same workload: compress + "
                      f"aggregate {N_PEERS} peers, {dt:.2f} s wall on {T} threads",
            "compress_gparams_per_s": g(m, dc), "aggregate_gparams_per_s": g(m, da),
            "single_thread": {"value": g(m1, dt1), "unit": "Gparams/s",
                              "compress_gparams_per_s": g(m1, dc1),
                              "aggregate_gparams_per_s": g(m1, da1),
                              "sample": f"first {S1} chunks, {dt1:.2f} s wall on 1 thread"},
            "host_cpu": host_cpu_model(), "host_cpus_visible": os.cpu_count()}



# ---------------------------------------------------------------------------
# rocprofv3 summaries.  `python bench.py --summarize-profile DIR` turns the CSV
# output of PROFILE_COMMANDS (run with DIR in place of <dir>) into the text
# files under profiles/; every figure there, and the traffic figure that the
# roofline object reads back, comes from this code.

PROFILE_ARGS = ("--no-cpu-baseline --copy-calibration --steps 3 --warmup 1 --progress "
                "--workload-shapes decoder_block,mlp_many_peers")
TRACE_ARGS = "--no-cpu-baseline --progress"
COUNTER_PASSES = (
    ("fetch", "FETCH_SIZE"),
    ("write", "WRITE_SIZE"),
    ("sq", "SQ_WAVES SQ_INSTS_VALU SQ_INSTS_SALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD "
           "SQ_INSTS_VMEM_WR SQ_WAVE_CYCLES"),
    ("occ", "VALUBusy OccupancyPercent MeanOccupancyPerCU"),
)
SQ_COUNTERS = COUNTER_PASSES[2][1].split()
OCC_COUNTERS = (("VALUBusy", "% of kernel time a CU issues VALU"),
                ("OccupancyPercent", "% of the 32 wave slots per CU"),
                ("MeanOccupancyPerCU", "waves resident per CU"))
PROFILE_COMMANDS = [
    f"cd /tmp && TMPDIR=/tmp timeout -s KILL 900 rocprofv3 --pmc {ctr} --output-format csv -d <dir>/{name} "
    f"-o {name} -- python3 <repo>/bench.py {PROFILE_ARGS} > <dir>/{name}.log"
    for name, ctr in COUNTER_PASSES] + [
    f"cd /tmp && TMPDIR=/tmp timeout -s KILL 900 rocprofv3 --kernel-trace --stats --output-format csv "
    f"-d <dir>/trace -o trace -- python3 <repo>/bench.py {TRACE_ARGS} > <dir>/trace.log",
    "python3 <repo>/bench.py --summarize-profile <dir>"]
COPY_KERNEL = "copyBuffer"             # the runtime's device copy (the calibration copies)
COPY_BYTES = 1 << 30                   # bench.py --copy-calibration copies exactly 1 GiB, three times
MLP_PARAMS = 8192 * 28672
DECODER_PARAMS = 855_638_016
WORKLOAD_CHUNKS = {256: "1M", 16384: "8192x8192", 57344: "8192x28672", 208896: "decoder block",
                   3906250: "16e9 span"}
# The streaming kernels (compress, compress from weights, apply_mean, the fused
# update on chunk-major records) run a long call as equal launches of at most
# 2^16 chunks (stream_launch_chunks in csrc/internal.h); their trace rows are
# labelled with the workload the launches belong to.
STREAM_LAUNCH_CHUNKS = 1 << 16


def _split_launch_labels():
    labels = {}
    for c, name in WORKLOAD_CHUNKS.items():
        parts = -(-c // STREAM_LAUNCH_CHUNKS)
        if parts <= 1:
            continue
        per = -(-c // parts)
        last = c - (parts - 1) * per
        labels[per] = f"{name}, {parts} launches of {per} chunks" if last == per else \
            f"{name}, {parts - 1} of {parts} launches ({per} chunks)"
        if last != per:
            labels[last] = f"{name}, last of {parts} launches ({last} chunks)"
    return labels


SPLIT_LAUNCH_LABELS = _split_launch_labels()


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(base, name, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(base, name, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {os.path.join(base, name)}")
    return hits[0]


def _bench_line(path):
    """The JSON line bench.py printed in a profiled run (its steps, warmup, sets)."""
    with open(path) as f:
        for line in f:
            if line.startswith("{"):
                return json.loads(line)
    raise ValueError(f"no bench JSON line in {path}")


def _counter_dispatches(path):
    """Dispatches in order, each with its kernel, total work-items and the sum of
    every row of each counter (some counters are reported in several rows)."""
    by = {}
    for r in _csv_rows(path):
        d = by.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size"]),
                                                  "wg": int(r["Workgroup_Size"])})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [dict(v, dispatch=k) for k, v in sorted(by.items())]


def _chunks_of(kernel, grid_items, wg):
    """Chunks covered by one launch of an sl:: kernel (grids are padded to a
    multiple of 8 workgroups, one per XCD; the run kernel sums 2 or 3 chunks per
    wavefront; beyond 81 peers one)."""
    groups = grid_items // max(wg, 1)
    if "aggregate_run_kernel" in kernel or "aggregate_interleaved_kernel" in kernel:
        cpw = int(kernel.split("<")[1].split(">")[0].split(",")[1])   # <NGMAX, chunks per wavefront>
        cands = [c for c in WORKLOAD_CHUNKS if ((c + cpw - 1) // cpw + 7) // 8 * 8 == groups]
    else:
        cands = [c for c in WORKLOAD_CHUNKS if (c + 7) // 8 * 8 == groups or c == groups]
    return cands[0] if cands else groups


def _sl_key(kernel):
    """Short kernel name: the function and its template arguments."""
    k = kernel.replace("sl::(anonymous namespace)::", "").replace("void ", "")
    return k.split("(")[0].strip()


def _label_mlp(dispatches, line):
    """Label the sl:: dispatches at the 8192 x 28672 shape by the role they play
    in bench.py's run, from its fixed call order."""
    W, K, S = line["warmup"], line["steps"], line["kernels"]["aggregate_cold"]["record_sets"]
    peers = line["config"]["peers"]
    n_il = S + K if "aggregate_cold_interleaved" in line["kernels"] else 0
    n_step = peers * S + W + K + S + K + n_il    # setup, warmup, timed, cold and chunk-major cold steps
    n_host = 6 if "next_rows" in line else 0  # then the host-resident EF row: 1 warmup + 5 timed
    C = MLP_PARAMS // CHUNK
    seen = {}
    out = []
    step_agg = None         # the step's aggregate kernel: the first one-chunk aggregate at this shape
    for d in dispatches:
        name = _sl_key(d["kernel"])
        if not name.startswith(("compress_kernel", "aggregate", "apply_mean")):
            continue
        chunks = _chunks_of(d["kernel"], d["grid"], d["wg"])
        if step_agg is None and chunks == C and name.startswith("aggregate_kernel<") and name.endswith("false>"):
            step_agg = name
        # every chunk-major aggregate variant shares one count (the step's calls come first)
        key = ("aggregate_interleaved_kernel" if name.startswith("aggregate_interleaved_kernel") else name, chunks)
        i = seen.get(key, 0)
        seen[key] = i + 1
        label = None
        if chunks == C:
            if name == "compress_kernel<false>":
                timed = peers * S + W <= i < peers * S + W + K
                label = "compress_host_ef" if n_step <= i < n_step + n_host else (
                    "compress_timed" if timed else "compress")
            elif name == step_agg:
                # after the step's calls, next_rows: the per-peer receive path,
                # then the packed receive buffers
                j = i - (W + K + S + K)
                label = ("aggregate_timed" if W <= i < W + K else "aggregate") if i < W + K else (
                    "aggregate_cold" if j < 0 else None if "next_rows" not in line else
                    "receive" if j < NEXT_ROW_CALLS else
                    "aggregate_cold_packed" if j < 2 * NEXT_ROW_CALLS else None)
            elif name == "apply_mean_kernel":
                label = "apply_mean"
            elif name.startswith("aggregate_apply4_kernel"):
                label = "aggregate_apply"
            elif name == "compress_kernel<true>":
                label = "compress_weights"
            elif name.startswith("aggregate_interleaved_kernel"):
                label = "aggregate_cold_interleaved" if i < n_il else (
                    "receive_chunk_major" if "next_rows" in line and i < n_il + NEXT_ROW_CALLS else None)
        if label:
            out.append((label, d))
    return out


def _label_decoder(ds):
    """The decoder block's 24-peer aggregate dispatches in call order: the first
    half re-read one record set, the second half alternate two (records from
    HBM)."""
    dec = [d for d in ds if _sl_key(d["kernel"]).startswith("aggregate_run_kernel") and
           _chunks_of(d["kernel"], d["grid"], d["wg"]) == DECODER_PARAMS // CHUNK]
    half = len(dec) // 2
    return [("decoder_one_set", d) for d in dec[:half]] + [("decoder_two_sets", d) for d in dec[half:]]


def _calibration(dispatches, counter):
    """The run's leading copy dispatches are the three calibration copies
    (bench.py makes them before any other kernel): KiB per copy and the factor
    that turns the counter into bytes."""
    vals = []
    for d in dispatches:
        if COPY_KERNEL not in d["kernel"]:
            break
        vals.append(d[counter])
    if len(vals) < 3 or len(vals) % 3:
        raise ValueError(f"expected the run to start with three copies of {COPY_BYTES} bytes, "
                         f"found {len(vals)} leading copy dispatches")
    kib = sum(vals) / 3
    return kib, COPY_BYTES / (kib * 1024)


def _header(title, extra=()):
    lines = [f"# rocprofv3 counters: {title}", "# commands (run on the GPU box; <dir> is the summary's input):"]
    lines += [f"#   {c}" for c in PROFILE_COMMANDS]
    lines += [f"# {e}" for e in extra]
    return lines


def _kernel_sources(which):
    csrc = [os.path.join(CSRC, f) for f in ("wave.h", "residency.h", "internal.h")]
    inc = [os.path.join(ROOT, "include", "sparseloco.h")]
    if which == "compress":
        return [os.path.join(CSRC, "compress.hip")] + csrc + inc
    if which == "validate":
        return [os.path.join(CSRC, "validate.hip")] + csrc + inc
    return [os.path.join(CSRC, "aggregate.hip"), os.path.join(CSRC, "record.h")] + csrc + inc


def _counter_block(ds, by_pass, algo_read, algo_write, f_fac, w_fac, per_chunk):
    """Averages of every counter over the given dispatches (matched by id in each
    pass), with traffic scaled by the copy calibration."""
    ids = [d["dispatch"] for d in ds]

    def mean(pass_name, ctr):
        rows = [by_pass[pass_name][i] for i in ids if i in by_pass[pass_name]]
        if not rows or ctr not in rows[0]:
            return None
        return sum(r[ctr] for r in rows) / len(rows)

    fk, wk = mean("fetch", "FETCH_SIZE"), mean("write", "WRITE_SIZE")
    rb, wb = fk * 1024 * f_fac, wk * 1024 * w_fac
    lines = [f"dispatches_sampled: {len(ids)}",
             f"FETCH_SIZE_KiB_per_dispatch: {fk:.1f}",
             f"WRITE_SIZE_KiB_per_dispatch: {wk:.1f}",
             f"hbm_read_bytes_per_launch: {rb:.4g}   (algorithmic {algo_read:.4g}, ratio {rb / algo_read:.3f})",
             f"hbm_write_bytes_per_launch: {wb:.4g}   (algorithmic {algo_write:.4g}, ratio {wb / algo_write:.3f})",
             ""]
    for c, what in OCC_COUNTERS:
        v = mean("occ", c)
        if v is not None:
            lines.append(f"{c:<24}{v:>12.2f}   ({what})")
    lines.append("")
    for c in SQ_COUNTERS:
        v = mean("sq", c)
        if v is not None:
            lines.append(f"{c:<24}{v:>13.4g}   per 4096-chunk {v / per_chunk:>10.2f}")
    return lines, rb + wb


def summarize_profile(base, outdir):
    """Write the counter summaries (if the four counter passes are under
    `base`) and the kernel-trace summary (if the trace run is)."""
    written = []
    if os.path.isdir(os.path.join(base, COUNTER_PASSES[0][0])):
        written += summarize_counters(base, outdir)
    if os.path.isdir(os.path.join(base, "trace")):
        written.append(summarize_trace(base, outdir))
    if not written:
        raise FileNotFoundError(f"no rocprofv3 output under {base}")
    for p in written:
        print(p)
    return written


def summarize_counters(base, outdir):
    """Counter summaries of the run under `base` (the four passes)."""
    by_pass, lines_of = {}, {}
    for name, _ in COUNTER_PASSES:
        ds = _counter_dispatches(_find(base, name, "counter_collection.csv"))
        by_pass[name] = {d["dispatch"]: d for d in ds}
        lines_of[name] = ds
    line = _bench_line(os.path.join(base, "fetch.log"))
    f_kib, f_fac = _calibration(lines_of["fetch"], "FETCH_SIZE")
    w_kib, w_fac = _calibration(lines_of["write"], "WRITE_SIZE")
    cal = [f"Calibration: bench.py --copy-calibration runs three device copies of exactly 1 GiB; FETCH_SIZE "
           f"reads {f_kib:.1f} KiB per copy (factor {f_fac:.4f}), WRITE_SIZE {w_kib:.1f} KiB (factor {w_fac:.4f})."]
    n, C = MLP_PARAMS, MLP_PARAMS // CHUNK
    P = line["config"]["peers"]
    rec = P * RECORD / CHUNK
    labelled = [(lab.replace("_timed", ""), d) for lab, d in _label_mlp(lines_of["fetch"], line)]
    roles = {
        "compress": ("compress_kernel<false>", 8.0, 4.0 + RECORD / CHUNK, "compress"),
        "compress_weights": ("compress_kernel<true>", 12.0, 4.0 + RECORD / CHUNK, "compress"),
        "aggregate": ("aggregate_kernel, records cache-resident (the same 24 peers every call)", rec, 4.0, "aggregate"),
        "aggregate_cold": ("aggregate_kernel, records from HBM (four rotating record sets)", rec, 4.0, "aggregate"),
        "aggregate_cold_interleaved": ("aggregate_interleaved_kernel, records from HBM laid out chunk-major across "
                                       "peers (the same four sets)", rec, 4.0, "aggregate"),
        "apply_mean": ("apply_mean_kernel", 8.0, 4.0, "aggregate"),
        "aggregate_apply": ("aggregate_apply4_kernel", 4.0 + rec, 4.0, "aggregate"),
    }
    written = []
    files = {"compress": "compress_mlp_8192x28672_counters.txt",
             "compress_weights": "compress_weights_mlp_8192x28672_counters.txt",
             "aggregate": "aggregate_mlp_8192x28672_counters.txt",
             "apply_mean": "apply_mean_mlp_8192x28672_counters.txt",
             "aggregate_apply": "aggregate_apply_mlp_8192x28672_counters.txt"}
    sections = {}
    for role, (title, rd, wr, src) in roles.items():
        ds = [d for lab, d in labelled if lab == role]
        if not ds:
            continue
        body, total = _counter_block(ds, by_pass, rd * n, wr * n, f_fac, w_fac, C)
        head = [f"[{title}]", f"{src}_code_sha256_16: {code_digest(_kernel_sources(src))}   "
                f"({src}.hip and the headers it includes, comments and whitespace removed)",
                f"params_per_launch: {n}"] + body
        if role == "compress":
            head.insert(3, f"compress_hbm_bytes_per_launch: {total:.6g}")
        sections[role] = head
    for role, fname in files.items():
        if role not in sections:
            continue
        body = list(sections[role])
        if role == "aggregate":
            for extra in ("aggregate_cold", "aggregate_cold_interleaved"):
                if extra in sections:
                    body += [""] + sections[extra]
        lines = _header(f"{roles[role][0].split(',')[0]}, 8192 x 28672 fp32 ({n:,} params), {P} peers", cal) + [""] + body
        path = os.path.join(outdir, fname)
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    # Run kernels: the decoder block (24 peers) and the many-peer aggregate.
    run_sections = []
    dec_label = {"decoder_one_set": "decoder block, 24 peers, one record set re-read (partly cached)",
                 "decoder_two_sets": "decoder block, 24 peers, two record sets alternated (records from HBM)"}
    for lab, d in _label_decoder(lines_of["fetch"]):
        run_sections.append((dec_label[lab], _sl_key(d["kernel"]), d, DECODER_PARAMS, 24))
    many = line.get("workloads", {}).get("mlp_many_peers", {})
    counts = [int(k) for k in many if k.isdigit()]
    if counts:
        # the many-peer section calls sl_aggregate 3 + reps times per count, in MANY_PEERS order
        ds = [d for d in lines_of["fetch"] if _chunks_of(d["kernel"], d["grid"], d["wg"]) == C and
              _sl_key(d["kernel"]).startswith(("aggregate_run_kernel", "aggregate_kernel<")) and
              _sl_key(d["kernel"]).endswith(("false>", "3>", "2>", "1>"))]
        taken = sum(1 for lab, _ in labelled if lab in ("aggregate", "aggregate_cold", "receive",
                                                          "aggregate_cold_packed"))
        ds = ds[taken:]
        per = len(ds) // len(counts) if counts else 0
        for j, Pm in enumerate(sorted(counts)):
            for d in ds[j * per:(j + 1) * per][3:]:
                run_sections.append((f"8192 x 28672, {Pm} peers", _sl_key(d["kernel"]), d, n, Pm))
    # Chunk-major records (sl_aggregate_interleaved): after the step's cold
    # calls, the decoder block's two alternated sets and the many-peer counts.
    il_ds = [d for d in lines_of["fetch"] if _sl_key(d["kernel"]).startswith("aggregate_interleaved_kernel")]
    for d in il_ds:
        if _chunks_of(d["kernel"], d["grid"], d["wg"]) == DECODER_PARAMS // CHUNK:
            run_sections.append(("decoder block, 24 peers, two record sets alternated, chunk-major",
                                 _sl_key(d["kernel"]), d, DECODER_PARAMS, 24))
    il_counts = sorted(int(k) for k in many.get("interleaved", {}))
    if il_counts:
        n_il = line["kernels"]["aggregate_cold_interleaved"]["record_sets"] + line["steps"] \
            if "aggregate_cold_interleaved" in line["kernels"] else 0
        n_il += NEXT_ROW_CALLS if "next_rows" in line else 0      # the chunk-major receive path
        mlp_il = [d for d in il_ds if _chunks_of(d["kernel"], d["grid"], d["wg"]) == C][n_il:]
        per = len(mlp_il) // len(il_counts)
        for j, Pm in enumerate(il_counts):
            for d in mlp_il[j * per:(j + 1) * per][3:]:
                run_sections.append((f"8192 x 28672, {Pm} peers, chunk-major", _sl_key(d["kernel"]), d, n, Pm))
    # Validation and per-peer statistics of the 24 peers (next rows: calls on one
    # record set re-read and on four sets taken in turn move the same bytes).
    stat_roles = (
        ("validate_kernel, 24 peers in one launch (sl_validate_payloads)",
         lambda d: _sl_key(d["kernel"]).startswith("validate_kernel") and d["grid"] == P * C),
        ("stats_kernel, 24 peers (sl_peer_stats)", lambda d: _sl_key(d["kernel"]).startswith("stats_kernel")),
        ("stats_interleaved_kernel, 24 peers, records chunk-major (sl_peer_stats_interleaved)",
         lambda d: _sl_key(d["kernel"]).startswith("stats_interleaved_kernel")),
    )
    stat_lines = []
    for title, pick in stat_roles:
        ds = [d for d in lines_of["fetch"] if pick(d)]
        if ds:
            body, _ = _counter_block(ds, by_pass, P * C * RECORD, P * C * 1.0, f_fac, w_fac, P * C)
            stat_lines += ["", f"[{title}]"] + body
    if stat_lines:
        lines = _header(f"validation and per-peer statistics, 8192 x 28672 ({C:,} records per peer), {P} peers", cal)
        lines += [f"validate_code_sha256_16: {code_digest(_kernel_sources('validate'))}   "
                  "(validate.hip and the headers it includes, comments and whitespace removed)",
                  "algorithmic bytes: each record's 112 bytes and its 4-byte scale read, one flag byte written; "
                  "'per 4096-chunk' below is per record"] + stat_lines
        path = os.path.join(outdir, "validate_stats_mlp_8192x28672_counters.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    if run_sections:
        lines = _header("aggregate kernels with records beyond the last-level cache", cal)
        lines += [f"aggregate_code_sha256_16: {code_digest(_kernel_sources('aggregate'))}   "
                  "(aggregate.hip and the headers it includes, comments and whitespace removed)"]
        groups = {}
        for label, name, d, params, Pm in run_sections:
            groups.setdefault((label, name, params, Pm), []).append(d)
        for (label, name, params, Pm), ds in groups.items():
            body, _ = _counter_block(ds, by_pass, Pm * RECORD / CHUNK * params, 4.0 * params, f_fac, w_fac,
                                     params // CHUNK)
            lines += ["", f"[{label}: {name}]"] + body
        path = os.path.join(outdir, "aggregate_beyond_cache_counters.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    return written


def summarize_trace(base, outdir):
    """Per-kernel durations of every sl:: dispatch in the kernel-trace run,
    grouped by kernel and workload shape, with the bench line of the same run."""
    rows = _csv_rows(_find(base, "trace", "kernel_trace.csv"))
    line = _bench_line(os.path.join(base, "trace.log"))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    ds = [{"kernel": r["Kernel_Name"], "grid": int(r["Grid_Size_X"]), "wg": int(r["Workgroup_Size_X"]),
           "peers": int(r["Grid_Size_Y"]), "us": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3}
          for r in rows if "sl::" in r["Kernel_Name"]]
    role = {id(d): lab for lab, d in _label_mlp(ds, line) + _label_decoder(ds)}
    suffix = {"aggregate": ", records cached", "aggregate_cold": ", records from HBM",
              "compress_host_ef": ", ef in host memory", "decoder_one_set": ", one record set re-read",
              "aggregate_cold_interleaved": ", records from HBM, chunk-major",
              "aggregate_cold_packed": ", records from HBM, packed receive buffers",
              "receive": ", records from HBM, after the statistics pass",
              "receive_chunk_major": ", records from HBM, chunk-major, after the statistics pass",
              "decoder_two_sets": ", two record sets alternated"}
    timed_of = {"compress_timed": "compress_kernel<false> [8192x28672, timed steps only]",
                "aggregate_timed": "step aggregate [8192x28672, records cached, timed steps only]"}
    groups = {}
    for d in ds:
        name = _sl_key(d["kernel"])
        if name.startswith(("validate_kernel", "stats_kernel", "stats_interleaved_kernel")):
            # one lane per record (validate) or a fixed grid (statistics): label by grid
            label = f"{name} [grid {d['grid']} x {d['peers']}]"
        else:
            chunks = _chunks_of(d["kernel"], d["grid"], d["wg"])
            lab = role.get(id(d), "").replace("_timed", "")
            where = WORKLOAD_CHUNKS.get(chunks) or SPLIT_LAUNCH_LABELS.get(chunks, f"{chunks} chunks")
            label = f"{name} [{where}{suffix.get(lab, '')}]"
            if d["peers"] > 1:
                label += f" x{d['peers']} peers"
        lab = role.get(id(d))
        if lab in timed_of:
            groups.setdefault(timed_of[lab], []).append(d["us"])
            label = label.replace(", timed", "")
        groups.setdefault(label, []).append(d["us"])
    lines = [f"# rocprofv3 kernel trace of the default bench run (every sl:: dispatch, all shapes)",
             "# command:", f"#   {PROFILE_COMMANDS[len(COUNTER_PASSES)]}", f"#   {PROFILE_COMMANDS[-1]}",
             "# Durations are per dispatch from the kernel trace, all dispatches of the run (setup, warmup,",
             "# timed).  The bench line's own HIP-event means for the same run follow the table.",
             "# validate/stats rows: grid = lanes along x (validate: one per record) x peers (grid rows);",
             "# each of these rows holds the calls on one record set re-read and on four sets taken in turn.", "",
             f"{'kernel [shape]':<58}{'calls':>7}{'avg_us':>11}{'min_us':>11}{'max_us':>11}"]
    for label, ds in groups.items():
        lines.append(f"{label:<58}{len(ds):>7}{sum(ds) / len(ds):>11.2f}{min(ds):>11.2f}{max(ds):>11.2f}")
    k = line["kernels"]
    lines += ["", "# bench.py line of the same run (HIP events on the launch stream, timed steps only):",
              f"#   value {line['value']} Gparams/s, ms_per_step {line['ms_per_step']}, compress ms "
              f"{k['compress']['ms']}, aggregate ms {k['aggregate']['ms']}, aggregate_cold ms "
              f"{k['aggregate_cold']['ms']}, apply_mean ms {k['apply_mean']['ms']}",
              f"#   roofline: {json.dumps(line['roofline'])}"]
    path = os.path.join(outdir, "sl_kernels_mlp_8192x28672_kernel_trace.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path


if __name__ == "__main__":
    main()
