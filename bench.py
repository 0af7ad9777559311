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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
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
RECORD = 112 + 4                 # payload bytes + fp32 scale per chunk

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
    return ap.parse_args()


def main():
    args = parse()
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
    del scratch_ef
    torch.cuda.synchronize()

    if args.copy_calibration:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

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
        },
        "wall_s_timed": round(wall, 4),
        "device": device_props(torch, dev),
    }

    if not args.no_next_rows:
        result["next_rows"] = next_rows(sl, delta, ef, payload, scales, peer_p, peer_s, theta, n,
                                        stream, kstats)

    if not args.no_workloads:
        del out
        result["workloads"] = workloads(sl, dev)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args, delta, ef0_host, peer_p, peer_s, theta, n)

    print(json.dumps(result), flush=True)


def next_rows(sl, delta, ef, payload, scales, peer_p, peer_s, theta, n, stream, kstats, reps=20):
    """The entry points beyond the compress + aggregate step, on the same
    workload (not part of `value`): fused aggregate + outer update, compression
    straight from pre/post weights, error feedback in pinned host memory, record
    validation for one peer and for all 24 in one launch."""
    import torch

    def timed(fn, k=reps, warm=3):
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
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) / k

    res = {}
    t = timed(lambda: sl.sl_aggregate_apply(peer_p, peer_s, theta))
    res["aggregate_apply_fused"] = kstats(t, 8 + N_PEERS * RECORD / CHUNK)
    pre = theta
    post = theta - delta               # so that pre - post carries the workload's values
    t = timed(lambda: sl.sl_compress_weights(pre, post, ef, BETA, payload, scales))
    res["compress_weights"] = kstats(t, 16 + RECORD / CHUNK)
    del post
    ef_host = torch.zeros(n, dtype=torch.float32, pin_memory=True)
    t = timed(lambda: sl.sl_compress_host_ef(delta, ef_host, BETA, payload, scales), k=2, warm=1)
    st = kstats(t, 4 + RECORD / CHUNK)       # HBM bytes only; ef moves over the host link
    st["host_link_gb_per_s"] = round(8 * n / (t * 1e-3) / 1e9, 1)
    res["compress_host_ef"] = st
    del ef_host
    flags = torch.empty(n // CHUNK, dtype=torch.uint8, device=delta.device)
    t = timed(lambda: sl.sl_validate_payload(peer_p[0], peer_s[0], flags))
    res["validate_one_peer"] = kstats(t, (RECORD + 1) / CHUNK)
    flags_all = torch.empty((N_PEERS, n // CHUNK), dtype=torch.uint8, device=delta.device)
    t = timed(lambda: sl.sl_validate_payloads(peer_p, peer_s, flags_all))
    res["validate_24_peers"] = kstats(t, N_PEERS * (RECORD + 1) / CHUNK)
    counts = torch.empty((N_PEERS, 4), dtype=torch.int64, device=delta.device)
    smax = torch.empty(N_PEERS, dtype=torch.float32, device=delta.device)
    peers = sl.PeerSet(peer_p, peer_s)
    t = timed(lambda: sl.sl_peer_stats(peers, None, counts, smax, flags=flags_all))
    res["peer_stats_24_peers"] = kstats(t, N_PEERS * (RECORD + 1) / CHUNK)
    res["small_round_1m"] = small_round(sl, delta.device)
    return res


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


def workloads(sl, dev, reps=10):
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
        if W == datagen.DECODER_BLOCK:
            theta = ef
            theta.copy_(a).mul_(0.02)
            t, ts = timed_calls(torch, stream, lambda: sl.sl_aggregate_apply(peers, None, theta), k=reps)
            r["aggregate_apply_fused"] = st(n, t, 8 + N_PEERS * RECORD / CHUNK, ts)
            t, ts = timed_calls(torch, stream, lambda: sl.sl_apply_mean(theta, out, N_PEERS), k=reps)
            r["apply_mean"] = st(n, t, BYTES_APPLY, ts)
        res[name] = r
        del a, ef, out, payload, scales, pp, ps, peers
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


if __name__ == "__main__":
    main()
