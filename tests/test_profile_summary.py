"""bench.py --summarize-profile on a small synthetic rocprofv3 output (CPU only).

The fixture mimics the CSV layout rocprofv3 writes for the four counter passes
and the kernel trace: a bench run with 1 warmup step, 3 timed steps and 4
record sets at 8192 x 28672, three 1 GiB calibration copies split into four
dispatches each at the start (later copies of the data generator are not
calibration), and some counters reported in several rows per dispatch.  The
counter values are chosen so that every expected figure is known in closed
form: the copy's FETCH_SIZE reads half its bytes (calibration factor 2), and
each kernel's calibrated traffic equals its algorithmic bytes times a known
ratio."""
import csv
import json
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

N = 8192 * 28672
C = N // 4096
P, W, K, S = 24, 1, 3, 4
REC = 116 / 4096
COUNTER_COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
                "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
                "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp",
                "End_Timestamp"]
TRACE_COLS = ["Kind", "Agent_Id", "Queue_Id", "Stream_Id", "Thread_Id", "Dispatch_Id", "Kernel_Id", "Kernel_Name",
              "Correlation_Id", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
              "Accum_VGPR_Count", "SGPR_Count", "Workgroup_Size_X", "Workgroup_Size_Y", "Workgroup_Size_Z",
              "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
COMPRESS = "void sl::(anonymous namespace)::compress_kernel<false>(float const*, float const*, float*, float, " \
           "unsigned char*, float*, long)"
AGG = "void sl::(anonymous namespace)::aggregate_kernel<3, false>(sl::PeerTable, int, float*, long, long, float)"
MEAN = "sl::(anonymous namespace)::apply_mean_kernel(float*, float const*, float, long)"
RUN63 = "void sl::(anonymous namespace)::aggregate_run_kernel<6, 3>(sl::PeerTable, int, float*, long, long)"
RUN151 = "void sl::(anonymous namespace)::aggregate_run_kernel<15, 1>(sl::PeerTable, int, float*, long, long)"
RUN_ITEMS = ((C + 2) // 3 + 7) // 8 * 8 * 64
IL31 = "void sl::(anonymous namespace)::aggregate_interleaved_kernel<3, 1>(unsigned char const*, float const*, int, " \
       "float*, long, long)"
IL62 = IL31.replace("<3, 1>", "<6, 2>")
IL151 = IL31.replace("<3, 1>", "<15, 1>")
IL2_ITEMS = ((C + 1) // 2 + 7) // 8 * 8 * 64
COPY = "__amd_rocclr_copyBuffer"
TORCH = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >(int, at::native::FillFunctor<float>, std::array<char*, 2ul>)"

# (kernel, work-items, workgroup size, KiB read, KiB written, duration us)
AGG_ITEMS = (C + 7) // 8 * 8 * 64
SEQUENCE = (
    [(COPY, 1 << 20, 512, 131072.0, 262144.0, 100.0)] * 12
    + [(TORCH, 1 << 20, 256, 10.0, 20.0, 5.0), (COPY, 1 << 16, 512, 500.0, 1000.0, 5.0)]
    + [(COMPRESS, C * 256, 256, 8 * N / 2048, (4 + REC) * N / 1024, 450.0)] * (P * S)
    + [(COMPRESS, C * 256, 256, 8 * N / 2048 * 1.01, (4 + REC) * N / 1024, 449.0)] * (W + K)
    + [(AGG, AGG_ITEMS, 64, P * REC * N / 2048, 4 * N / 1024, 152.0)] * (W + K)
    + [(COMPRESS, C * 256, 256, 8 * N / 2048, (4 + REC) * N / 1024, 451.0), (AGG, AGG_ITEMS, 64,
                                                                            P * REC * N / 2048, 4 * N / 1024,
                                                                            220.0)] * (S + K)
    # the same cold steps with chunk-major records
    + [(COMPRESS, C * 256, 256, 8 * N / 2048, (4 + REC) * N / 1024, 452.0), (IL31, AGG_ITEMS, 64,
                                                                            P * REC * N / 2048, 4 * N / 1024,
                                                                            199.0)] * (S + K)
    + [(MEAN, C * 256, 256, 8 * N / 2048, 4 * N / 1024, 430.0)] * (W + K)
    # the many-peer section: 36 peers (three chunks per wavefront), then 128 (one), 3 + 2 calls each
    + [(RUN63, RUN_ITEMS, 64, 36 * REC * N / 2048, 4 * N / 1024, 240.0)] * 5
    + [(RUN151, AGG_ITEMS, 64, 128 * REC * N / 2048, 4 * N / 1024, 500.0)] * 5
    # then chunk-major: 36 peers (two chunks per wavefront), 128 (one)
    + [(IL62, IL2_ITEMS, 64, 36 * REC * N / 2048, 4 * N / 1024, 215.0)] * 5
    + [(IL151, AGG_ITEMS, 64, 128 * REC * N / 2048, 4 * N / 1024, 373.0)] * 5
)


def bench_line():
    return {"metric": bench.METRIC, "value": 350.0, "steps": K, "warmup": W, "ms_per_step": 0.67,
            "config": {"peers": P}, "roofline": {"bound": "hbm", "frac": 0.79},
            "workloads": {"mlp_many_peers": {"params": N, "chunks": C, "36": {"ms": 0.24}, "128": {"ms": 0.56},
                                             "interleaved": {"36": {"ms": 0.215}, "128": {"ms": 0.373}}}},
            "kernels": {"compress": {"ms": 0.45}, "aggregate": {"ms": 0.152},
                        "aggregate_cold": {"ms": 0.22, "record_sets": S},
                        "aggregate_cold_interleaved": {"ms": 0.199, "record_sets": S}, "apply_mean": {"ms": 0.43}}}


def write_fixture(base):
    for name, ctrs in bench.COUNTER_PASSES:
        d = os.path.join(base, name)
        os.makedirs(d)
        with open(os.path.join(d, f"{name}_counter_collection.csv"), "w", newline="") as f:
            w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
            w.writerow(COUNTER_COLS)
            for i, (kern, items, wg, rd, wr, _) in enumerate(SEQUENCE, start=1):
                for c in ctrs.split():
                    val = {"FETCH_SIZE": rd, "WRITE_SIZE": wr}.get(c, 1.0 * i)
                    # FETCH_SIZE arrives in two rows per dispatch; the summary adds them
                    parts = [val / 2, val / 2] if c == "FETCH_SIZE" else [val]
                    for v in parts:
                        w.writerow([i, i, "Agent 1", 1, 1, 1, items, 1, kern, wg, 0, 0, 8, 0, 16, c, v, 0, 0])
        with open(os.path.join(base, f"{name}.log"), "w") as f:
            f.write("rocprofv3 banner\n" + json.dumps(bench_line()) + "\n")
    d = os.path.join(base, "trace")
    os.makedirs(d)
    t = 1000
    with open(os.path.join(d, "trace_kernel_trace.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(TRACE_COLS)
        for i, (kern, items, wg, _, _, us) in enumerate(SEQUENCE, start=1):
            w.writerow(["KERNEL_DISPATCH", "Agent 1", 1, 0, 1, i, 1, kern, i, t, t + int(us * 1000), 0, 0, 8, 0, 16,
                        wg, 1, 1, items, 1, 1])
            t += int(us * 1000) + 500
    with open(os.path.join(base, "trace.log"), "w") as f:
        f.write(json.dumps(bench_line()) + "\n")


@pytest.fixture()
def summary(tmp_path):
    base, out = tmp_path / "prof", tmp_path / "profiles"
    os.makedirs(base)
    os.makedirs(out)
    write_fixture(str(base))
    files = bench.summarize_profile(str(base), str(out))
    return out, files


def test_compress_summary_carries_calibrated_traffic_and_the_code_digest(summary, monkeypatch):
    out, files = summary
    txt = (out / "compress_mlp_8192x28672_counters.txt").read_text()
    assert "factor 2.0000" in txt and "factor 1.0000" in txt
    digest = re.search(r"compress_code_sha256_16:\s*([0-9a-f]{16})", txt).group(1)
    assert digest == bench.code_digest(bench.KERNEL_SOURCES)
    # 96 setup + 4 step + 7 cold-step + 7 chunk-major cold-step dispatches; the step ones read 1% more
    assert "dispatches_sampled: 114" in txt
    reads = (P * S * 1.0 + (W + K) * 1.01 + 2 * (S + K) * 1.0) / 114 * 8 * N
    writes = (4 + REC) * N
    got = float(re.search(r"compress_hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt).group(1))
    assert got == pytest.approx(reads + writes, rel=1e-5)
    # the roofline object reads exactly this figure back
    monkeypatch.setattr(bench, "PROFILE", str(out / "compress_mlp_8192x28672_counters.txt"))
    assert bench.traffic_from_profile(N) == pytest.approx(got, rel=1e-6)
    assert bench.traffic_from_profile(N + 4096) is None


def test_aggregate_summary_separates_cache_resident_and_cold_calls(summary):
    out, _ = summary
    txt = (out / "aggregate_mlp_8192x28672_counters.txt").read_text()
    warm, cold, chunk_major = txt.split("records from HBM")
    assert "dispatches_sampled: 4" in warm and "dispatches_sampled: 7" in cold
    assert "laid out chunk-major" in chunk_major and "dispatches_sampled: 7" in chunk_major
    assert txt.count("ratio 1.000") == 6
    assert (out / "apply_mean_mlp_8192x28672_counters.txt").exists()


def test_many_peer_sections_take_the_timed_calls_of_each_count(summary):
    out, _ = summary
    txt = (out / "aggregate_beyond_cache_counters.txt").read_text()
    for label in ("[8192 x 28672, 36 peers: aggregate_run_kernel<6, 3>]",
                  "[8192 x 28672, 128 peers: aggregate_run_kernel<15, 1>]",
                  "[8192 x 28672, 36 peers, chunk-major: aggregate_interleaved_kernel<6, 2>]",
                  "[8192 x 28672, 128 peers, chunk-major: aggregate_interleaved_kernel<15, 1>]"):
        block = txt.split(label)[1].split("\n[")[0]
        assert "dispatches_sampled: 2" in block and "ratio 1.000" in block


def test_headers_name_commands_that_run_committed_files_only(summary):
    out, files = summary
    for path in files:
        head = open(path).read().split("\n\n")[0]
        assert "rocprofv3" in head and "bench.py" in head
        assert "_work" not in head and "gpurun" not in head


def test_trace_summary_groups_dispatches_by_kernel_and_shape(summary):
    out, _ = summary
    txt = (out / "sl_kernels_mlp_8192x28672_kernel_trace.txt").read_text()
    def row(prefix):
        r = [l for l in txt.splitlines() if l.startswith(prefix)][0].split()
        return int(r[-4]), float(r[-3])
    assert row("aggregate_kernel<3, false> [8192x28672, records cached]") == (W + K, 152.0)
    assert row("aggregate_kernel<3, false> [8192x28672, records from HBM]") == (S + K, 220.0)
    calls, avg = row("compress_kernel<false> [8192x28672]")
    assert calls == P * S + W + K + 2 * (S + K)
    assert row("aggregate_interleaved_kernel<3, 1> [8192x28672, records from HBM, chunk-major]") == (S + K, 199.0)
    assert row("compress_kernel<false> [8192x28672, timed steps only]") == (K, 449.0)
    assert row("step aggregate [8192x28672, records cached, timed steps only]") == (K, 152.0)


def test_command_line_entry_point(tmp_path):
    base = tmp_path / "prof"
    os.makedirs(base)
    write_fixture(str(base))
    out = tmp_path / "out"
    os.makedirs(out)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-profile", str(base),
                        "--profile-out", str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "compress_mlp_8192x28672_counters.txt" in r.stdout
    assert (out / "compress_mlp_8192x28672_counters.txt").exists()


def test_next_row_aggregates_are_labelled_by_call_order():
    """After the step's aggregates, a bench line with next rows labels the
    per-peer aggregates of the receive path, then those of the packed receive
    buffers (NEXT_ROW_CALLS each), and the chunk-major aggregates after the
    step's as the chunk-major receive path; calls beyond those get no role."""
    line = bench_line()
    line["next_rows"] = {}
    n_row = bench.NEXT_ROW_CALLS
    agg = [{"kernel": AGG, "grid": AGG_ITEMS, "wg": 64, "peers": 1, "us": 1.0}
           for _ in range(W + K + S + K + 2 * n_row + 3)]
    il = [{"kernel": IL31, "grid": AGG_ITEMS, "wg": 64, "peers": 1, "us": 1.0} for _ in range(S + K + n_row + 2)]
    labels = [lab for lab, _ in bench._label_mlp(agg + il, line)]
    assert labels.count("aggregate_timed") == K and labels.count("aggregate") == W
    assert labels.count("aggregate_cold") == S + K
    assert labels.count("receive") == n_row and labels.count("aggregate_cold_packed") == n_row
    assert labels.count("aggregate_cold_interleaved") == S + K
    assert labels.count("receive_chunk_major") == n_row
    assert len(labels) == len(agg) + len(il) - 3 - 2
    # without next rows the calls after the step's get no role
    line.pop("next_rows")
    labels = [lab for lab, _ in bench._label_mlp(agg + il, line)]
    assert "receive" not in labels and "aggregate_cold_packed" not in labels and "receive_chunk_major" not in labels
