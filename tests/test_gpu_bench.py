"""bench.py on the GPU: one short run in a child process prints one JSON line
carrying every field the benchmark contract names, with the roofline and CPU
baseline objects, and numbers that are consistent with each other."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import note, require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_contract_line():
    require_gpu()
    note("bench.py --steps 3 --warmup 2 --no-next-rows --no-workloads --cpu-sample-chunks 256")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "2",
                        "--no-next-rows", "--no-workloads", "--cpu-sample-chunks", "256"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in j, k
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 2
    assert j["higher_is_better"] is True and j["vs_baseline"] is None and j["dtype"] == "f32"
    assert j["config"]["workload"] == "mlp_8192x28672_student_t3_zero20"
    n = j["config"]["params"]
    assert n == 8192 * 28672
    # value is params per step time
    assert abs(j["value"] - n / (j["ms_per_step"] * 1e-3) / 1e9) <= 1e-3 * j["value"]
    rf = j["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # achieved = algorithmic bytes per launch / the compressor's mean event time
    assert abs(rf["achieved"] - rf["algorithmic_bytes_per_launch"] / (j["kernels"]["compress"]["ms"] * 1e-3) / 1e9) \
        <= 1e-3 * rf["achieved"]
    cb = j["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "Gparams/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert "sample" in cb
