"""Host-side checks of bench.py's command line: it measures one GPU only and
refuses more, before touching torch or a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused_too():
    env = dict(os.environ, WORLD_SIZE="8")
    r = run(env=env)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_defaults_leave_the_timed_steps_after_the_warmup():
    sys.path.insert(0, ROOT)
    import importlib
    bench = importlib.import_module("bench")
    old = sys.argv
    try:
        sys.argv = ["bench.py"]
        a = bench.parse()
    finally:
        sys.argv = old
    assert a.gpus == 1 and a.warmup >= 25 and a.steps >= 20
