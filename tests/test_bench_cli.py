"""bench.py's command line, on the CPU: it measures one GPU and says so for any other count, it
refuses step counts it cannot time, and its options parse."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_options_parse():
    r = run("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--prefill-only", "--counters-only", "--bpbh"):
        assert opt in r.stdout


def test_step_counts_it_cannot_time_are_refused():
    for args in (("--steps", "0"), ("--warmup", "-1"), ("--steady-steps", "0"), ("--timing-steps", "0")):
        r = run(*args)
        assert r.returncode == 2, args
        assert ">= 1" in r.stderr, args
