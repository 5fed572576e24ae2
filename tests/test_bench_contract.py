"""bench.py's command-line contract that needs no GPU: it measures one GPU
and refuses more, with a message and a non-zero status, before touching the
device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2", RANK="0", LOCAL_RANK="0")
    r = _run("--steps", "1", env=env)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_help_lists_the_workloads_and_modes():
    r = _run("--help")
    assert r.returncode == 0
    for word in ("--workload", "--mode", "--root-period", "--precision", "--steps", "--warmup"):
        assert word in r.stdout, word
