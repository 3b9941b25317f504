"""bench.py's contract on the CPU: a request for more than one GPU (flag or a
multi-rank launch) ends at once with a message and a non-zero status, before
any device is touched."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300,
                          env=dict(os.environ, **(env or {})))


def test_more_than_one_gpu_is_refused():
    r = _bench(["--gpus", "2"])
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _bench([], env={"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""
