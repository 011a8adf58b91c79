"""bench.py's host-side contract (CPU): it measures one GPU and refuses
--gpus N > 1 (or a multi-rank launch) with a message and exit status 2,
before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, env=e, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run([], env={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
