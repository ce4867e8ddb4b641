"""bench.py's command line on the CPU: it measures one GPU, so a request for
more (--gpus N > 1, or a launcher's WORLD_SIZE > 1) exits with status 2 and
says why, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          env=e, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run(["--gpus", "1"], env={"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
