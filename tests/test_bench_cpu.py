"""bench.py's host-side contract on a machine without a GPU: it refuses more than one GPU
with a message (the path is single-GPU) before touching any device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, timeout=120, env=e)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run(["--steps", "1"], env={"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_legs():
    r = _run(["--help"])
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--gpus", "--no-backward", "--no-two-level", "--only"):
        assert flag in r.stdout
