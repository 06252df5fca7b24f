"""CPU checks of bench.py's command line: it runs on exactly one GPU and
refuses anything else before touching torch or the GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "exactly one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run(env=env)
    assert r.returncode != 0
    assert "exactly one GPU" in r.stderr
