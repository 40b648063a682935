"""bench.py's command line on the CPU: it measures one GPU only, and says so."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=120, env=env)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = _run("--gpus", n)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no JSON line


def test_world_size_above_one_exits_with_a_message():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run(env=env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_without_a_gpu_exits_nonzero():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0
    assert r.stdout == ""
