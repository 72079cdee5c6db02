"""bench.py's command-line contract on a host without a GPU (CPU tests).

The bench runs on one GPU: asked for more, it exits with status 2 and says so
before touching the device.  Without a GPU it fails loudly (status 1) rather
than timing anything on the host.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_is_refused(n):
    r = _bench("--gpus", n)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_gpu_fails_loudly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    r = _bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1, r.stderr
    assert "needs a GPU" in r.stderr
    assert r.stdout == ""
