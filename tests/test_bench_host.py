"""Host-side contract of bench.py: a request for more than one GPU (by flag
or by a torchrun-style WORLD_SIZE) exits with status 2 and a message before
anything touches a GPU, and prints no result line."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, **env})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
