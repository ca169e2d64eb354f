"""bench.py's one-GPU contract, without a GPU: asked for more than one GPU
(by flag or by WORLD_SIZE) it prints why and exits with status 2 before it
touches the device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args,world", [(["--gpus", "2"], "1"), (["--gpus", "8"], "1"),
                                        ([], "4")])
def test_bench_refuses_more_than_one_gpu(args, world):
    env = dict(os.environ, WORLD_SIZE=world)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], env=env,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stdout
