"""The bench's command-line contract that holds without a GPU: the library
runs on one GPU, so any other GPU count is refused with a message, before
torch is imported or any device is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", ["2", "8"])
def test_bench_refuses_more_than_one_gpu(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
