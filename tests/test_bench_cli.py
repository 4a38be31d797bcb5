"""bench.py's host-side contract that needs no GPU: it measures one GPU only and refuses more with
a message and exit status 2, before touching the device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_bench_refuses_several_gpus(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert r.stdout == ""
    assert f"--gpus {n}" in r.stderr and "one GPU only" in r.stderr
