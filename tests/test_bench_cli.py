"""Host-side checks of bench.py's command line (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_exits_with_a_message(n):
    """The library has no multi-GPU path: bench.py --gpus N (N > 1) stops before
    touching a GPU, with a non-zero status and a message on stderr."""
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=60)
    assert p.returncode == 2
    assert p.stdout == ""
    assert "one GPU only" in p.stderr and f"--gpus {n}" in p.stderr
