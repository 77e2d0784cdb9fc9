"""bench.py's command line on the host: the flag combinations it refuses
exit with a message before any GPU work (no GPU needed)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*argv):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=120, cwd=ROOT)
    return r.returncode, r.stdout + r.stderr


def test_more_than_one_gpu_exits_with_a_message():
    rc, out = bench("--gpus", "2")
    assert rc != 0 and "one GPU" in out


@pytest.mark.parametrize("argv, text", [
    (["--workload", "packed", "--constrained"], "1D forward"),
    (["--workload", "dcn2d", "--constrained"], "1D forward"),
    (["--workload", "depthwise", "--backward", "--constrained"], "times the forward"),
])
def test_refused_combinations(argv, text):
    rc, out = bench(*argv)
    assert rc != 0 and text in out, out
