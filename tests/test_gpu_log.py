"""DC1D_LOG: with the variable set, each call that launches work writes one
line to stderr naming the entry and the kernel chosen (checked in a child
process, since the library reads the variable once)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, torch
sys.path.insert(0, %r)
from deformable_convolution_amd import dc1d, inputs
w = inputs.WORKLOADS["tiny"]
t = inputs.make_inputs(w, seed=0)
g = {k: (v.cuda() if v is not None else None) for k, v in t.items()}
dc1d.forward(g["x"], g["offsets"], g["weight"], g["bias"], g["mask"])
torch.cuda.synchronize()
print("child done", flush=True)
"""


@pytest.mark.parametrize("value, logged", [("1", True), ("0", False)])
def test_dispatch_log(value, logged):
    env = dict(os.environ, DC1D_LOG=value)
    r = subprocess.run([sys.executable, "-c", CHILD % ROOT], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "child done" in r.stdout
    lines = [l for l in r.stderr.splitlines() if l.startswith("dc1d: ")]
    if logged:
        assert len(lines) == 1 and "forward B=1 C_in=4" in lines[0] and "-> direct" in lines[0], lines
    else:
        assert not lines, lines
