"""Importing the binding before torch must still bind libtaco to torch's HIP
runtime (the binding loads torch first).  Runs in a fresh interpreter."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

pytestmark = pytest.mark.gpu

SCRIPT = r"""
import gradients_taco_compress_amd as taco   # before any explicit torch import
import torch
x = torch.ones((4, 256), dtype=torch.bfloat16, device="cuda")
c, a, s = taco.compress(x, block=128)
y = taco.decompress(c, a, s, block=128)
_, sums = taco.roundtrip(x, block=128, variant="tensor")
torch.cuda.synchronize()
assert torch.equal(y.float(), x.float()), y
print("ok", taco.fidelity_metrics(sums, x.numel())["tensor_absmax"])
"""


def test_binding_imported_before_torch():
    print("[case] import order (fresh interpreter)", flush=True)
    res = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True,
                         text=True, timeout=240, env={**os.environ, "PYTHONPATH": ROOT})
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().startswith("ok 1.0"), res.stdout
