"""The library loaded before torch: the binding then imports torch first, so the library
shares torch's HIP runtime and its first launch on a torch stream works.  Runs in a child
process (this process has torch loaded already) and compares the child's forward with
this process's, bit for bit."""

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

from tests.gpu_util import gen, gs_tensor, sync

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import numpy as np
import fp8_grouped_gemm_ragged_amd as g
g.load()  # before any torch import by this script
import torch
from tests.gpu_util import gen, gs_tensor
x, _ = gen((300, 256), 1.0, 71)
w, _ = gen((3, 256, 384), 0.02, 72)
wq, ws = g.gmm_quantize_rhs(w, "e4m3", 0, "nk")
y = g.gmm_fwd(x, wq, ws, gs_tensor([100, 0, 200]))
torch.cuda.synchronize()
np.save({out!r}, y.view(torch.int16).cpu().numpy())
print("child ok", flush=True)
"""


def test_library_loaded_before_torch(lib, tmp_path):
    out = str(tmp_path / "y.npy")
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, out=out)], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-3000:]
    x, _ = gen((300, 256), 1.0, 71)
    w, _ = gen((3, 256, 384), 0.02, 72)
    wq, ws = lib.gmm_quantize_rhs(w, "e4m3", 0, "nk")
    y = lib.gmm_fwd(x, wq, ws, gs_tensor([100, 0, 200]))
    sync()
    assert np.array_equal(np.load(out), y.view(torch.int16).cpu().numpy())
