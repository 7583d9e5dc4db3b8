"""GPU: the binding works whatever the caller imports first.

torch ships its own HIP runtime under the same soname as the system runtime
the library links against, and the first one loaded serves the process. The
binding imports torch before it loads the library; this test runs, in a child
process, a caller that touches the binding before importing torch itself.
"""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import numpy as np
import newton_schulz_step_amd as nss
h = nss.hyper(ns_method="standard", ns_dtype="bf16", grad_dtype="bf16")   # loads the library
import torch
n = 64 * 96
p = torch.randn(n, device="cuda:0")
g = torch.randn(n, device="cuda:0").to(torch.bfloat16)
m = torch.zeros(n, device="cuda:0")
u = torch.zeros(n, device="cuda:0")
nss.step(p, g, m, [(0, 64, 96, 0)], h, update_out=u)
torch.cuda.synchronize()
assert torch.isfinite(u).all() and u.abs().sum() > 0
print("ok")
"""


def test_binding_before_torch(lib):
    r = subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, capture_output=True, text=True, timeout=180)
    assert r.returncode == 0 and "ok" in r.stdout, (r.returncode, r.stdout[-500:], r.stderr[-2000:])
