"""The library binds to the HIP runtime torch uses, whatever the import
order: loading librowred.so before torch must not leave a second HIP
runtime in the process (torch's stream handles would be invalid to it).
Run in a fresh interpreter, since load order is per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import numpy as np
import row_wise_reduction_amd as R
R.lib()                      # the library first, torch after
import torch
import oracle
x = np.random.default_rng(0).standard_normal((33, 300)).astype(np.float32)
xd = torch.from_numpy(x).cuda()
y = torch.empty_like(xd)
s = torch.cuda.Stream()
with torch.cuda.stream(s):   # a non-default torch stream handle
    R.rowred_softmax(xd, y)
s.synchronize()
ok, excess, idx = oracle.within_tolerance(y.cpu().numpy(), oracle.softmax(x))
assert ok, (excess, idx)
print("runtime-order ok", flush=True)
"""


def test_library_loaded_before_torch():
    r = subprocess.run([sys.executable, "-c", SCRIPT], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "runtime-order ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
