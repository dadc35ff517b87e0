"""One row of ROWRED_MAX_WIDTH floats (8.6 GB per matrix) through the plain
entry points (looped and head+tail kernels) and a _ws entry point (three
split kernels), x one float past a 16-byte boundary.  The rows are built on
the device with closed-form results, so the oracle is the formula itself:
the widest row the library takes, with every 32-bit index near its top."""
import math

import numpy as np
import pytest

import row_wise_reduction_amd as R
from tests.gpu_util import print_case, torch

pytestmark = pytest.mark.gpu

N = R.ROWRED_MAX_WIDTH
GUARD = 64
SAMPLES = (0, 1, 2, 3, 4097, 65535, 65536, 65537, 1 << 24, N // 2, N - 16389, N - 4097, N - 5, N - 2, N - 1)


def _row(fill):
    """A row of N floats one float past an aligned allocation, filled on the
    device, and an output row with NaN guards after it."""
    t = torch()
    xs = t.empty(N + 4, dtype=t.float32, device="cuda")
    x = xs[1:1 + N]
    fill(x)
    ys = t.full((N + GUARD + 1,), float("nan"), dtype=t.float32, device="cuda")
    y = ys[1:1 + N]
    return xs, x, ys, y


def _guards_ok(ys):
    t = torch()
    t.cuda.synchronize()
    return bool(t.isnan(ys[0]).item()) and bool(t.isnan(ys[1 + N:]).all().item())


def _at(y, idx):
    t = torch()
    i = t.tensor(idx, dtype=t.int64, device="cuda")
    return y[i].double().cpu().numpy()


@pytest.fixture(autouse=True)
def _free():
    yield
    torch().cuda.empty_cache()


def test_row_sum_at_max_width():
    t = torch()
    print_case("max width row_sum")
    xs, x, _, _ = _row(lambda v: v.fill_(1.0))
    out = t.full((3,), float("nan"), device="cuda")
    R.rowred_row_sum(x.view(1, N), out[1:2])
    t.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert abs(got[1] - N) <= 1e-5 * N, got
    assert np.isnan(got[0]) and np.isnan(got[2])
    lo, hi = t.empty(1, device="cuda"), t.empty(1, device="cuda")
    x[N - 1] = 7.0
    x[0] = -3.0
    R.rowred_row_minmax(x.view(1, N), lo, hi)
    assert (lo.item(), hi.item()) == (-3.0, 7.0)


@pytest.mark.parametrize("entry", ["plain", "ws"])
def test_softmax_at_max_width(entry):
    """x = 0, -1, 0, -1, ... with 1.0 at one even tail element k: the max is
    found in the tail (the running sum rescales), and the terms e^-1 and
    e^-2 are inexact in FP32, so the sum over 2^31 of them shows how it is
    accumulated.  Checked relative to each value (the absolute bar alone
    would pass any y of this size)."""
    t = torch()
    print_case("max width softmax", entry)
    k = N - 3001  # even, in the tail, not among SAMPLES

    def fill(v):
        v.zero_()
        v[1::2] = -1.0
        v[k] = 1.0

    xs, x, ys, y = _row(fill)
    if entry == "plain":
        R.rowred_softmax(x.view(1, N), y.view(1, N))
    else:
        ws = R.new_workspace("softmax", 1, N)
        R.rowred_softmax_ws(x.view(1, N), y.view(1, N), ws)
    assert _guards_ok(ys)
    n_even, n_odd = (N + 1) // 2, (N - 1) // 2
    den = (n_even - 1) * math.exp(-1.0) + n_odd * math.exp(-2.0) + 1.0
    idx = np.array(SAMPLES + (k,))
    want = np.where(idx % 2 == 0, math.exp(-1.0), math.exp(-2.0)) / den
    want[-1] = 1.0 / den
    got = _at(y, SAMPLES + (k,))
    assert np.all(np.abs(got / want - 1.0) <= 1e-5), np.max(np.abs(got / want - 1.0))


@pytest.mark.parametrize("entry", ["plain", "ws"])
def test_rmsnorm_at_max_width(entry):
    """A constant row of float32(0.1): 2^31 inexact squares."""
    t = torch()
    print_case("max width rmsnorm", entry)
    xs, x, ys, y = _row(lambda v: v.fill_(0.1))
    if entry == "plain":
        R.rowred_rmsnorm(x.view(1, N), y.view(1, N), eps=1e-6)
    else:
        ws = R.new_workspace("rmsnorm", 1, N)
        R.rowred_rmsnorm_ws(x.view(1, N), y.view(1, N), ws, eps=1e-6)
    assert _guards_ok(ys)
    v = float(np.float32(0.1))
    want = v / math.sqrt(v * v + float(np.float32(1e-6)))
    got = _at(y, SAMPLES)
    assert np.all(np.abs(got - want) <= 1e-5 + 1e-5 * want), got


def test_layernorm_residual_at_max_width():
    """x = +1, -1, +1, ... (N odd: mean 1/N, biased variance 1 - 1/N^2) and
    r = 0, through the head+tail LayerNorm kernel."""
    t = torch()
    print_case("max width layernorm_residual")

    def fill(v):
        v.fill_(1.0)
        v[1::2] = -1.0

    xs, x, ys, y = _row(fill)
    rs = t.zeros(N + 4, dtype=t.float32, device="cuda")
    r = rs[1:1 + N]
    R.rowred_layernorm_residual(x.view(1, N), r.view(1, N), y.view(1, N), eps=1e-5)
    assert _guards_ok(ys)
    del rs, r
    mean = 1.0 / N
    var = 1.0 - mean * mean
    scale = 1.0 / math.sqrt(var + float(np.float32(1e-5)))
    idx = np.array(SAMPLES)
    want = ((1.0 - 2.0 * (idx % 2)) - mean) * scale
    got = _at(y, SAMPLES)
    assert np.all(np.abs(got - want) <= 1e-5 + 1e-5 * np.abs(want)), (got, want)
