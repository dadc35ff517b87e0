"""More rows than 32 bits count: 2^31 + 5 rows of one float (rows at every
16-byte phase, 256 rows per workgroup, outputs staged) and 2^29 + 3 rows
of four floats (16-byte-aligned rows, XCD remap), 8.6 GB per matrix, built
on the device with closed-form results; sampled rows at both ends and in
the middle, and the last workgroup's replayed row slots."""
import math

import numpy as np
import pytest

import row_wise_reduction_amd as R
from tests.gpu_util import print_case, torch

pytestmark = pytest.mark.gpu


def _sample_rows(rows):
    picks = {0, 1, 2, 3, 255, 256, 257, (1 << 31) - 1, 1 << 31, rows // 2, rows - 257, rows - 5, rows - 2, rows - 1}
    return sorted(i for i in picks if 0 <= i < rows)


@pytest.fixture(autouse=True)
def _free():
    yield
    torch().cuda.empty_cache()


def _matrix(rows, width, pattern):
    """x = pattern repeated on every row, and y with NaN guard rows after it."""
    t = torch()
    x = t.tensor(pattern, dtype=t.float32, device="cuda").view(1, width).expand(rows, width).contiguous()
    ys = t.full(((rows + 2) * width,), float("nan"), dtype=t.float32, device="cuda")
    return x, ys, ys[:rows * width].view(rows, width)


def _guards_ok(ys, rows, width):
    t = torch()
    t.cuda.synchronize()
    return bool(t.isnan(ys[rows * width:]).all().item())


def _rows_at(y, idx):
    t = torch()
    i = t.tensor(idx, dtype=t.int64, device="cuda")
    return y[i].double().cpu().numpy()


CASES = [((1 << 31) + 5, 1, [0.1]), ((1 << 29) + 3, 4, [0.1, -0.2, 0.3, 0.4])]


@pytest.mark.parametrize("rows,width,pattern", CASES, ids=["width1", "width4"])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax", "layernorm_residual"])
def test_matrix_operators_on_many_rows(op, rows, width, pattern):
    t = torch()
    print_case("max rows", op, rows, width)
    x, ys, y = _matrix(rows, width, pattern)
    p = np.array([float(np.float32(v)) for v in pattern])
    if op == "rmsnorm":
        R.rowred_rmsnorm(x, y, eps=1e-6)
        want = p / math.sqrt(float(np.mean(p * p)) + float(np.float32(1e-6)))
    elif op == "softmax":
        R.rowred_softmax(x, y)
        e = np.exp(p - p.max())
        want = e / e.sum()
    else:
        r = t.zeros_like(x)
        R.rowred_layernorm_residual(x, r, y, eps=1e-5)
        del r
        d = p - p.mean()
        want = d / math.sqrt(float(np.mean(d * d)) + float(np.float32(1e-5)))
    assert _guards_ok(ys, rows, width)
    idx = _sample_rows(rows)
    got = _rows_at(y, idx)
    assert np.all(np.abs(got - want) <= 1e-5 + 1e-5 * np.abs(want)), (op, got[:3], want)


@pytest.mark.parametrize("rows,width,pattern", CASES, ids=["width1", "width4"])
def test_row_reductions_on_many_rows(rows, width, pattern):
    t = torch()
    print_case("max rows row_sum/minmax", rows, width)
    x, _, _ = _matrix(rows, width, pattern)
    out = t.full((rows + 64,), float("nan"), dtype=t.float32, device="cuda")
    R.rowred_row_sum(x, out[:rows])
    t.cuda.synchronize()
    assert bool(t.isnan(out[rows:]).all().item())
    p = np.array(pattern, dtype=np.float32)
    idx = _sample_rows(rows)
    got = _rows_at(out, idx)
    want = float(np.sum(p.astype(np.float64)))
    assert np.all(np.abs(got - want) <= 1e-5 + 1e-5 * abs(want)), got
    hi = t.empty(rows, dtype=t.float32, device="cuda")
    R.rowred_row_minmax(x, out[:rows], hi)
    assert np.all(_rows_at(out, idx) == float(p.min())) and np.all(_rows_at(hi, idx) == float(p.max()))
