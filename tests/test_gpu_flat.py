"""Flat plans (ROWRED_POLICY_FLAT) against the FP64 oracle.

A workgroup takes its rows as one run of 16-byte granules, lane
after lane, and folds per-granule partials per row in LDS.  Checked at every
geometry, short and ragged widths (4 upward), every 16-byte phase of x and y,
row counts around rows_per_group, IEEE special values, and bitwise
reproducibility over three dispatches.

Bar: |y - ref| <= 1e-5 + 1e-5 |ref|, NaN exactly where the oracle has NaN."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch
from tests.test_gpu_parity import oracle_of

pytestmark = pytest.mark.gpu

FLAT = R.ROWRED_POLICY_FLAT
NT = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES


def run_plan(op, x, plan, sx=0, sy=0, r=None, sr=0, g=None, b=None):
    t = torch()
    rows, width = x.shape
    xd = shifted_input(x, sx)
    rd = shifted_input(r, sr) if r is not None else None
    out = Guarded(rows, width, sy)
    eps = synthetic.EPS.get(op, 0.0)
    if op.startswith("layernorm"):
        gd = t.from_numpy(g).cuda() if g is not None else None
        bd = t.from_numpy(b).cuda() if b is not None else None
        R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=1e-5)
    else:
        R.rowred_run_plan(op, xd, None, out.y, plan, eps=eps)
    t.cuda.synchronize()
    assert out.guards_intact(), f"{op} {x.shape} {plan} wrote outside y"
    return out.host()


def flat(T, C, policy=NT):
    return R.Plan(lanes_per_row=0, rows_per_group=0, chunks=C, threads=T, grid=0, policy=FLAT | policy)


@pytest.mark.parametrize("width", [4, 5, 7, 9, 31, 63, 127, 129, 257, 300, 511, 1000, 1537, 2047])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_flat_every_geometry(op, width):
    x = synthetic.random_matrix(17 * width, 300, width, "normal")
    ref = oracle_of(op, x)
    n = 0
    for T in (64, 128, 256, 512):
        for C in (1, 2, 4):
            if 4 * T * C - 3 < width:
                continue  # not one row per workgroup: refused
            for pol, (sx, sy) in ((NT, (1, 1)), (0, (3, 3)), (NT | R.ROWRED_POLICY_XCD_REMAP, (2, 0)), (NT, (0, 0))):
                plan = flat(T, C, pol)
                print_case("flat", op, width, T, C, pol, sx, sy)
                assert_close(run_plan(op, x, plan, sx, sy), ref, f"{op} {width} T{T} C{C} pol{pol} x{sx} y{sy}")
                n += 1
    assert n > 0


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
@pytest.mark.parametrize("width", [127, 257])
def test_flat_row_counts(op, width):
    """1 row, rows_per_group - 1, rows_per_group, + 1, and a longer tail."""
    for T, C in ((256, 4), (512, 2), (64, 1)):
        plan = flat(T, C)
        P = min(T, (4 * T * C - 3) // width)
        if P < 1:
            continue  # a row longer than the workgroup's run: refused (test_flat_refused_elsewhere)
        for rows in sorted({1, max(1, P - 1), P, P + 1, 3 * P + 2}):
            x = synthetic.random_matrix(rows * 131 + width, rows, width, "normal")
            print_case("flat rows", op, width, T, C, rows)
            assert_close(run_plan(op, x, plan, 1, 1), oracle_of(op, x), f"{op} {rows}x{width} T{T} C{C}")


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_flat_special_values(op):
    rows, width = 40, 127
    x = synthetic.random_matrix(91, rows, width, "normal")
    x[0, :] = -np.inf              # softmax: NaN row
    x[1, :100] = -np.inf
    x[2, 60] = np.nan
    x[3, 0] = np.inf               # first element of a row
    x[4, 126] = np.inf             # last element of a row
    x[5, :] = 3.0
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    x[7, :] = 0.0
    x[8, :] = 80.0
    x[9, :] = -80.0                # neighbours far apart: a granule shared by rows 8 and 9
    for T, C in ((256, 4), (64, 1)):
        got = run_plan(op, x, flat(T, C), 1, 1)
        assert_close(got, oracle_of(op, x), f"{op} special T{T} C{C}")


def test_flat_is_reproducible():
    x = synthetic.random_matrix(93, 4099, 127, "normal")
    for op in ("rmsnorm", "softmax"):
        outs = [run_plan(op, x, flat(256, 4), 3, 3) for _ in range(3)]
        assert all(np.array_equal(outs[0].view(np.uint32), o.view(np.uint32)) for o in outs[1:])


@pytest.mark.parametrize("op", ["layernorm_residual", "row_sum"])
def test_flat_refused_elsewhere(op):
    """Flat plans exist for RMSNorm and softmax only, for rows of at least 4
    elements and workgroups that hold one row."""
    t = torch()
    x = t.zeros(8, 127, device="cuda")
    y = t.empty_like(x)
    with pytest.raises(R.RowRedError) as e:
        if op == "row_sum":
            R.rowred_row_reduce_run_plan(op, x, t.empty(8, device="cuda"), None, flat(256, 4))
        else:
            R.rowred_run_plan(op, x, x.clone(), y, flat(256, 4), eps=1e-5)
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG
    for width, T, C in ((3, 64, 1), (300, 64, 1)):
        xx = t.zeros(8, width, device="cuda")
        with pytest.raises(R.RowRedError) as e:
            R.rowred_run_plan("softmax", xx, None, t.empty_like(xx), flat(T, C))
        assert e.value.status == R.ROWRED_ERR_INVALID_ARG
