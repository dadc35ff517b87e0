"""Looped path (ROWRED_POLICY_LOOPED): the plain entry points at widths
beyond one register-resident pass, and explicit looped plans with many
tiles, against the FP64 oracle (|y - ref| <= 1e-5 + 1e-5 |ref|, NaN where
the oracle has NaN; row min/max bit for bit)."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, print_case, shifted_input, torch
from tests.test_gpu_split import OPS, check, guarded_vec, make_inputs, reference, vec_guards_ok

pytestmark = pytest.mark.gpu

LOOPED = R.ROWRED_POLICY_LOOPED
STREAM = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES


def run(op, x, r, g, b, plan=None, shift=0):
    """Through the plain entry point (plan None) or with an explicit plan."""
    t = torch()
    rows, width = x.shape
    xd = shifted_input(x, shift)
    rd = shifted_input(r, shift) if r is not None else None
    gd = t.from_numpy(g).cuda() if g is not None else None
    bd = t.from_numpy(b).cuda() if b is not None else None
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    if op in ("row_sum", "row_minmax"):
        b0, o0 = guarded_vec(rows)
        b1, o1 = guarded_vec(rows)
        o1a = o1 if op == "row_minmax" else None
        if plan is not None:
            R.rowred_row_reduce_run_plan(op, xd, o0, o1a, plan)
        elif op == "row_sum":
            R.rowred_row_sum(xd, o0)
        else:
            R.rowred_row_minmax(xd, o0, o1)
        t.cuda.synchronize()
        assert vec_guards_ok(b0, rows) and vec_guards_ok(b1, rows)
        return (o0.cpu().numpy(), o1.cpu().numpy()) if op == "row_minmax" else o0.cpu().numpy()
    out = Guarded(rows, width, shift)
    if op.startswith("layernorm"):
        if plan is not None:
            R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=eps)
        else:
            R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=eps)
    elif plan is not None:
        R.rowred_run_plan(op, xd, None, out.y, plan, eps=eps)
    elif op == "rmsnorm":
        R.rowred_rmsnorm(xd, out.y, eps=eps)
    else:
        R.rowred_softmax(xd, out.y)
    t.cuda.synchronize()
    assert out.guards_intact(), f"{op} {x.shape} wrote outside y"
    return out.host()


def looped_plan(T, C, policy=STREAM):
    return R.Plan(lanes_per_row=T, rows_per_group=0, chunks=C, threads=T, grid=0, policy=LOOPED | policy)


@pytest.mark.parametrize("width", [32769, 40000, 100003, 131075])
@pytest.mark.parametrize("op", OPS)
def test_entry_points_any_width(op, width):
    rows = 3
    print_case("looped entry", op, rows, width)
    x, r, g, b = make_inputs(op, rows, width, seed=width + 3)
    check(op, run(op, x, r, g, b, shift=width % 4), reference(op, x, r, g, b), f"{op} {rows}x{width}")


@pytest.mark.parametrize("geom", [(64, 2), (64, 4), (256, 2), (256, 4), (1024, 2), (1024, 4)],
                         ids=lambda g: f"T{g[0]}C{g[1]}")
@pytest.mark.parametrize("op", OPS)
def test_explicit_looped_plans(op, geom):
    """Many tiles per row, odd and even tile counts (the two-deep loop's
    tail), a partial last tile, misaligned rows, both memory policies."""
    T, C = geom
    if op.startswith("layernorm") and C == 4:
        # LayerNorm loops at 2 chunks only: the plan is refused before
        # anything runs
        x, r, g, b = make_inputs(op, 2, 40000, seed=9)
        with pytest.raises(R.RowRedError) as e:
            run(op, x, r, g, b, plan=looped_plan(T, C))
        assert e.value.status == R.ROWRED_ERR_INVALID_ARG
        return
    G = T * C
    for width, shift in ((4 * G * 3 - 7, 1), (4 * G * 4 + 5, 3), (4 * G, 0), (5, 2)):
        x, r, g, b = make_inputs(op, 4, width, seed=width * 7 + T)
        ref = reference(op, x, r, g, b)
        for policy in (0, STREAM, STREAM | R.ROWRED_POLICY_XCD_REMAP):
            plan = looped_plan(T, C, policy)
            print_case("looped", op, width, shift, plan)
            check(op, run(op, x, r, g, b, plan=plan, shift=shift), ref, f"{op} {width} {plan}")


@pytest.mark.parametrize("op", ["softmax", "row_sum", "row_minmax", "rmsnorm", "layernorm"])
def test_special_values(op):
    rows, width = 8, 5000
    x = synthetic.random_matrix(92, rows, width, "normal")
    x[0, :] = -np.inf                   # softmax: NaN row
    x[1, :2600] = -np.inf               # whole tiles of -inf before finite ones
    x[2, 4000] = np.nan
    x[3, 10] = np.inf
    x[4, :] = np.nan
    x[5, :] = 3.0
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    x[7, 4990:] = 50.0                  # the max arrives in the last tile: the running sum rescales
    plan = looped_plan(64, 2, 0)        # 128-granule tiles: 10 per row
    ref = reference(op, x, None, None, None)
    got = run(op, x, None, None, None, plan=plan)
    check(op, got, ref, f"{op} special")
    if op == "softmax":
        assert np.isnan(got[0]).all() and not np.isnan(got[1]).any() and not np.isnan(got[7]).any()


@pytest.mark.parametrize("op", ["softmax", "layernorm_residual", "row_sum"])
def test_deterministic(op):
    x, r, g, b = make_inputs(op, 4, 70001, seed=9)
    first = run(op, x, r, g, b)
    again = run(op, x, r, g, b)
    assert np.array_equal(np.asarray(first).view(np.uint32), np.asarray(again).view(np.uint32))


@pytest.mark.parametrize("case", synthetic.NEXT_WORKLOADS[10], ids=lambda c: c.name)
def test_full_size_wide_rows(case):
    """The many-wide-rows workload at full size through the plain entry
    points; sampled rows against the oracle."""
    t = torch()
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
    got = run(case.op, x, r, None, None)
    for i in (0, case.rows // 2, case.rows - 1):
        ref = reference(case.op, x[i:i + 1], r[i:i + 1] if r is not None else None, None, None)
        check(case.op, got[i:i + 1], ref, f"{case.name} row {i}")
    t.cuda.empty_cache()


@pytest.mark.parametrize("op", ["row_sum", "row_minmax"])
def test_ws_entry_loops_many_wide_rows(op):
    """2048 rows beyond the register-resident window: the _ws entry points
    of the row reductions run the looped kernels and never touch the
    workspace (None is fine)."""
    t = torch()
    rows, width = 2048, 33001
    x = synthetic.random_matrix(77, rows, width, "normal")
    xd = shifted_input(x, 1)
    lo = t.empty(rows, device="cuda")
    hi = t.empty(rows, device="cuda")
    if op == "row_minmax":
        R.rowred_row_minmax_ws(xd, lo, hi, None)
        t.cuda.synchronize()
        got = (lo.cpu().numpy(), hi.cpu().numpy())
    else:
        R.rowred_row_sum_ws(xd, lo, None)
        t.cuda.synchronize()
        got = lo.cpu().numpy()
    check(op, got, reference(op, x, None, None, None), f"ws looped {op}")


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_ws_entry_needs_workspace_for_matrix_outputs(op):
    """Same shape, matrix operators: the _ws entry points run the exchange
    kernels, which need the workspace (None is an invalid argument)."""
    t = torch()
    rows, width = 2048, 33001
    x = synthetic.random_matrix(78, rows, width, "normal")
    xd = shifted_input(x, 1)
    y = t.empty(rows, width, device="cuda")
    with pytest.raises(R.RowRedError) as e:
        if op == "rmsnorm":
            R.rowred_rmsnorm_ws(xd, y, None, eps=1e-6)
        else:
            R.rowred_softmax_ws(xd, y, None)
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG
    ws = R.new_workspace(op, rows, width)
    if op == "rmsnorm":
        R.rowred_rmsnorm_ws(xd, y, ws, eps=1e-6)
    else:
        R.rowred_softmax_ws(xd, y, ws)
    t.cuda.synchronize()
    yh = y.cpu().numpy()
    for i in (0, 1, 1024, 2047):
        check(op, yh[i:i + 1], reference(op, x[i:i + 1], None, None, None), f"ws exchange {op} row {i}")
