"""Seeded random shapes across the plan chooser's whole range: every
operator, the plain and the _ws entry points, widths log-uniform in
[1, 300000], rows up to 3M elements per matrix, x, r and y each at a random
16-byte phase; and the widths around the kernels' boundaries.  Each call is
compared with the FP64 oracle at the usual bar (row min/max bit for bit),
with guard words around every output and, for the _ws calls that run the
exchange kernels, the workspace status word clear."""
import math

import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, print_case, shifted_input, torch
from tests.test_gpu_split import c_op, guarded_vec, make_inputs, reference, vec_guards_ok

pytestmark = pytest.mark.gpu

OPS = ["softmax", "rmsnorm", "layernorm_residual", "layernorm", "layernorm_affine", "row_sum", "row_minmax"]


def _case(rng, i):
    op = OPS[rng.integers(len(OPS))]
    width = int(math.exp(rng.uniform(0, math.log(300000))))
    max_rows = max(1, min(5000, (3 << 20) // width))
    rows = max(1, min(max_rows, int(math.exp(rng.uniform(0, math.log(max_rows + 1))))))
    shifts = tuple(int(v) for v in rng.integers(4, size=3))  # x, r, y: each its own 16-byte phase
    return op, rows, width, shifts, bool(rng.integers(2))


def check_case(op, rows, width, shifts, ws_entry, seed, what):
    """One call of `op` (plain or _ws entry point) with x, r and y at the
    given 16-byte phases, against the oracle, with guard words around the
    output and (exchange kernels) the status word clear."""
    t = torch()
    sx, sr, sy = shifts
    x, r, g, b = make_inputs(op, rows, width, seed=seed, dist="normal")
    ref = reference(op, x, r, g, b)
    xd = shifted_input(x, sx)
    rd = shifted_input(r, sr) if r is not None else None
    gd = t.from_numpy(g).cuda() if g is not None else None
    bd = t.from_numpy(b).cuda() if b is not None else None
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    ws = None
    if ws_entry:
        ws = R.new_workspace(c_op(op), rows, width)
        ws.zero_()
    if op in ("row_sum", "row_minmax"):
        b0, o0 = guarded_vec(rows)
        b1, o1 = guarded_vec(rows)
        if op == "row_sum":
            R.rowred_row_sum_ws(xd, o0, ws) if ws_entry else R.rowred_row_sum(xd, o0)
        else:
            R.rowred_row_minmax_ws(xd, o0, o1, ws) if ws_entry else R.rowred_row_minmax(xd, o0, o1)
        t.cuda.synchronize()
        assert vec_guards_ok(b0, rows) and vec_guards_ok(b1, rows), what
        if op == "row_sum":
            got = o0.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got - ref) <= 1e-5 + 1e-5 * np.abs(ref)), what
        else:
            assert np.array_equal(o0.cpu().numpy().view(np.uint32), ref[0].astype(np.float32).view(np.uint32)), what
            assert np.array_equal(o1.cpu().numpy().view(np.uint32), ref[1].astype(np.float32).view(np.uint32)), what
    else:
        out = Guarded(rows, width, sy)
        if op.startswith("layernorm"):
            if ws_entry:
                R.rowred_layernorm_ws(xd, rd, gd, bd, out.y, ws, eps=eps)
            else:
                R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=eps)
        elif op == "rmsnorm":
            R.rowred_rmsnorm_ws(xd, out.y, ws, eps=eps) if ws_entry else R.rowred_rmsnorm(xd, out.y, eps=eps)
        else:
            R.rowred_softmax_ws(xd, out.y, ws) if ws_entry else R.rowred_softmax(xd, out.y)
        t.cuda.synchronize()
        assert out.guards_intact(), what
        got = out.host().astype(np.float64)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), what
        fin = ~np.isnan(ref)
        assert np.all(np.abs(got[fin] - ref[fin]) <= 1e-5 + 1e-5 * np.abs(ref[fin])), what
    if ws is not None and op not in ("row_sum", "row_minmax"):
        plan = R.rowred_split_plan_query(c_op(op), xd)
        if plan.window > 8192 and plan.policy & R.ROWRED_POLICY_EXCHANGE:  # the call ran the exchange kernels
            assert int(ws[:8].view(t.int64).item()) == 0, what + ": a wait gave up"
    del xd, rd, ws


@pytest.mark.parametrize("block", range(4))
def test_random_shapes(block):
    rng = np.random.default_rng(np.random.SeedSequence([20261202, block]))
    for i in range(100):
        op, rows, width, shifts, ws_entry = _case(rng, i)
        what = f"{op} {rows}x{width} shifts {shifts} ws {ws_entry}"
        print_case("random", block, i, what)
        check_case(op, rows, width, shifts, ws_entry, 7919 * block + i, what)


# Widths around the kernels' boundaries, in floats: the register-resident
# window (8192 granules), the LayerNorm head of the head+tail kernels (8192
# granules of x and r) and the RMSNorm / softmax LDS stripe and head (16384
# granules); at each, offsets -3..+3 so that rows at every 16-byte phase land
# on either side of the boundary.
BOUNDARY_WIDTHS = sorted({base + d for base in (4 * 8192, 4 * 16384) for d in range(-3, 4)})


@pytest.mark.parametrize("op", OPS)
def test_boundary_widths(op):
    rng = np.random.default_rng(np.random.SeedSequence([20261203, OPS.index(op)]))
    for i, width in enumerate(BOUNDARY_WIDTHS):
        for ws_entry in (False, True):
            rows = int(rng.integers(4, 9))
            shifts = tuple(int(v) for v in rng.integers(4, size=3))
            what = f"{op} {rows}x{width} shifts {shifts} ws {ws_entry}"
            print_case("boundary", what)
            check_case(op, rows, width, shifts, ws_entry, 104729 + 31 * i + ws_entry, what)


def test_random_large_calls():
    """Calls of 128-640 MiB per input at seeded random widths of 8193-40000
    floats, x, r and y at random 16-byte phases, every matrix operator
    through the plain entry points: the range where the chooser takes the
    exchange kernels through y's rows for some rows and the row kernels for
    others.  Sampled rows against the oracle, every element finite, guard
    words intact."""
    t = torch()
    rng = np.random.default_rng(np.random.SeedSequence([20261204]))
    ops = ["softmax", "rmsnorm", "layernorm_residual", "layernorm", "layernorm_affine"]
    taken = 0
    for i in range(10):
        op = ops[i % len(ops)]
        width = int(rng.integers(8193, 40001))
        rows = int(rng.integers(128, 641)) * (1 << 20) // (4 * width)
        sx, sr, sy = (int(v) for v in rng.integers(4, size=3))
        what = f"{op} {rows}x{width} shifts {(sx, sr, sy)}"
        print_case("large", what)
        x = synthetic.random_matrix(900 + i, rows, width, "normal")
        r = synthetic.random_matrix(950 + i, rows, width, "normal", tensor="r") if op == "layernorm_residual" else None
        g = b = None
        if op == "layernorm_affine":
            g = (1.0 + 0.1 * synthetic.random_matrix(980 + i, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
            b = (0.1 * synthetic.random_matrix(990 + i, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
        xd = shifted_input(x, sx)
        rd = shifted_input(r, sr) if r is not None else None
        gd = t.from_numpy(g).cuda() if g is not None else None
        bd = t.from_numpy(b).cuda() if b is not None else None
        out = Guarded(rows, width, sy)
        if op.startswith("layernorm"):
            p = R.rowred_layernorm_plan_query(xd, rd, gd, bd, out.y)
            R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=1e-5)
        else:
            p = R.rowred_plan_query(op, xd, None, out.y)
            R.rowred_rmsnorm(xd, out.y, eps=1e-6) if op == "rmsnorm" else R.rowred_softmax(xd, out.y)
        taken += bool(p.policy & R.ROWRED_POLICY_EXCHANGE)
        t.cuda.synchronize()
        assert out.guards_intact(), what
        y = out.host()
        assert np.isfinite(y).all(), what
        pick = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 14)]))
        ref = reference(op, x[pick], r[pick] if r is not None else None, g, b)
        got = y[pick].astype(np.float64)
        assert np.all(np.abs(got - ref) <= 1e-5 + 1e-5 * np.abs(ref)), f"{what} {p}"
        del x, r, xd, rd, out, y
    assert taken >= 3  # the draw reaches the exchange rule more than once
