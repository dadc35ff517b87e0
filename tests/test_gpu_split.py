"""Split-row path (the _ws entry points and rowred_split_run_plan) against
the FP64 oracle: rows beyond the register-resident window, few rows, every
split geometry and policy, ragged and misaligned rows, empty segments, IEEE
special values, determinism and workspace reuse.

Bar: |y - ref| <= 1e-5 + 1e-5 |ref| (NaN exactly where the oracle has NaN);
row min/max bit for bit."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

OPS = ("layernorm_residual", "layernorm", "layernorm_affine", "rmsnorm", "softmax", "row_sum", "row_minmax")
GEOMETRIES = [(64, 1), (64, 2), (128, 4), (256, 1), (256, 4), (512, 2), (1024, 1), (1024, 4)]
GUARD_BITS = np.uint32(0x7FC0DEAD)


def c_op(op):
    return "layernorm_residual" if op.startswith("layernorm") else op


def make_inputs(op, rows, width, seed, dist="normal"):
    x = synthetic.random_matrix(seed, rows, width, dist)
    r = synthetic.random_matrix(seed + 1, rows, width, dist, tensor="r") if op == "layernorm_residual" else None
    g = b = None
    if op == "layernorm_affine":
        g = (1.0 + 0.1 * synthetic.random_matrix(seed + 2, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
        b = (0.1 * synthetic.random_matrix(seed + 3, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
    return x, r, g, b


def reference(op, x, r, g, b):
    if op == "row_sum":
        return oracle.row_sum(x)
    if op == "row_minmax":
        return oracle.row_minmax(x)
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    if op.startswith("layernorm"):
        return oracle.layernorm(x, r, eps=eps, gamma=g, beta=b)
    return oracle.run_op(op, x, eps=eps)


def guarded_vec(n):
    t = torch()
    buf = t.empty(n + 128, dtype=t.int32, device="cuda")
    buf.fill_(int(GUARD_BITS.view(np.int32)))
    return buf, buf[64:64 + n].view(t.float32)


def vec_guards_ok(buf, n):
    v = buf.cpu().numpy().view(np.uint32)
    return bool((v[:64] == GUARD_BITS).all() and (v[64 + n:] == GUARD_BITS).all())


def run(op, x, r, g, b, plan=None, shift=0, ws=None):
    """Run on the GPU (x, r, y `shift` floats off 16-byte alignment) through
    the _ws entry point, or rowred_split_run_plan with `plan`."""
    t = torch()
    rows, width = x.shape
    xd = shifted_input(x, shift)
    rd = shifted_input(r, shift) if r is not None else None
    gd = t.from_numpy(g).cuda() if g is not None else None
    bd = t.from_numpy(b).cuda() if b is not None else None
    if ws is None:
        need = R.rowred_workspace_size(c_op(op), rows, width)
        if plan is not None:
            need = max(need, R.rowred_split_plan_query(c_op(op), xd, plan=plan).workspace_bytes)
        ws = t.empty(max(need, 16), dtype=t.uint8, device="cuda")
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    if op in ("row_sum", "row_minmax"):
        b0, o0 = guarded_vec(rows)
        b1, o1 = guarded_vec(rows)
        if plan is not None:
            R.rowred_split_run_plan(op, xd, None, None, None, o0, o1 if op == "row_minmax" else None, plan, ws)
        elif op == "row_sum":
            R.rowred_row_sum_ws(xd, o0, ws)
        else:
            R.rowred_row_minmax_ws(xd, o0, o1, ws)
        t.cuda.synchronize()
        assert vec_guards_ok(b0, rows) and vec_guards_ok(b1, rows)
        return (o0.cpu().numpy(), o1.cpu().numpy()) if op == "row_minmax" else o0.cpu().numpy()
    out = Guarded(rows, width, shift)
    if plan is not None:
        R.rowred_split_run_plan(c_op(op), xd, rd, gd, bd, out.y, None, plan, ws, eps=eps)
    elif op.startswith("layernorm"):
        R.rowred_layernorm_ws(xd, rd, gd, bd, out.y, ws, eps=eps)
    elif op == "rmsnorm":
        R.rowred_rmsnorm_ws(xd, out.y, ws, eps=eps)
    else:
        R.rowred_softmax_ws(xd, out.y, ws)
    t.cuda.synchronize()
    assert out.guards_intact(), f"{op} {x.shape} wrote outside y"
    return out.host()


def check(op, got, ref, what):
    if op == "row_minmax":
        lo, hi = got
        assert np.array_equal(lo.view(np.uint32), ref[0].astype(np.float32).view(np.uint32)), what + " min"
        assert np.array_equal(hi.view(np.uint32), ref[1].astype(np.float32).view(np.uint32)), what + " max"
    else:
        assert_close(got, ref, what)


@pytest.mark.parametrize("width", [1, 3, 127, 1537, 8191, 32769, 40000, 131075])
@pytest.mark.parametrize("op", OPS)
def test_ws_entry_any_width(op, width):
    """Within the register-resident window the _ws entry runs the row kernels;
    beyond it, the split kernels.  Both must match the oracle."""
    rows = max(2, min(9, (1 << 21) // width))
    print_case("ws", op, rows, width)
    x, r, g, b = make_inputs(op, rows, width, seed=width + 17)
    check(op, run(op, x, r, g, b, shift=width % 4), reference(op, x, r, g, b), f"{op} {rows}x{width}")


@pytest.mark.parametrize("geom", GEOMETRIES, ids=lambda g: f"T{g[0]}C{g[1]}")
@pytest.mark.parametrize("op", OPS)
def test_every_split_geometry(op, geom):
    """Explicit split plans at widths inside and beyond the row kernels'
    window, ragged and misaligned, several segments per row."""
    T, C = geom
    for width, shift in ((1000, 1), (4 * T * C + 5, 3), (33000, 0)):
        rows = 5
        x, r, g, b = make_inputs(op, rows, width, seed=7 * width + T + C)
        ref = reference(op, x, r, g, b)
        for policy in (0, R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_REVERSE,
                       R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_REVERSE):
            plan = R.SplitPlan(threads=T, chunks=C, policy=policy)
            print_case("split", op, rows, width, shift, plan)
            check(op, run(op, x, r, g, b, plan=plan, shift=shift), ref, f"{op} {width} {plan}")


@pytest.mark.parametrize("op", OPS)
def test_empty_last_segment(op):
    """Width 255 with 64-granule segments: rows starting at phase 2 or 3 span
    65 granules (2 segments), the others 64, whose second segment is empty."""
    rows, width = 8, 255
    x, r, g, b = make_inputs(op, rows, width, seed=255)
    plan = R.SplitPlan(threads=64, chunks=1, policy=0)
    for shift in range(4):
        xd = shifted_input(x, shift)
        assert R.rowred_split_plan_query(c_op(op), xd, plan=plan).segments == 2
        check(op, run(op, x, r, g, b, plan=plan, shift=shift), reference(op, x, r, g, b), f"{op} shift {shift}")


@pytest.mark.parametrize("op", ["softmax", "row_sum", "row_minmax", "rmsnorm", "layernorm"])
def test_special_values(op):
    rows, width = 8, 5000
    x = synthetic.random_matrix(91, rows, width, "normal")
    x[0, :] = -np.inf                   # softmax: NaN row
    x[1, :2600] = -np.inf               # whole segments of -inf next to finite ones
    x[2, 4000] = np.nan                 # poisons sums; skipped by min/max
    x[3, 10] = np.inf
    x[4, :] = np.nan                    # min/max: (+inf, -inf)
    x[5, :] = 3.0                       # constant row
    # large values that cancel; their squares (1e30, times 5000) stay inside
    # FP32's range, where RMSNorm and LayerNorm accumulate them
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    plan = R.SplitPlan(threads=64, chunks=2, policy=0)  # 128-granule segments: 10 per row
    ref = reference(op, x, None, None, None)
    got = run(op, x, None, None, None, plan=plan)
    check(op, got, ref, f"{op} special")
    if op == "softmax":
        assert np.isnan(got[0]).all() and not np.isnan(got[1]).any()
        assert np.abs(got[1].astype(np.float64).sum() - 1.0) < 1e-5


@pytest.mark.parametrize("op", ["softmax", "layernorm_residual", "row_sum"])
def test_deterministic_and_workspace_reuse(op):
    t = torch()
    x, r, g, b = make_inputs(op, 6, 70001, seed=5)
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    first = run(op, x, r, g, b, ws=ws)
    # another shape through the same workspace in between
    x2, r2, g2, b2 = make_inputs(op, 3, 50000, seed=6)
    check(op, run(op, x2, r2, g2, b2, ws=ws), reference(op, x2, r2, g2, b2), "reuse")
    again = run(op, x, r, g, b, ws=ws)
    assert np.array_equal(np.asarray(first).view(np.uint32), np.asarray(again).view(np.uint32))


@pytest.mark.parametrize("case", synthetic.NEXT_WORKLOADS.get(9, []) + synthetic.NEXT_WORKLOADS.get(11, []),
                         ids=lambda c: c.name)
def test_wide_workloads_full_size(case):
    """The wide-row, few-row and many-wide-row workload shapes at full size
    through the _ws entry point (exchange, three-kernel or looped path, as
    the chooser picks); sampled rows against the oracle."""
    t = torch()
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
    got = run(case.op, x, r, None, None)
    pick = sorted({0, case.rows // 2, case.rows - 1})
    for i in pick:
        ref = reference(case.op, x[i:i + 1], r[i:i + 1] if r is not None else None, None, None)
        if case.op == "row_minmax":
            check(case.op, (got[0][i:i + 1], got[1][i:i + 1]), ref, f"{case.name} row {i}")
        else:
            check(case.op, got[i:i + 1], ref, f"{case.name} row {i}")
    del got
    t.cuda.empty_cache()


@pytest.mark.parametrize("op", OPS)
def test_row_blocks(op):
    """Passes over blocks of rows give bitwise the one-pass result (each row's
    records and their order do not depend on the blocks)."""
    rows, width, shift = 7, 33001, 2
    x, r, g, b = make_inputs(op, rows, width, seed=33)
    whole = run(op, x, r, g, b, plan=R.SplitPlan(threads=256, chunks=2, policy=3), shift=shift)
    check(op, whole, reference(op, x, r, g, b), f"{op} one pass")
    for br in (1, 3, 6):
        got = run(op, x, r, g, b, plan=R.SplitPlan(threads=256, chunks=2, policy=3, block_rows=br), shift=shift)
        assert np.array_equal(np.asarray(got).view(np.uint32), np.asarray(whole).view(np.uint32)), (op, br)


def test_graph_capture_and_replay():
    """The three split kernels of each _ws call captured in one HIP graph
    with one shared workspace (no memset nodes: the workspace needs no
    clearing), replayed several times with eager work and synchronisation
    in between; every replay equals the eager results bitwise."""
    t = torch()
    rows, width = 5, 40001
    x = synthetic.random_matrix(404, rows, width, "normal")
    r = synthetic.random_matrix(405, rows, width, "normal", tensor="r")
    xd, rd = shifted_input(x, 1), shifted_input(r, 1)
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    outs = [t.empty(rows, width, device="cuda") for _ in range(3)] + [t.empty(rows, device="cuda") for _ in range(3)]

    def calls():
        R.rowred_layernorm_ws(xd, rd, None, None, outs[0], ws, eps=1e-5)
        R.rowred_rmsnorm_ws(xd, outs[1], ws, eps=1e-6)
        R.rowred_softmax_ws(xd, outs[2], ws)
        R.rowred_row_sum_ws(xd, outs[3], ws)
        R.rowred_row_minmax_ws(xd, outs[4], outs[5], ws)

    calls()
    t.cuda.synchronize()
    eager = [o.clone() for o in outs]
    assert_close(eager[0].cpu().numpy(), oracle.layernorm_residual(x, r, 1e-5), "graph ln")
    assert_close(eager[2].cpu().numpy(), oracle.softmax(x), "graph softmax")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            calls()
    t.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for o in outs:
            o.fill_(float("nan"))
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert t.equal(o.view(t.int32), e.view(t.int32)), (rep, i)
        calls()  # eager work between replays, through the same workspace
        t.cuda.synchronize()
