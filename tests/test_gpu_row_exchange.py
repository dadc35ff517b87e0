"""Row plans with ROWRED_POLICY_EXCHANGE: the exchange kernels behind the
plain entry points, each row's statistics swapped through words kept in y's
own row (no workspace), which segment 0 writes its outputs over last.

Each plan is checked bitwise against the same geometry through the
workspace entry (the same kernels, the words elsewhere) and against the FP64
oracle (atol = rtol = 1e-5), with y's guard bands intact: one, three and the
most segments per row, every LDS stripe, ragged rows, y at every 16-byte
phase against x, IEEE special values, a y left dirty by an earlier call, and
the chooser's own plans at full size."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch
from tests.test_gpu_split import c_op, check, make_inputs, reference, run

pytestmark = pytest.mark.gpu

MATRIX_OPS = ("layernorm_residual", "layernorm", "layernorm_affine", "rmsnorm", "softmax")
EXCHANGE = R.ROWRED_POLICY_EXCHANGE
STREAM = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES
LDS = R.ROWRED_POLICY_LDS_STRIPE
# (threads, chunks, policy) of the kernels the chooser takes, and small ones
GEOMETRIES = [(64, 1, 0), (256, 2, 0), (1024, 4, 0), (256, 8, 0), (256, 8, LDS), (256, 12, LDS), (256, 16, LDS)]


def max_segments(op, T, C):
    """The most segments whose words (2 S + 1 for LayerNorm, S + 1 otherwise,
    from the row's first 16-byte boundary) end inside segment 0's outputs
    (LayerNorm: inside the granules of its first slot)."""
    ln = op.startswith("layernorm")
    rounds = 2 if ln else 1
    S = min(128, T)
    while 15 + 8 * (rounds * S + 1) > 16 * T * (1 if ln else C) - 12:
        S -= 1
    return S


def fits(op, T, C, policy):
    """LayerNorm exchanges hold at most 4 register slots (more only with the
    LDS stripe at 256 threads)."""
    return not op.startswith("layernorm") or C <= 4 or (policy & LDS and T == 256)


def plain(op, xd, rd, g, b, plan, rows, width, y_shift, y=None):
    """The plain run-plan entry with a row plan; y (a Guarded) may be reused."""
    t = torch()
    out = y or Guarded(rows, width, y_shift)
    gd = t.from_numpy(g).cuda() if g is not None else None
    bd = t.from_numpy(b).cuda() if b is not None else None
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    if op.startswith("layernorm"):
        R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=eps)
    else:
        R.rowred_run_plan(op, xd, None, out.y, plan, eps=eps)
    t.cuda.synchronize()
    assert out.guards_intact(), f"{op} {plan}: guard band"
    return out


@pytest.mark.parametrize("geom", GEOMETRIES, ids=lambda g: f"T{g[0]}C{g[1]}P{g[2]}")
@pytest.mark.parametrize("op", MATRIX_OPS)
def test_row_exchange_matches_workspace_exchange(op, geom):
    T, C, pol = geom
    if not fits(op, T, C, pol):
        return
    G = T * C
    S_max = max_segments(op, T, C)
    for S, shift in ((1, 0), (3, 3), (S_max, 1)):
        width = 4 * G * S - 7 if S > 1 else max(4 * G - 5, 40)
        rows = max(2, min(5, (1 << 21) // width))
        x, r, g, b = make_inputs(op, rows, width, seed=17 * width + T + C)
        ref = reference(op, x, r, g, b)
        xd = shifted_input(x, shift)
        rd = shifted_input(r, shift) if r is not None else None
        for policy in (EXCHANGE | pol, EXCHANGE | pol | STREAM):
            plan = R.Plan(T, 0, C, T, 0, policy=policy)
            print_case("row exchange", op, rows, width, shift, plan)
            y = plain(op, xd, rd, g, b, plan, rows, width, shift).host()
            check(op, y, ref, f"{op} {width} shift {shift} {plan}")
            ws_y = run(op, x, r, g, b, plan=R.SplitPlan(threads=T, chunks=C, policy=policy), shift=shift)
            assert np.array_equal(y.view(np.uint32), ws_y.view(np.uint32)), f"{op} {width} {plan}"


@pytest.mark.parametrize("op", MATRIX_OPS)
def test_row_exchange_y_at_every_phase(op):
    """x at one 16-byte phase, y (and so the row's words) at each of the four;
    r at yet another for residual LayerNorm."""
    rows, width = 6, 4 * 2048 * 5 + 9
    x, r, g, b = make_inputs(op, rows, width, seed=301)
    ref = reference(op, x, r, g, b)
    xd = shifted_input(x, 2)
    rd = shifted_input(r, 1) if r is not None else None
    for y_shift in range(4):
        for policy in (EXCHANGE | STREAM, EXCHANGE | LDS | STREAM):
            plan = R.Plan(256, 0, 8, 256, 0, policy=policy)
            if not fits(op, 256, 8, policy):
                continue
            print_case("row exchange phase", op, y_shift, plan)
            y = plain(op, xd, rd, g, b, plan, rows, width, y_shift).host()
            check(op, y, ref, f"{op} y shift {y_shift} {plan}")


@pytest.mark.parametrize("op", ("layernorm_residual", "rmsnorm", "softmax"))
def test_row_exchange_special_values(op):
    """Rows of +-inf, NaN, huge and tiny values across segments: NaN exactly
    where the oracle has NaN, bitwise the workspace path."""
    rows, width = 8, 4 * 256 * 8 * 6 - 3
    x, r, g, b = make_inputs(op, rows, width, seed=911)
    x[0, :] = -np.inf                   # softmax: NaN row
    x[1, :30000] = -np.inf              # whole segments of -inf next to finite ones
    x[2, 9000] = np.nan
    x[3, 10] = np.inf
    x[4, :] = np.nan
    x[5, :] = 3.0
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    x[7, width - 10:] = 50.0            # the max sits in the last segment
    ref = reference(op, x, r, g, b)
    xd = shifted_input(x, 0)
    rd = shifted_input(r, 0) if r is not None else None
    pol = EXCHANGE | STREAM | (LDS if op == "softmax" else 0)
    C = 16 if op == "softmax" else 8
    if op.startswith("layernorm"):
        pol |= LDS
    plan = R.Plan(256, 0, C, 256, 0, policy=pol)
    print_case("row exchange special", op, plan)
    y = plain(op, xd, rd, g, b, plan, rows, width, 0).host()
    check(op, y, ref, f"{op} special {plan}")
    ws_y = run(op, x, r, g, b, plan=R.SplitPlan(threads=256, chunks=C, policy=pol))
    assert np.array_equal(y.view(np.uint32), ws_y.view(np.uint32))


@pytest.mark.parametrize("op", ("layernorm_residual", "softmax"))
def test_row_exchange_reused_output(op):
    """Two calls on one y: the second's words start from the clear kernel,
    not from the first call's outputs."""
    rows, width = 4, 4 * 256 * 8 * 9 + 1
    plan = R.Plan(256, 0, 8, 256, 0, policy=EXCHANGE | STREAM | (LDS if op.startswith("layernorm") else 0))
    out = Guarded(rows, width, 1)
    for seed in (5, 6):
        x, r, g, b = make_inputs(op, rows, width, seed=seed)
        ref = reference(op, x, r, g, b)
        print_case("row exchange reuse", op, seed)
        plain(op, shifted_input(x, 1), shifted_input(r, 1) if r is not None else None, g, b, plan, rows, width, 1,
              y=out)
        check(op, out.host(), ref, f"{op} call with seed {seed}")


def test_row_exchange_many_rows():
    """More (row, segment) workgroups than the device holds at once: rows
    whose segments start late still meet (every row's segments are adjacent
    in launch order)."""
    op = "rmsnorm"
    rows, width = 3000, 4 * 256 * 8 * 4 - 11
    x, r, g, b = make_inputs(op, rows, width, seed=44)
    xd = shifted_input(x, 0)
    plan = R.Plan(256, 0, 8, 256, 0, policy=EXCHANGE | STREAM)
    print_case("row exchange many rows", rows, width)
    y = plain(op, xd, None, None, None, plan, rows, width, 0).host()
    pick = np.unique(np.concatenate([np.arange(4), rows - 1 - np.arange(4),
                                     np.random.default_rng(3).integers(0, rows, 60)]))
    assert np.isfinite(y).all()
    assert_close(y[pick], reference(op, x[pick], None, None, None), "many rows")


# the chooser's plans for rows beyond the register window, and for large
# calls of narrower rows, at full size; affine LayerNorm keeps the head+tail
# kernels beyond the register window from 256 rows; small calls keep the row
# kernels.
FULL = [("softmax", 4096, 65536), ("rmsnorm", 2048, 131072), ("layernorm_residual", 1024, 65536),
        ("softmax", 64, 1 << 20), ("layernorm_residual", 256, 1 << 18), ("rmsnorm", 2048, 40000),
        ("softmax", 16, 65536), ("layernorm", 5461, 24576), ("layernorm_affine", 4096, 32768),
        ("layernorm_affine", 1024, 65536), ("rmsnorm", 6710, 20001), ("layernorm_residual", 600, 20480),
        ("softmax", 1024, 24576), ("layernorm_affine", 64, 1 << 20)]
EXPECT_EXCHANGE = {("layernorm_affine", 1024, 65536): False, ("rmsnorm", 6710, 20001): False,
                   ("layernorm_residual", 600, 20480): False, ("softmax", 1024, 24576): False}


@pytest.mark.parametrize("op,rows,width", FULL, ids=lambda v: str(v))
def test_chooser_full_size(op, rows, width):
    t = torch()
    dist = "normal" if op == "softmax" else "uniform"
    x = synthetic.random_matrix(rows + width, rows, width, dist)
    r = synthetic.random_matrix(rows + width + 1, rows, width, dist, tensor="r") \
        if op == "layernorm_residual" else None
    xd = shifted_input(x, 0)
    rd = shifted_input(r, 0) if r is not None else None
    out = Guarded(rows, width)
    g = b = gd = bd = None
    if op == "layernorm_affine":
        g, b = synthetic.affine_vectors(synthetic.Case(7, op, rows, width, "uniform"))
        gd, bd = t.from_numpy(g).cuda(), t.from_numpy(b).cuda()
    if op.startswith("layernorm"):
        p = R.rowred_layernorm_plan_query(xd, rd, gd, bd, out.y)
    else:
        p = R.rowred_plan_query(op, xd, rd, out.y)
    print_case("chooser", op, rows, width, p)
    assert bool(p.policy & EXCHANGE) == EXPECT_EXCHANGE.get((op, rows, width), True), p
    eps = synthetic.EPS.get("layernorm" if op.startswith("layernorm") else op, 0.0)
    if op.startswith("layernorm"):
        R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=eps)
    elif op == "rmsnorm":
        R.rowred_rmsnorm(xd, out.y, eps=eps)
    else:
        R.rowred_softmax(xd, out.y)
    t.cuda.synchronize()
    assert out.guards_intact()
    y = out.host()
    assert np.isfinite(y).all()
    pick = np.unique(np.concatenate([np.arange(2), rows - 1 - np.arange(2),
                                     np.random.default_rng(rows ^ width).integers(0, rows, 24)]))
    ref = oracle.run_op(op, x[pick], r[pick] if r is not None else None, eps=synthetic.EPS.get(
        "layernorm" if op.startswith("layernorm") else op), gamma=g, beta=b)
    assert_close(y[pick], ref, f"{op} {rows}x{width} {p}")


def test_graph_capture_and_replay():
    """Row exchange calls of three operators captured in one HIP graph (the
    words' clear is a kernel: no memset node), replayed with eager work and
    garbage written over y in between: every replay equals the eager results
    bitwise."""
    t = torch()
    rows, width = 6, 140001
    x = synthetic.random_matrix(506, rows, width, "normal")
    r = synthetic.random_matrix(507, rows, width, "normal", tensor="r")
    xd, rd = shifted_input(x, 1), shifted_input(r, 1)
    outs = [t.empty(rows, width, device="cuda") for _ in range(3)]
    plans = [R.Plan(256, 0, 8, 256, 0, policy=EXCHANGE | STREAM | LDS), R.Plan(256, 0, 8, 256, 0, policy=EXCHANGE | STREAM),
             R.Plan(256, 0, 16, 256, 0, policy=EXCHANGE | STREAM | LDS)]

    def calls():
        R.rowred_run_plan("layernorm_residual", xd, rd, outs[0], plans[0], eps=1e-5)
        R.rowred_run_plan("rmsnorm", xd, None, outs[1], plans[1], eps=1e-6)
        R.rowred_run_plan("softmax", xd, None, outs[2], plans[2])

    print_case("row exchange graph", rows, width)
    calls()
    t.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for i, op in enumerate(("layernorm_residual", "rmsnorm", "softmax")):
        check(op, eager[i].cpu().numpy(), reference(op, x, r if i == 0 else None, None, None), f"graph {op}")
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            calls()
    t.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for o in outs:
            o.view(t.int32).fill_(0x3F800000 + rep)  # nonzero garbage where the words go
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert t.equal(o.view(t.int32), e.view(t.int32)), (rep, i)
        calls()
        t.cuda.synchronize()


def test_two_streams_at_once():
    """Row exchange calls on two streams at the same time (softmax and
    residual LayerNorm through the plain entry points): the two kernels share
    the chip, every wait still ends, and every row is finite and matches the
    oracle on sampled rows, each replay bitwise the first."""
    t = torch()
    rows, width = 512, 65536
    xs = [synthetic.random_matrix(600 + i, rows, width, "normal") for i in range(2)]
    r = synthetic.random_matrix(602, rows, width, "normal", tensor="r")
    xd = [t.from_numpy(x).cuda() for x in xs]
    rd = t.from_numpy(r).cuda()
    ys = [t.empty(rows, width, device="cuda") for _ in range(2)]
    for op, x in (("softmax", xd[0]), ("layernorm_residual", xd[1])):
        p = R.rowred_plan_query(op, x, rd if op == "layernorm_residual" else None, ys[0])
        assert p.policy & EXCHANGE, (op, p)
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    first = None
    t.cuda.synchronize()
    for rep in range(3):
        print_case("row exchange two streams", rep)
        with t.cuda.stream(streams[0]):
            R.rowred_softmax(xd[0], ys[0])
        with t.cuda.stream(streams[1]):
            R.rowred_layernorm_residual(xd[1], rd, ys[1], eps=1e-5)
        t.cuda.synchronize()
        got = [y.cpu().numpy() for y in ys]
        assert all(np.isfinite(g).all() for g in got), rep
        if first is None:
            first = got
        else:
            assert all(np.array_equal(a.view(np.uint32), b.view(np.uint32)) for a, b in zip(first, got)), rep
    pick = [0, 255, 511]
    assert_close(first[0][pick], oracle.softmax(xs[0][pick]), "softmax stream 0")
    assert_close(first[1][pick], oracle.layernorm_residual(xs[1][pick], r[pick], 1e-5), "layernorm stream 1")
