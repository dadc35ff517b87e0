"""One-kernel split rows (ROWRED_POLICY_EXCHANGE) against the FP64 oracle:
every geometry up to 64 segments per row, ragged and misaligned rows, both
memory policies, IEEE special values, row blocks, workspace reuse after the
three-kernel path left it dirty, graph capture, and the status word (no wait
may give up).

Bar: |y - ref| <= 1e-5 + 1e-5 |ref|, NaN exactly where the oracle has NaN."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import assert_close, print_case, shifted_input, torch
from tests.test_gpu_split import c_op, check, make_inputs, reference, run

pytestmark = pytest.mark.gpu

MATRIX_OPS = ("layernorm_residual", "layernorm", "layernorm_affine", "rmsnorm", "softmax")
EXCHANGE = R.ROWRED_POLICY_EXCHANGE
STREAM = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES
LDS = R.ROWRED_POLICY_LDS_STRIPE
GEOMETRIES = [(64, 1), (64, 2), (128, 4), (256, 1), (256, 2), (512, 2), (1024, 1), (1024, 2), (1024, 4), (64, 8),
              (256, 8), (512, 8)]


def workspace(op, rows, width, plan, xd):
    t = torch()
    need = max(R.rowred_workspace_size(c_op(op), rows, width),
               R.rowred_split_plan_query(c_op(op), xd, plan=plan).workspace_bytes)
    ws = t.empty(need, dtype=t.uint8, device="cuda")
    ws.fill_(0xA5)  # garbage the clear kernel must zero
    return ws


def status_ok(ws):
    return int(ws[:8].view(torch().int64).item()) == 0


def assert_refused(op, x, r, g, b, plan):
    """A plan the library does not support: ROWRED_ERR_INVALID_ARG from the
    host-side query and from the run, with the output untouched."""
    t = torch()
    xd = shifted_input(x, 0)
    with pytest.raises(R.RowRedError) as e:
        R.rowred_split_plan_query(c_op(op), xd, plan=plan)
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG
    with pytest.raises(R.RowRedError) as e:
        run(op, x, r, g, b, plan=plan)
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG
    t.cuda.synchronize()


def run_exchange(op, x, r, g, b, plan, shift=0):
    ws = workspace(op, x.shape[0], x.shape[1], plan, shifted_input(x, shift))
    got = run(op, x, r, g, b, plan=plan, shift=shift, ws=ws)
    assert status_ok(ws), f"{op} {x.shape} {plan}: a wait gave up"
    return got


@pytest.mark.parametrize("geom", GEOMETRIES, ids=lambda g: f"T{g[0]}C{g[1]}")
@pytest.mark.parametrize("op", MATRIX_OPS)
def test_every_exchange_geometry(op, geom):
    """One, three, 32 and the most (min(128, T)) segments per row; ragged,
    misaligned."""
    T, C = geom
    if C == 8 and op.startswith("layernorm"):
        # LayerNorm exchanges at up to 4 chunks: the plan is refused before
        # anything runs
        x, r, g, b = make_inputs(op, 2, 40000, seed=5)
        assert_refused(op, x, r, g, b, R.SplitPlan(threads=T, chunks=C, policy=EXCHANGE))
        return
    G = T * C
    for width, shift in ((1000, 1), (4 * G * 3 - 7, 3), (4 * G * 32 - 5, 1), (4 * G * min(128, T) - 9, 2)):
        rows = max(2, min(6, (1 << 21) // width))
        x, r, g, b = make_inputs(op, rows, width, seed=11 * width + T + C)
        ref = reference(op, x, r, g, b)
        for policy in (EXCHANGE, EXCHANGE | STREAM):
            plan = R.SplitPlan(threads=T, chunks=C, policy=policy)
            print_case("exchange", op, rows, width, shift, plan)
            check(op, run_exchange(op, x, r, g, b, plan, shift=shift), ref, f"{op} {width} {plan}")


LDS_STRIPES = [8, 12, 16]  # 4 + 4, 8 + 4 and 8 + 8 slots per lane (registers + LDS), 256 threads


@pytest.mark.parametrize("chunks", LDS_STRIPES, ids=lambda c: f"C{c}")
@pytest.mark.parametrize("op", MATRIX_OPS)
def test_lds_stripe_exchange(op, chunks):
    """Exchange kernels with part of each segment in LDS: one, three and 128
    segments per row, ragged, misaligned (r and y at another 16-byte phase
    than x too), both memory policies."""
    G = 256 * chunks
    for width, shift in ((1000, 1), (4 * G * 3 - 7, 3), (4 * G * 128 - 9, 2)):
        rows = max(2, min(6, (1 << 21) // width))
        x, r, g, b = make_inputs(op, rows, width, seed=13 * width + chunks)
        ref = reference(op, x, r, g, b)
        for policy in (EXCHANGE | LDS, EXCHANGE | LDS | STREAM):
            plan = R.SplitPlan(threads=256, chunks=chunks, policy=policy)
            print_case("exchange lds", op, rows, width, shift, plan)
            check(op, run_exchange(op, x, r, g, b, plan, shift=shift), ref, f"{op} {width} {plan}")


@pytest.mark.parametrize("chunks", LDS_STRIPES, ids=lambda c: f"C{c}")
def test_lds_stripe_misaligned_residual(chunks):
    """LayerNorm with r at another 16-byte phase than x: the LDS slots of r are
    filled by 4-byte loads."""
    t = torch()
    rows, width = 5, 40003 + 20000 * (chunks // 8 - 1)
    x, r, g, b = make_inputs("layernorm_residual", rows, width, seed=77 + chunks)
    ref = reference("layernorm_residual", x, r, None, None)
    xd, rd = shifted_input(x, 1), shifted_input(r, 3)
    out = t.empty(rows, width, device="cuda")
    plan = R.SplitPlan(threads=256, chunks=chunks, policy=EXCHANGE | LDS | STREAM)
    ws = workspace("layernorm_residual", rows, width, plan, xd)
    R.rowred_split_run_plan("layernorm_residual", xd, rd, None, None, out, None, plan, ws, eps=1e-5)
    t.cuda.synchronize()
    assert status_ok(ws)
    check("layernorm_residual", out.cpu().numpy(), ref, "misaligned r")


@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm"])
def test_special_values(op):
    rows, width = 8, 5000
    x = synthetic.random_matrix(93, rows, width, "normal")
    x[0, :] = -np.inf                   # softmax: NaN row
    x[1, :2600] = -np.inf               # whole segments of -inf next to finite ones
    x[2, 4000] = np.nan
    x[3, 10] = np.inf
    x[4, :] = np.nan
    x[5, :] = 3.0
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    x[7, 4990:] = 50.0                  # the max sits in the last segment
    ref = reference(op, x, None, None, None)
    # 128-granule segments (10 per row), and 8 + 8 LDS-stripe ones (2 per row)
    for plan in (R.SplitPlan(threads=64, chunks=2, policy=EXCHANGE),
                 R.SplitPlan(threads=256, chunks=16, policy=EXCHANGE | LDS)):
        got = run_exchange(op, x, None, None, None, plan)
        check(op, got, ref, f"{op} special {plan}")
    if op == "softmax":
        assert np.isnan(got[0]).all() and not np.isnan(got[1]).any()
        assert np.abs(got[1].astype(np.float64).sum() - 1.0) < 1e-5


@pytest.mark.parametrize("op", MATRIX_OPS)
def test_row_blocks_and_determinism(op):
    """Blocks of rows give bitwise the one-pass result; so does a second
    call through a workspace the three-kernel path has just filled."""
    t = torch()
    rows, width, shift = 7, 33001, 2
    x, r, g, b = make_inputs(op, rows, width, seed=34)
    plan = R.SplitPlan(threads=256, chunks=2, policy=EXCHANGE | STREAM)
    whole = run_exchange(op, x, r, g, b, plan, shift=shift)
    check(op, whole, reference(op, x, r, g, b), f"{op} one pass")
    for br in (1, 3, 6):
        bp = R.SplitPlan(threads=256, chunks=2, policy=EXCHANGE | STREAM, block_rows=br)
        got = run_exchange(op, x, r, g, b, bp, shift=shift)
        assert np.array_equal(np.asarray(got).view(np.uint32), np.asarray(whole).view(np.uint32)), (op, br)
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    run(op, x, r, g, b, plan=R.SplitPlan(threads=256, chunks=2, policy=STREAM), shift=shift, ws=ws)
    again = run(op, x, r, g, b, plan=plan, shift=shift, ws=ws)
    assert status_ok(ws)
    assert np.array_equal(np.asarray(again).view(np.uint32), np.asarray(whole).view(np.uint32))


@pytest.mark.parametrize("op", ["softmax", "rmsnorm", "layernorm_residual"])
def test_agrees_with_three_kernel_split(op):
    """Same rows through both split paths: within the bar of each other (the
    summation orders differ), each within the bar of the oracle."""
    x, r, g, b = make_inputs(op, 9, 250001, seed=55, dist="uniform")
    ref = reference(op, x, r, g, b)
    a = run_exchange(op, x, r, g, b, R.SplitPlan(threads=1024, chunks=4, policy=EXCHANGE | STREAM), shift=1)
    s = run(op, x, r, g, b, plan=R.SplitPlan(threads=256, chunks=2, policy=STREAM), shift=1)
    check(op, a, ref, f"{op} exchange")
    check(op, s, ref, f"{op} three kernels")
    assert_close(a, s.astype(np.float64), f"{op} exchange vs three kernels")


def test_graph_capture_and_replay():
    """Clear and exchange kernels of three calls captured in one HIP graph
    with a shared workspace (a kernel clears it: no memset node), replayed
    with eager work in between; every replay equals the eager results
    bitwise and leaves the status word clear."""
    t = torch()
    rows, width = 5, 140001
    x = synthetic.random_matrix(406, rows, width, "normal")
    r = synthetic.random_matrix(407, rows, width, "normal", tensor="r")
    xd, rd = shifted_input(x, 3), shifted_input(r, 3)
    ws = t.empty(1 << 20, dtype=t.uint8, device="cuda")
    outs = [t.empty(rows, width, device="cuda") for _ in range(3)]
    plan = R.SplitPlan(threads=512, chunks=2, policy=EXCHANGE | STREAM)

    def calls():
        R.rowred_split_run_plan("layernorm_residual", xd, rd, None, None, outs[0], None, plan, ws, eps=1e-5)
        R.rowred_split_run_plan("rmsnorm", xd, None, None, None, outs[1], None, plan, ws, eps=1e-6)
        R.rowred_split_run_plan("softmax", xd, None, None, None, outs[2], None, plan, ws)

    calls()
    t.cuda.synchronize()
    assert status_ok(ws)
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
            o.fill_(float("nan"))
        ws.fill_(0x5A)
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert status_ok(ws), rep
        for i, (o, e) in enumerate(zip(outs, eager)):
            assert t.equal(o.view(t.int32), e.view(t.int32)), (rep, i)
        calls()
        t.cuda.synchronize()


@pytest.mark.parametrize("case", [c for c in synthetic.NEXT_WORKLOADS.get(9, []) + synthetic.NEXT_WORKLOADS.get(10, [])
                                  if c.op in ("softmax", "rmsnorm", "layernorm_residual")],
                         ids=lambda c: c.name)
def test_full_size_wide_rows(case):
    """The wide-row workload shapes at full size through an exchange plan
    with 1024 x 4 segments; sampled rows against the oracle."""
    t = torch()
    print_case("exchange", case.name)
    x = synthetic.case_input(case, "x")
    r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
    plan = R.SplitPlan(threads=1024, chunks=4, policy=EXCHANGE | STREAM)
    got = run_exchange(case.op, x, r, None, None, plan)
    for i in sorted({0, case.rows // 2, case.rows - 1}):
        ref = reference(case.op, x[i:i + 1], r[i:i + 1] if r is not None else None, None, None)
        check(case.op, got[i:i + 1], ref, f"{case.name} row {i}")
    del got
    t.cuda.empty_cache()


@pytest.mark.parametrize("width", [32769, 65536, 100003, 262147])
@pytest.mark.parametrize("op", MATRIX_OPS)
def test_ws_entry_chooses_exchange(op, width):
    """Beyond the register-resident window the _ws entry points pick an
    exchange plan for the matrix operators; through a workspace full of
    garbage the results match the oracle and the status word stays clear."""
    t = torch()
    rows = 3
    x, r, g, b = make_inputs(op, rows, width, seed=width + 5)
    xd = shifted_input(x, width % 4)
    plan = R.rowred_split_plan_query(c_op(op), xd)
    assert plan.policy & EXCHANGE, plan
    ws = t.empty(R.rowred_workspace_size(c_op(op), rows, width), dtype=t.uint8, device="cuda")
    ws.fill_(0xFF)
    got = run(op, x, r, g, b, shift=width % 4, ws=ws)
    assert status_ok(ws)
    check(op, got, reference(op, x, r, g, b), f"{op} {rows}x{width}")


def test_two_streams_at_once():
    """Exchange calls on two streams at the same time, each with its own
    workspace: the two kernels share the chip, every wait still ends (status
    words clear) and both match the oracle on sampled rows."""
    t = torch()
    rows, width = 512, 65536
    xs = [synthetic.random_matrix(500 + i, rows, width, "normal") for i in range(2)]
    xd = [t.from_numpy(x).cuda() for x in xs]
    ys = [t.empty(rows, width, device="cuda") for _ in range(2)]
    ws = [R.new_workspace(op, rows, width) for op in ("softmax", "rmsnorm")]
    for w in ws:
        w.fill_(0x77)
    streams = [t.cuda.Stream(), t.cuda.Stream()]
    t.cuda.synchronize()
    for rep in range(3):
        with t.cuda.stream(streams[0]):
            R.rowred_softmax_ws(xd[0], ys[0], ws[0])
        with t.cuda.stream(streams[1]):
            R.rowred_rmsnorm_ws(xd[1], ys[1], ws[1], eps=1e-6)
    t.cuda.synchronize()
    assert all(status_ok(w) for w in ws)
    for i, op in enumerate(("softmax", "rmsnorm")):
        yh = ys[i].cpu().numpy()
        for rr in (0, 255, 511):
            check(op, yh[rr:rr + 1], reference(op, xs[i][rr:rr + 1], None, None, None), f"{op} stream {i} row {rr}")


def test_wait_give_up_path():
    """The bounded wait's give-up path, forced from the host: an explicit plan
    with wait_polls = 1 gives up after one empty re-poll, so every kernel
    still ends.  Then each output is either NaN (its segment gave up) or the
    oracle's value (its segment saw every record); some segment gives up and
    raises the status word.  The next call through the entry point (the
    default bound), on the same workspace, clears the word and is exact."""
    t = torch()
    rows, width = 256, 65536
    gave_up = False
    for op in ("softmax", "rmsnorm", "layernorm_residual"):
        x, r, g, b = make_inputs(op, rows, width, seed=4242)
        ref = reference(op, x, r, g, b)
        plan = R.rowred_split_plan_query(c_op(op), shifted_input(x, 0))
        assert plan.policy & EXCHANGE and plan.segments > 1
        ws = workspace(op, rows, width, plan, shifted_input(x, 0))
        plan.wait_polls = 1
        print_case("exchange give-up", op, rows, width, plan)
        got = run(op, x, r, g, b, plan=plan, ws=ws)
        status = int(ws[:8].view(t.int64).item())
        nan = np.isnan(got)
        ok = ~nan & ~np.isnan(ref)
        assert np.all(np.abs(got[ok] - ref[ok]) <= 1e-5 + 1e-5 * np.abs(ref[ok])), op
        assert status in (0, 1)
        assert (status == 1) == bool(nan.any()), (op, status, int(nan.sum()))
        gave_up |= status == 1
        print_case("exchange after give-up", op)
        again = run(op, x, r, g, b, ws=ws)
        assert status_ok(ws)
        assert_close(again, ref, f"{op} after a give-up")
    assert gave_up, "no wait gave up at wait_polls = 1"


def test_status_survives_row_blocks():
    """A call in row blocks zeroes the status word once: a give-up in the
    first block stays visible after the later blocks ran."""
    t = torch()
    rows, width = 64, 65536
    x, r, g, b = make_inputs("softmax", rows, width, seed=4343)
    plan = R.rowred_split_plan_query(c_op("softmax"), shifted_input(x, 0))
    assert plan.policy & EXCHANGE
    ws = workspace("softmax", rows, width, plan, shifted_input(x, 0))
    for _ in range(3):
        plan.wait_polls = 1
        plan.block_rows = rows // 4
        print_case("exchange blocks give-up", plan)
        got = run("softmax", x, r, g, b, plan=plan, ws=ws)
        status = int(ws[:8].view(t.int64).item())
        nan_rows = np.isnan(got).any(axis=1)
        assert (status == 1) == bool(nan_rows.any()), (status, int(nan_rows.sum()))
    plan.wait_polls = 0
    got = run("softmax", x, r, g, b, plan=plan, ws=ws)
    assert status_ok(ws)
    assert_close(got, reference("softmax", x, r, g, b), "softmax blocks after give-up")
