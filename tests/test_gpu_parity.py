"""Parity of the HIP path (through the C ABI) with the FP64 oracle.

Every comparison is element by element at |y - ref| <= 1e-5 + 1e-5 |ref|
(NaN exactly where the oracle has NaN), with sentinel guard bands around the
output that must stay untouched.
"""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, all_plans, assert_close, dev, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

OPS = ("layernorm_residual", "rmsnorm", "softmax")


def run_case(op, x, r=None, eps=None, shift=(0, 0, 0), plan=None):
    """Run `op` on the GPU with x / r / y placed `shift` floats off 16-byte
    alignment; return the host result after checking the guard bands."""
    rows, width = x.shape
    xd = shifted_input(x, shift[0])
    rd = shifted_input(r, shift[1]) if r is not None else None
    out = Guarded(rows, width, shift[2])
    if eps is None:
        eps = synthetic.EPS.get(op, 0.0)
    if plan is None:
        R.run_op(op, xd, rd, out.y, eps=eps)
    else:
        R.rowred_run_plan(op, xd, rd, out.y, plan, eps=eps)
    torch().cuda.synchronize()
    assert out.guards_intact(), f"{op} {x.shape} wrote outside y"
    return out.host()


def oracle_of(op, x, r=None, eps=None):
    if eps is None:
        eps = synthetic.EPS.get(op)
    return oracle.run_op(op, x, r, eps=eps)


def inputs(op, rows, width, seed, dist="uniform"):
    x = synthetic.random_matrix(seed, rows, width, dist)
    r = synthetic.random_matrix(seed + 1, rows, width, dist, tensor="r") if op == "layernorm_residual" else None
    return x, r


# ---------------------------------------------------------------------------
# Ragged widths, row tails, every op
# ---------------------------------------------------------------------------

WIDTHS = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 33, 63, 64, 65, 127, 128, 129, 255, 257, 511, 513, 1023, 1024,
          1025, 1537, 2047, 2049, 4095, 4096, 4097, 8191, 8192, 8193, 12288, 16383, 16384, 32765, 32768]


@pytest.mark.parametrize("width", WIDTHS)
@pytest.mark.parametrize("op", OPS)
def test_ragged_widths(op, width):
    # rows: enough to cover several workgroups plus a partial last one
    p = R.rowred_plan_query(op, 0x10000, 0x20000000000 if op == "layernorm_residual" else None,
                            0x40000000000, rows=1000, width=width)
    rows = min(3 * p.rows_per_group + 1, max(2, (1 << 21) // width))
    print_case(op, rows, width)
    x, r = inputs(op, rows, width, seed=100 + width, dist="normal")
    assert_close(run_case(op, x, r), oracle_of(op, x, r), f"{op} {rows}x{width}")


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("width", [127, 257, 1537])
def test_row_tails(op, width):
    """rows = P-1, P, P+1 and 2P+3 around the rows packed per workgroup."""
    p = R.rowred_plan_query(op, 0x10000, 0x20000000000 if op == "layernorm_residual" else None,
                            0x40000000000, rows=1000, width=width)
    P = p.rows_per_group
    for rows in sorted({1, max(1, P - 1), P, P + 1, 2 * P + 3}):
        print_case(op, rows, width)
        x, r = inputs(op, rows, width, seed=7 * rows + width)
        assert_close(run_case(op, x, r), oracle_of(op, x, r), f"{op} {rows}x{width}")


# ---------------------------------------------------------------------------
# Pointer alignment: x, r, y at every phase of the 16-byte grid
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("shift", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (0, 1, 2), (3, 0, 1), (1, 3, 0), (2, 0, 0),
                                   (0, 0, 3)])
@pytest.mark.parametrize("width", [5, 127, 256, 1537, 4096])
def test_misaligned_pointers(op, shift, width):
    rows = 37
    print_case(op, shift, width)
    x, r = inputs(op, rows, width, seed=3 * width + sum(shift))
    assert_close(run_case(op, x, r, shift=shift), oracle_of(op, x, r), f"{op} shift {shift} width {width}")


def test_misaligned_widest_row():
    # 32764 columns shifted by 3 floats span exactly 8192 granules.
    x, _ = inputs("softmax", 3, 32764, seed=5)
    assert_close(run_case("softmax", x, shift=(3, 0, 3)), oracle_of("softmax", x), "softmax 32764 shift 3")


# ---------------------------------------------------------------------------
# Every launch geometry gives the same answer
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("width", [3, 5, 100, 257, 1000, 4096])
def test_every_plan(op, width):
    rows = 67
    x, r = inputs(op, rows, width, seed=11 * width)
    ref = oracle_of(op, x, r)
    window = (width + 3 + 3) // 4
    n = 0
    for plan in all_plans(window):
        print_case(op, width, plan)
        assert_close(run_case(op, x, r, plan=plan, shift=(1, 1, 1)), ref, f"{op} {width} {plan}")
        n += 1
    assert n >= 3


@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("width", [1, 2, 3, 4, 5, 6, 7, 9, 127, 129, 255, 257, 513, 1023])
@pytest.mark.parametrize("shift", [0, 1, 3])
def test_staged_stores(op, width, shift):
    """Outputs assembled in LDS and stored as whole granules: several
    geometries, rows that end the matrix mid-workgroup, every phase."""
    window = (width + 3 + 3) // 4
    for L in (1, 4, 8, 16, 32, 64, 128, 256):
        C = next((c for c in (1, 2, 3, 4) if L * c >= window), None)
        if C is None:
            continue
        for T in (64, 256, 512):
            if T < L:
                continue
            P = T // L
            for rows in sorted({1, 2, P - 1, P, P + 1, 2 * P + 3} - {0}):
                x, r = inputs(op, rows, width, seed=width * 131 + rows + shift)
                plan = R.Plan(lanes_per_row=L, rows_per_group=0, chunks=C, threads=T, grid=0,
                              policy=R.ROWRED_POLICY_STAGE_STORES | R.ROWRED_POLICY_NT_STORES)
                print_case(op, width, shift, L, C, T, rows)
                assert_close(run_case(op, x, r, plan=plan, shift=(shift, shift, shift)), oracle_of(op, x, r),
                             f"{op} staged w{width} L{L} C{C} T{T} rows {rows} shift {shift}")


# ---------------------------------------------------------------------------
# Determinism, streams, graphs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("op", OPS)
def test_three_dispatches_bitwise_identical(op):
    x, r = inputs(op, 512, 3000, seed=9)
    xd = dev(x)
    rd = dev(r) if r is not None else None
    outs = []
    for _ in range(3):
        o = Guarded(512, 3000)
        R.run_op(op, xd, rd, o.y)
        outs.append(o)
    torch().cuda.synchronize()
    ys = [o.host() for o in outs]
    assert all(o.guards_intact() for o in outs)
    assert np.array_equal(ys[0].view(np.uint32), ys[1].view(np.uint32))
    assert np.array_equal(ys[0].view(np.uint32), ys[2].view(np.uint32))
    assert_close(ys[0], oracle_of(op, x, r), op)


@pytest.mark.parametrize("op", OPS)
def test_side_stream(op):
    t = torch()
    x, r = inputs(op, 300, 777, seed=13)
    xd = dev(x)
    rd = dev(r) if r is not None else None
    t.cuda.synchronize()
    s = t.cuda.Stream()
    o = Guarded(300, 777)
    with t.cuda.stream(s):
        R.run_op(op, xd, rd, o.y)
    s.synchronize()
    assert o.guards_intact()
    assert_close(o.host(), oracle_of(op, x, r), op)


def test_graph_capture_and_replay():
    """All three entry points captured in one HIP graph (they enqueue no
    memset and allocate nothing), replayed several times with eager work in
    between; every replay matches the eager result bitwise."""
    t = torch()
    rows, width = 256, 2049
    x = synthetic.random_matrix(21, rows, width, "normal")
    r = synthetic.random_matrix(22, rows, width, "normal", tensor="r")
    xd, rd = dev(x), dev(r)
    ys = [t.empty(rows, width, device="cuda") for _ in range(3)]
    eager = [t.empty(rows, width, device="cuda") for _ in range(3)]
    R.rowred_layernorm_residual(xd, rd, eager[0])
    R.rowred_rmsnorm(xd, eager[1])
    R.rowred_softmax(xd, eager[2])
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    s = t.cuda.Stream()
    s.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            R.rowred_layernorm_residual(xd, rd, ys[0])
            R.rowred_rmsnorm(xd, ys[1])
            R.rowred_softmax(xd, ys[2])
    t.cuda.current_stream().wait_stream(s)
    for k in range(4):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        t.cuda.synchronize()
        for y, e in zip(ys, eager):
            assert t.equal(y.view(t.int32), e.view(t.int32)), f"replay {k}"
        _ = (xd * 2).sum().item()  # eager work between replays
    assert_close(eager[0].cpu().numpy(), oracle.layernorm_residual(x, r, 1e-5), "graph ln")
    assert_close(eager[1].cpu().numpy(), oracle.rmsnorm(x, 1e-6), "graph rms")
    assert_close(eager[2].cpu().numpy(), oracle.softmax(x), "graph softmax")


# ---------------------------------------------------------------------------
# Special values and degenerate rows
# ---------------------------------------------------------------------------

def test_softmax_special_rows():
    w = 300
    x = synthetic.random_matrix(31, 8, w, "normal")
    x[0, :] = -np.inf                    # all -inf -> NaN row
    x[1, 5] = np.inf                     # +inf -> NaN row
    x[2, 7] = np.nan                     # NaN -> NaN row
    x[3, :] = 0.0                        # uniform -> 1/w
    x[4, ::2] = -np.inf                  # half the row masked
    x[5, :] += np.float32(1000.0)        # large offset: max subtraction needed
    x[6, :] = -1000.0
    x[6, 17] = 1000.0                    # one-hot
    y = run_case("softmax", x)
    assert_close(y, oracle.softmax(x), "softmax special rows")
    assert np.isnan(y[0]).all() and np.isnan(y[1]).all() and np.isnan(y[2]).all()
    assert (y[4, ::2] == 0).all()
    assert y[6, 17] == 1.0


def test_layernorm_special_rows():
    w = 513
    x = synthetic.random_matrix(41, 6, w, "uniform")
    r = synthetic.random_matrix(42, 6, w, "uniform", tensor="r")
    x[0, :] = 3.0
    r[0, :] = 0.5                        # constant combined row -> 0
    x[1, :] = -r[1, :]                   # x + r == 0 exactly -> 0
    x[2, :] += np.float32(1000.0)        # large common offset
    x[3, 9] = np.nan
    y = run_case("layernorm_residual", x, r)
    assert_close(y, oracle.layernorm_residual(x, r, 1e-5), "ln special rows")
    assert np.abs(y[0]).max() <= 1e-5 and np.abs(y[1]).max() <= 1e-5
    assert np.isnan(y[3]).all()


@pytest.mark.parametrize("width", [2, 3, 16, 257, 4096])
def test_layernorm_ill_conditioned_rows(width):
    """Rows whose spread is far below their magnitude: the centring must stay
    accurate to FP32 rounding of the centred value itself."""
    rng = np.random.default_rng(width)
    rows = 12
    x = np.empty((rows, width), np.float32)
    r = np.empty((rows, width), np.float32)
    n = lambda: rng.standard_normal(width)
    x[0], r[0] = 1e4 + n(), -1e4 + n()                    # large x and r that cancel
    x[1], r[1] = 1000 + 1e-3 * n(), 0.0                   # tiny spread on a large mean
    x[2], r[2] = 1 + 1e-4 * n(), 1e-4 * n()               # variance ~1e-8 << eps
    x[3], r[3] = 1 + 3e-3 * n(), 0.0                      # variance ~ eps
    x[4], r[4] = -5e3 + 10 * n(), 5e3 + 10 * n()
    x[5], r[5] = 1 + 2.0 ** -20 * n(), 2.0 ** -22 * n()
    x[6], r[6] = 3e7 + n(), -3e7 + n()                    # inputs beyond 2^24: x + r not exact in FP32
    x[7], r[7] = n() * 1e-15, n() * 1e-15                 # tiny values (squares stay above FLT_MIN)
    x[8:], r[8:] = rng.uniform(-1, 1, (rows - 8, width)), rng.uniform(-1, 1, (rows - 8, width))
    for eps in (1e-5, 0.0):
        y = run_case("layernorm_residual", x, r, eps=eps)
        ref = oracle.layernorm_residual(x, r, eps)
        assert_close(y, ref, f"ill-conditioned LN width {width} eps {eps}")
    xp = (x.astype(np.float64) + r).astype(np.float32)
    out = Guarded(rows, width)
    R.rowred_layernorm(dev(xp), None, None, None, out.y, eps=1e-5)
    torch().cuda.synchronize()
    assert_close(out.host(), oracle.layernorm(xp, None, eps=1e-5), f"ill-conditioned plain LN width {width}")


def test_layernorm_eps_zero_constant_row_is_nan():
    x = np.full((2, 64), 2.0, np.float32)
    x[1] = np.arange(64, dtype=np.float32)
    r = np.zeros_like(x)
    y = run_case("layernorm_residual", x, r, eps=0.0)
    assert np.isnan(y[0]).all()
    assert_close(y[1:], oracle.layernorm_residual(x[1:], r[1:], 0.0), "ln eps 0")


def test_rmsnorm_special_rows():
    w = 129
    x = synthetic.random_matrix(51, 5, w, "normal")
    x[0, :] = 0.0                        # zero row -> 0
    x[1, :] = 1e-20                      # tiny row: eps dominates
    x[2, :] *= np.float32(1e15)          # huge row (sum of squares ~1e32, finite)
    x[3, 0] = np.inf                     # inf -> NaN/inf propagation like the oracle
    y = run_case("rmsnorm", x, eps=1e-6)
    assert_close(y, oracle.rmsnorm(x, 1e-6), "rms special rows")
    assert (y[0] == 0).all()


def test_empty_inputs_launch_nothing():
    t = torch()
    x = t.empty(0, 128, device="cuda")
    y = t.empty(0, 128, device="cuda")
    R.rowred_softmax(x, y)
    R.rowred_rmsnorm(x, y)
    x2 = t.empty(5, 0, device="cuda")
    R.rowred_layernorm_residual(x2, x2, t.empty(5, 0, device="cuda"))
    t.cuda.synchronize()


def test_copy_probe():
    t = torch()
    x = dev(synthetic.random_matrix(61, 1000, 1024, "normal"))
    y = t.empty_like(x)
    R.rowred_copy(x, y)
    t.cuda.synchronize()
    assert t.equal(x, y)


# ---------------------------------------------------------------------------
# Workloads at full size
# ---------------------------------------------------------------------------

def _blocks(rows, blk):
    for s in range(0, rows, blk):
        yield s, min(rows, s + blk)


@pytest.mark.parametrize("case", list(synthetic.all_cases()), ids=lambda c: c.name)
def test_workload_full_size(case):
    """Every configured workload at its full shape, in the launch geometry the
    chooser (and the benchmark) uses, compared element by element."""
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
    xd = dev(x)
    rd = dev(r) if r is not None else None
    out = Guarded(case.rows, case.width)
    R.run_op(case.op, xd, rd, out.y, eps=case.eps)
    torch().cuda.synchronize()
    assert out.guards_intact()
    del xd, rd
    y = out.host()
    blk = max(1, (1 << 24) // case.width)
    for s, t in _blocks(case.rows, blk):
        ref = oracle_of(case.op, x[s:t], r[s:t] if r is not None else None, case.eps)
        assert_close(y[s:t], ref, f"{case.name} rows {s}:{t}")
    if case.op == "softmax":
        sums = y.astype(np.float64).sum(axis=1)
        np.testing.assert_allclose(sums, 1.0, atol=1e-4)
