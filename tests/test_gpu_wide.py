"""LDS-stripe kernels (ROWRED_POLICY_LDS_STRIPE): RMSNorm and softmax rows of
4097-8192 granules, slots 0-3 of each lane in registers and the rest loaded
straight into LDS.  Same arithmetic in the same order as the register-resident
kernel with the same stripe: the results must be bitwise equal to it, and so
within the oracle's bar (|y - ref| <= 1e-5 + 1e-5 |ref|)."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch
from tests.test_gpu_parity import oracle_of

pytestmark = pytest.mark.gpu

LDS = R.ROWRED_POLICY_LDS_STRIPE


def run(op, xd, plan, rows, width, shift, y_shift=None):
    out = Guarded(rows, width, shift if y_shift is None else y_shift)
    R.rowred_run_plan(op, xd, None, out.y, plan, eps=synthetic.EPS.get(op, 0.0))
    torch().cuda.synchronize()
    assert out.guards_intact(), f"{op} {rows}x{width} wrote outside y"
    return out.host()


@pytest.mark.parametrize("width", [16385, 20000, 24576, 28673, 32765, 32768])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_matches_register_stripe_bitwise(op, width):
    """Every stripe length 5-8, ragged and misaligned rows (y at x's phase and
    at another), both memory policies, XCD remap."""
    rows = 37
    x = synthetic.random_matrix(width + 11, rows, width, "normal")
    ref = oracle_of(op, x)
    for shift, y_shift in ((0, 0), (1, 1), (3, 2)):
        xd = shifted_input(x, shift)
        C = -(-((width + shift + 3) // 4) // 1024)
        if C > 8:
            continue  # a window of 8193 granules: beyond the register-resident kernels
        for pol in (0, R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP):
            base = R.Plan(1024, 0, C, 1024, 0, policy=pol)
            wide = R.Plan(1024, 0, C, 1024, 0, policy=pol | LDS)
            print_case("lds stripe", op, width, shift, y_shift, wide)
            y0 = run(op, xd, base, rows, width, shift, y_shift)
            y1 = run(op, xd, wide, rows, width, shift, y_shift)
            assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{op} {width} {shift} {wide}"
            assert_close(y1, ref, f"{op} {width} {wide}")


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_special_values(op):
    rows, width = 8, 32768
    x = synthetic.random_matrix(95, rows, width, "normal")
    x[0, :] = -np.inf
    x[1, :20000] = -np.inf             # the max sits in the LDS slots
    x[2, 30000] = np.nan
    x[3, 17] = np.inf
    x[4, :] = np.nan
    x[5, :] = 3.0
    x[6, 31000:] = 60.0                # large values in the LDS slots only
    x[7, ::2] = 1e15
    x[7, 1::2] = -1e15
    xd = shifted_input(x, 0)
    base = run(op, xd, R.Plan(1024, 0, 8, 1024, 0, policy=0), rows, width, 0)
    wide = run(op, xd, R.Plan(1024, 0, 8, 1024, 0, policy=LDS), rows, width, 0)
    assert np.array_equal(base.view(np.uint32), wide.view(np.uint32))
    assert_close(wide, oracle_of(op, x), f"{op} special")


@pytest.mark.parametrize("case", synthetic.CORE_WORKLOADS[5], ids=lambda c: c.name)
def test_full_size_stress(case):
    """The softmax stress workload at full size through the LDS stripe:
    bitwise the register-resident result."""
    t = torch()
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    xd = t.from_numpy(x).cuda()
    y0 = t.empty_like(xd)
    y1 = t.empty_like(xd)
    pol = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP
    R.rowred_run_plan(case.op, xd, None, y0, R.Plan(1024, 0, 8, 1024, 0, policy=pol))
    R.rowred_run_plan(case.op, xd, None, y1, R.Plan(1024, 0, 8, 1024, 0, policy=pol | LDS))
    t.cuda.synchronize()
    assert t.equal(y0.view(t.int32), y1.view(t.int32))
    for i in (0, case.rows // 2, case.rows - 1):
        assert_close(y1[i:i + 1].cpu().numpy(), oracle_of(case.op, x[i:i + 1]), f"{case.name} row {i}")
    del y0, y1, xd
    t.cuda.empty_cache()


@pytest.mark.parametrize("width", [32769, 40000, 50257, 61440, 65533, 65536])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_rows_held_in_registers_and_lds(op, width):
    """Rows of 8193-16384 granules (9-16 slots per lane: 8 in registers, the
    rest in LDS), through the plain entry point and as explicit plans with
    both memory policies, ragged and misaligned: the oracle's bar, and within
    it of the looped kernels, which read the row twice."""
    t = torch()
    rows = 9
    x = synthetic.random_matrix(width + 21, rows, width, "normal")
    ref = oracle_of(op, x)
    for shift, y_shift in ((0, 0), (2, 2), (1, 3)):
        if (width + shift + 3) // 4 > 16384:
            continue
        xd = shifted_input(x, shift)
        C = -(-((width + shift + 3) // 4) // 1024)
        plan = R.rowred_plan_query(op, xd, None, Guarded(rows, width, y_shift).y)
        # the entry point: the exchange kernels (words in y's rows) where the
        # device holds a row's segments, else the LDS stripe
        assert (plan.policy & LDS and plan.chunks == C) or plan.policy & R.ROWRED_POLICY_EXCHANGE, plan
        out = Guarded(rows, width, y_shift)
        if op == "rmsnorm":
            R.rowred_rmsnorm(xd, out.y, eps=synthetic.EPS["rmsnorm"])
        else:
            R.rowred_softmax(xd, out.y)
        t.cuda.synchronize()
        assert out.guards_intact()
        assert_close(out.host(), ref, f"{op} {width} entry point")
        for pol in (0, R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP):
            wide = R.Plan(1024, 0, C, 1024, 0, policy=pol | LDS)
            print_case("lds stripe 9-16", op, width, shift, y_shift, wide)
            y1 = run(op, xd, wide, rows, width, shift, y_shift)
            assert_close(y1, ref, f"{op} {width} {wide}")
        looped = run(op, xd, R.Plan(1024, 0, 4, 1024, 0, policy=R.ROWRED_POLICY_LOOPED), rows, width, shift, y_shift)
        assert_close(y1, looped.astype(np.float64), f"{op} {width} vs looped")


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_wide_special_values(op):
    rows, width = 6, 65536
    x = synthetic.random_matrix(96, rows, width, "normal")
    x[0, :] = -np.inf
    x[1, :60000] = -np.inf             # the max sits in the LDS slots
    x[2, 50000] = np.nan
    x[3, 5] = np.inf
    x[4, 64000:] = 70.0
    x[5, ::2] = 1e15
    x[5, 1::2] = -1e15
    xd = shifted_input(x, 0)
    got = run(op, xd, R.Plan(1024, 0, 16, 1024, 0, policy=LDS), rows, width, 0)
    assert_close(got, oracle_of(op, x), f"{op} special 16 slots")


TAIL = R.ROWRED_POLICY_LDS_STRIPE | R.ROWRED_POLICY_LOOPED


@pytest.mark.parametrize("width", [65537, 70001, 100003, 128256, 262147])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_head_held_tail_walked(op, width):
    """Rows wider than 16384 granules: the first 16384 held in registers and
    LDS, the rest walked twice in tiles (one, two and many tiles, odd tile
    counts, a partial last tile), ragged and misaligned, both memory
    policies; the oracle's bar and within it of the looped kernels."""
    rows = 5
    x = synthetic.random_matrix(width + 31, rows, width, "normal")
    ref = oracle_of(op, x)
    for shift, y_shift in ((0, 0), (3, 3), (1, 2)):
        xd = shifted_input(x, shift)
        outs = []
        for pol in (0, R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP,
                    R.ROWRED_POLICY_REVERSE, R.ROWRED_POLICY_REVERSE | R.ROWRED_POLICY_NT_LOADS):
            plan = R.Plan(1024, 0, 16, 1024, 0, policy=pol | TAIL)
            print_case("head + tail", op, width, shift, y_shift, plan)
            got = run(op, xd, plan, rows, width, shift, y_shift)
            assert_close(got, ref, f"{op} {width} {plan}")
            outs.append(got)
        # the second walk's order changes no arithmetic
        assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
        looped = run(op, xd, R.Plan(1024, 0, 4, 1024, 0, policy=R.ROWRED_POLICY_LOOPED), rows, width, shift, y_shift)
        assert_close(got, looped.astype(np.float64), f"{op} {width} vs looped")


@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_head_tail_special_values(op):
    rows, width = 7, 100000
    x = synthetic.random_matrix(97, rows, width, "normal")
    x[0, :] = -np.inf
    x[1, :90000] = -np.inf             # the max only in the tail
    x[2, 10] = np.nan                  # NaN in the head
    x[3, 99000] = np.inf               # +inf in the tail
    x[4, 99990:] = 80.0                # the max in the last tile: the running sum rescales
    x[5, :65536] = -1e15               # the head far below the tail
    x[6, ::2] = 1e15
    x[6, 1::2] = -1e15
    xd = shifted_input(x, 0)
    got = run(op, xd, R.Plan(1024, 0, 16, 1024, 0, policy=TAIL), rows, width, 0)
    assert_close(got, oracle_of(op, x), f"{op} special head + tail")


def run_ln(x, r, g, b, plan, shift_x, shift_r, shift_y):
    t = torch()
    rows, width = x.shape
    xd = shifted_input(x, shift_x)
    rd = shifted_input(r, shift_r) if r is not None else None
    gd = t.from_numpy(g).cuda() if g is not None else None
    bd = t.from_numpy(b).cuda() if b is not None else None
    out = Guarded(rows, width, shift_y)
    if plan is None:
        R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=1e-5)
    else:
        R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=1e-5)
    t.cuda.synchronize()
    assert out.guards_intact()
    return out.host()


@pytest.mark.parametrize("width", [32769, 40003, 65536, 100003])
@pytest.mark.parametrize("variant", ["residual", "plain", "affine"])
def test_layernorm_head_held_tail_walked(variant, width):
    """LayerNorm rows wider than 8192 granules: x and r of the first 8192
    held in registers and LDS, the rest walked twice; through the entry point
    and as an explicit plan, r at x's phase and at another, both memory
    policies; the oracle's bar and within it of the looped kernel."""
    import oracle
    rows = 5
    x = synthetic.random_matrix(width + 41, rows, width, "uniform")
    r = synthetic.random_matrix(width + 42, rows, width, "uniform", tensor="r") if variant == "residual" else None
    g = b = None
    if variant == "affine":
        g = (1.0 + 0.1 * synthetic.random_matrix(width + 43, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
        b = (0.1 * synthetic.random_matrix(width + 44, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g, beta=b)
    for sx, sr, sy in ((0, 0, 0), (1, 1, 1), (2, 3, 2)):
        got = run_ln(x, r, g, b, None, sx, sr, sy)
        assert_close(got, ref, f"{variant} {width} entry point")
        outs = []
        for pol in (0, R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP,
                    R.ROWRED_POLICY_REVERSE, R.ROWRED_POLICY_REVERSE | R.ROWRED_POLICY_NT_STORES):
            plan = R.Plan(1024, 0, 8, 1024, 0, policy=pol | TAIL)
            print_case("layernorm head + tail", variant, width, sx, sr, sy, plan)
            outs.append(run_ln(x, r, g, b, plan, sx, sr, sy))
            assert_close(outs[-1], ref, f"{variant} {width} {plan}")
        # the second walk's order changes no arithmetic
        assert np.array_equal(outs[0].view(np.uint32), outs[2].view(np.uint32))
        looped = run_ln(x, r, g, b, R.Plan(1024, 0, 2, 1024, 0, policy=R.ROWRED_POLICY_LOOPED), sx, sr, sy)
        assert_close(got, looped.astype(np.float64), f"{variant} {width} vs looped")


def test_layernorm_head_tail_offset_rows():
    """Rows with a large common offset (spread << magnitude): the TwoSum pair
    and the FP64 statistics keep the centred values exact."""
    import oracle
    rows, width = 4, 70001
    x = (synthetic.random_matrix(301, rows, width, "uniform") + 1e4).astype(np.float32)
    r = synthetic.random_matrix(302, rows, width, "uniform", tensor="r")
    ref = oracle.layernorm(x, r, eps=1e-5)
    assert_close(run_ln(x, r, None, None, R.Plan(1024, 0, 8, 1024, 0, policy=TAIL), 1, 1, 1), ref, "offset rows")


@pytest.mark.parametrize("which", ["gamma", "beta", "both", "gamma_offset"])
def test_layernorm_head_tail_affine_loads(which):
    """gamma and/or beta over the head and the tail: read 16 bytes at a time
    when rows, gamma and beta start on 16-byte boundaries, else 4 bytes at a
    time (gamma_offset: gamma one element past an aligned start)."""
    import oracle
    t = torch()
    rows, width = 3, 65536 + 4096
    x = synthetic.random_matrix(311, rows, width, "uniform")
    r = synthetic.random_matrix(312, rows, width, "uniform", tensor="r")
    g = (1.0 + 0.1 * synthetic.random_matrix(313, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
    b = (0.1 * synthetic.random_matrix(314, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
    use_g = which != "beta"
    use_b = which in ("beta", "both", "gamma_offset")
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g if use_g else None, beta=b if use_b else None)
    xd = shifted_input(x, 0)
    rd = shifted_input(r, 0)
    gd = shifted_input(g[None, :], 1 if which == "gamma_offset" else 0)[0] if use_g else None
    bd = t.from_numpy(b).cuda() if use_b else None
    for plan in (None, R.Plan(1024, 0, 8, 1024, 0, policy=TAIL | R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES)):
        out = Guarded(rows, width, 0)
        print_case("layernorm head + tail affine", which, plan)
        if plan is None:  # the entry point's own plan
            R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=1e-5)
        else:
            R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=1e-5)
        t.cuda.synchronize()
        assert out.guards_intact()
        assert_close(out.host(), ref, f"affine {which} {plan}")


def offset_rows(seed, rows, width):
    """N(0, 8^2) rows shifted by per-row offsets in [-80, 80] (the softmax
    stress recipe), so a row's max is far from its neighbour's."""
    x = synthetic.random_matrix(seed, rows, width, "normal") * 8.0
    off = np.linspace(-80.0, 80.0, rows)[::-1].copy()
    off[1::2] *= -1.0
    return (x + off[:, None]).astype(np.float32)


@pytest.mark.parametrize("width", [65534, 65535])
@pytest.mark.parametrize("op", ["rmsnorm", "softmax"])
def test_head_boundary_widths(op, width):
    """Widths whose row windows straddle the 16384-granule head: at some
    16-byte phases a row's window is exactly the head (nothing left for the
    tail) and its last head granule holds elements of the next row, at others
    it is one granule longer.  Every x phase, rows at every phase, y at x's
    phase and at another; the entry point and explicit plans."""
    t = torch()
    rows = 8
    x = offset_rows(width + 7, rows, width)
    ref = oracle_of(op, x)
    for shift, y_shift in ((0, 0), (1, 1), (2, 3), (3, 3)):
        xd = shifted_input(x, shift)
        out = Guarded(rows, width, y_shift)
        plan = R.rowred_plan_query(op, xd, None, out.y)
        print_case("head boundary", op, width, shift, y_shift, plan)
        if op == "rmsnorm":
            R.rowred_rmsnorm(xd, out.y, eps=synthetic.EPS["rmsnorm"])
        else:
            R.rowred_softmax(xd, out.y)
        t.cuda.synchronize()
        assert out.guards_intact()
        assert_close(out.host(), ref, f"{op} {width} shift {shift} entry point {plan}")
        if (width + shift + 3) // 4 > 16384 or (width + (shift + width) % 4 + 3) // 4 > 16384:
            for pol in (R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_REVERSE):
                p = R.Plan(1024, 0, 16, 1024, 0, policy=pol | TAIL)
                assert_close(run(op, xd, p, rows, width, shift, y_shift), ref, f"{op} {width} shift {shift} {p}")


@pytest.mark.parametrize("width", [32766, 32767])
@pytest.mark.parametrize("variant", ["residual", "plain", "affine"])
def test_layernorm_head_boundary_widths(variant, width):
    """LayerNorm widths whose row windows straddle the 8192-granule head (x
    and r held): rows whose window is exactly the head must count and centre
    only their own elements.  Every x phase, r and y at x's phase and at
    others, the entry point and explicit plans."""
    import oracle
    rows = 8
    x = offset_rows(width + 51, rows, width)
    r = synthetic.random_matrix(width + 52, rows, width, "uniform", tensor="r") if variant == "residual" else None
    g = b = None
    if variant == "affine":
        g = (1.0 + 0.1 * synthetic.random_matrix(width + 53, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
        b = (0.1 * synthetic.random_matrix(width + 54, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g, beta=b)
    for sx, sr, sy in ((0, 0, 0), (1, 1, 1), (2, 3, 2), (3, 3, 0)):
        print_case("layernorm head boundary", variant, width, sx, sr, sy)
        assert_close(run_ln(x, r, g, b, None, sx, sr, sy), ref, f"{variant} {width} {sx} entry point")
        if (width + sx + 3) // 4 > 8192 or (width + (sx + width) % 4 + 3) // 4 > 8192:
            for pol in (R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_REVERSE):
                p = R.Plan(1024, 0, 8, 1024, 0, policy=pol | TAIL)
                assert_close(run_ln(x, r, g, b, p, sx, sr, sy), ref, f"{variant} {width} {sx} {p}")
