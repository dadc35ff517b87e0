"""Softmax with one (max, sum) collective (ROWRED_POLICY_ONLINE) through the
C ABI against the FP64 oracle at atol = rtol = 1e-5, NaN exactly where the
oracle has NaN: every register-kernel geometry, the LDS-stripe kernels (bit
for bit equal to the register kernel of the same stripe under the same
policy), special rows, full-size rows."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, all_plans, assert_close, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

ON = R.ROWRED_POLICY_ONLINE
LDS = R.ROWRED_POLICY_LDS_STRIPE
NTR = R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP


def run(xd, plan, rows, width, y_shift=0):
    out = Guarded(rows, width, y_shift)
    R.rowred_run_plan("softmax", xd, None, out.y, plan)
    torch().cuda.synchronize()
    assert out.guards_intact(), f"softmax {rows}x{width} {plan} wrote outside y"
    return out.host()


@pytest.mark.parametrize("width", [1, 3, 5, 17, 100, 257, 1000, 4096, 8191])
def test_online_every_plan(width):
    """Every register-kernel geometry (lanes, chunks, threads, memory
    policy, staging) with rows one float past 16-byte boundaries."""
    rows = 67
    x = synthetic.random_matrix(7 * width + 3, rows, width, "normal")
    ref = oracle.softmax(x)
    xd = shifted_input(x, 1)
    n = 0
    for plan in all_plans((width + 6) // 4):
        plan = R.Plan(plan.lanes_per_row, 0, plan.chunks, plan.threads, 0, policy=plan.policy | ON)
        print_case("online", width, plan)
        assert_close(run(xd, plan, rows, width, 1), ref, f"online {width} {plan}")
        n += 1
    assert n >= 3


@pytest.mark.parametrize("width", [16385, 20000, 24576, 28673, 32765, 32768])
def test_online_lds_matches_register_bitwise(width):
    """5-8 chunks: the LDS stripe computes the register kernel's online
    arithmetic in the same order; ragged and misaligned rows."""
    rows = 37
    x = synthetic.random_matrix(width + 23, rows, width, "normal")
    ref = oracle.softmax(x)
    for shift, y_shift in ((0, 0), (1, 1), (3, 2)):
        xd = shifted_input(x, shift)
        C = -(-((width + shift + 3) // 4) // 1024)
        if C > 8:
            continue
        for pol in (0, NTR):
            base = R.Plan(1024, 0, C, 1024, 0, policy=pol | ON)
            wide = R.Plan(1024, 0, C, 1024, 0, policy=pol | ON | LDS)
            print_case("online lds", width, shift, y_shift, wide)
            y0 = run(xd, base, rows, width, y_shift)
            y1 = run(xd, wide, rows, width, y_shift)
            assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{width} {shift} {wide}"
            assert_close(y1, ref, f"online {width} {wide}")


@pytest.mark.parametrize("width", [32769, 40000, 50257, 65536])
def test_online_lds_wide_rows(width):
    """9-16 chunks (8 register + up to 8 LDS slots per lane)."""
    rows = 19
    x = synthetic.random_matrix(width + 5, rows, width, "normal")
    ref = oracle.softmax(x)
    for shift in (0, 3):
        xd = shifted_input(x, shift)
        C = -(-((width + shift + 3) // 4) // 1024)
        if C > 16:
            continue
        plan = R.Plan(1024, 0, C, 1024, 0, policy=NTR | ON | LDS)
        print_case("online lds wide", width, shift, plan)
        assert_close(run(xd, plan, rows, width, shift), ref, f"online {width} {plan}")


def special_rows(width):
    x = synthetic.random_matrix(width + 41, 12, width, "normal")
    x[0, :] = -np.inf                    # all -inf -> NaN row
    x[1, 5] = np.inf                     # +inf -> NaN row
    x[2, width - 2] = np.nan             # NaN -> NaN row
    x[3, :] = 0.0                        # uniform -> 1/width
    x[4, ::2] = -np.inf                  # half the row masked
    x[5, :] += np.float32(1000.0)        # large offset
    x[6, :] = -1000.0
    x[6, 17] = 1000.0                    # one-hot
    x[7, : width - 9] = -np.inf          # only the last lanes hold finite values
    x[8, ::2] = 1e15
    x[8, 1::2] = -1e15
    x[9, :] = np.nan
    x[10, width // 2:] = 80.0            # maxima far apart in different lanes
    x[10, : width // 2] = -80.0
    x[11, :] = -3e38
    x[11, 3] = 3e38
    return x


@pytest.mark.parametrize("width", [300, 4096, 32768])
def test_online_special_rows(width):
    x = special_rows(width)
    ref = oracle.softmax(x)
    window = (width + 3) // 4
    plans = [R.Plan(256, 0, -(-window // 256), 256, 0, policy=ON | 3)] if window <= 256 * 16 else []
    if window > 4096:
        plans += [R.Plan(1024, 0, 8, 1024, 0, policy=ON), R.Plan(1024, 0, 8, 1024, 0, policy=ON | LDS)]
    else:
        plans += [R.Plan(64, 0, -(-window // 64), 256, 0, policy=ON)] if window <= 64 * 16 else []
        plans += [R.Plan(1024, 0, -(-window // 1024), 1024, 0, policy=ON | 3)]
    outs = []
    for plan in plans:
        print_case("online special", width, plan)
        y = run(shifted_input(x, 0), plan, x.shape[0], width)
        assert_close(y, ref, f"online special {width} {plan}")
        outs.append(y)
    y = outs[-1]
    assert np.isnan(y[0]).all() and np.isnan(y[1]).all() and np.isnan(y[2]).all() and np.isnan(y[9]).all()
    assert (y[4, ::2] == 0).all() and (y[7, : width - 9] == 0).all()
    assert y[6, 17] == 1.0
    if window > 4096:
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


FULL = {(8192, 32768): (1024, 8, 1024, NTR | LDS), (16384, 8192): (1024, 2, 1024, NTR),
        (131072, 127): (16, 3, 256, 3)}


@pytest.mark.parametrize("rows,width", list(FULL))
def test_online_full_size(rows, width):
    """Full-size matrices in the geometry the chooser uses for them (a
    register plan for the short rows), sampled rows against the oracle, every
    element finite."""
    L, C, T, pol = FULL[(rows, width)]
    x = synthetic.random_matrix(rows ^ width, rows, width, "normal")
    xd = shifted_input(x, 0)
    plan = R.Plan(L, 0, C, T, 0, policy=pol | ON)
    print_case("online full", rows, width, plan)
    y = run(xd, plan, rows, width)
    assert np.isfinite(y).all()
    pick = np.unique(np.concatenate([np.arange(3), rows - 1 - np.arange(3),
                                     np.random.default_rng(rows + width).integers(0, rows, 100)]))
    assert_close(y[pick], oracle.softmax(x[pick]), f"online full {rows}x{width} {plan}")
