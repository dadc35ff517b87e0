"""Row sum and paired row min/max through the C ABI against the FP64 oracle:
sums within |d| <= 1e-5 + 1e-5 |ref|, min/max bit for bit."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import all_plans, assert_close, dev, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

GUARD_BITS = np.uint32(0x7FC0DEAD)


def guarded_vec(n):
    t = torch()
    buf = t.empty(n + 128, dtype=t.int32, device="cuda")
    buf.fill_(int(GUARD_BITS.view(np.int32)))
    return buf, buf[64:64 + n].view(t.float32)


def guards_ok(buf, n):
    b = buf.cpu().numpy().view(np.uint32)
    return bool((b[:64] == GUARD_BITS).all() and (b[64 + n:] == GUARD_BITS).all())


def run(x, shift=0, plan=None):
    rows = x.shape[0]
    xd = shifted_input(x, shift)
    bs, s = guarded_vec(rows)
    bl, lo = guarded_vec(rows)
    bh, hi = guarded_vec(rows)
    if plan is None:
        R.rowred_row_sum(xd, s)
        R.rowred_row_minmax(xd, lo, hi)
    else:
        R.rowred_row_reduce_run_plan("row_sum", xd, s, None, plan)
        R.rowred_row_reduce_run_plan("row_minmax", xd, lo, hi, plan)
    torch().cuda.synchronize()
    assert guards_ok(bs, rows) and guards_ok(bl, rows) and guards_ok(bh, rows)
    return s.cpu().numpy(), lo.cpu().numpy(), hi.cpu().numpy()


def check(x, got, what):
    s, lo, hi = got
    rs = oracle.row_sum(x)
    rlo, rhi = oracle.row_minmax(x)
    assert_close(s, rs, what + " sum")
    assert np.array_equal(lo.view(np.uint32), rlo.astype(np.float32).view(np.uint32)), what + " min"
    assert np.array_equal(hi.view(np.uint32), rhi.astype(np.float32).view(np.uint32)), what + " max"


@pytest.mark.parametrize("width", [1, 2, 3, 4, 5, 7, 31, 64, 127, 129, 257, 1000, 1537, 4096, 4097, 8192, 32765,
                                   32768])
def test_widths(width):
    rows = max(3, min(700, (1 << 21) // width))
    print_case("row reduce", rows, width)
    x = synthetic.random_matrix(9 * width, rows, width, "normal")
    check(x, run(x), f"{rows}x{width}")


@pytest.mark.parametrize("shift", [1, 2, 3])
@pytest.mark.parametrize("width", [3, 130, 4096])
def test_misaligned(shift, width):
    x = synthetic.random_matrix(width + shift, 77, width, "uniform")
    check(x, run(x, shift=shift), f"shift {shift} width {width}")


def test_special_values():
    w = 300
    x = synthetic.random_matrix(5, 8, w, "normal")
    x[0, 3] = np.nan                      # skipped by min/max, poisons the sum
    x[1, :] = np.nan                      # all NaN: (+inf, -inf), sum NaN
    x[2, 7] = np.inf                      # max +inf, sum +inf
    x[3, 9] = -np.inf                     # min -inf, sum -inf
    x[4, :] = 1e30                        # large sum, still finite in FP64 and FP32 (3e32)
    x[5, ::2] = 1e20
    x[5, 1::2] = -1e20                    # exact cancellation in FP64
    s, lo, hi = run(x)
    assert np.isnan(s[0]) and np.isnan(s[1])
    assert lo[1] == np.inf and hi[1] == -np.inf
    assert hi[2] == np.inf and s[2] == np.inf and lo[3] == -np.inf and s[3] == -np.inf
    check(x, (s, lo, hi), "special")


@pytest.mark.parametrize("width", [3, 100, 257, 4096])
def test_every_plan(width):
    x = synthetic.random_matrix(31 * width, 67, width, "normal")
    n = 0
    for plan in all_plans((width + 6) // 4):
        if plan.policy & R.ROWRED_POLICY_STAGE_STORES:
            continue
        print_case("row reduce", width, plan)
        check(x, run(x, shift=1, plan=plan), f"{width} {plan}")
        n += 1
    assert n >= 3


@pytest.mark.parametrize("case", synthetic.NEXT_WORKLOADS[8], ids=lambda c: c.name)
def test_full_size(case):
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    check(x, run(x), case.name)
