"""The per-phase reload variant (ROWRED_POLICY_RELOAD): the same plan with
the bit set must give bitwise the resident kernel's result (same arithmetic
on the same values, read again), and so the oracle's within tolerance."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, all_plans, assert_close, print_case, shifted_input, torch
from tests.test_gpu_parity import inputs, oracle_of

pytestmark = pytest.mark.gpu

CASES = ("layernorm_residual", "layernorm", "rmsnorm", "softmax")


def run(op, xd, rd, plan, rows, width, shift):
    out = Guarded(rows, width, shift)
    eps = synthetic.EPS.get(op, 0.0)
    if op == "layernorm":
        R.rowred_layernorm_run_plan(xd, None, None, None, out.y, plan, eps=eps)
    else:
        R.rowred_run_plan(op, xd, rd, out.y, plan, eps=eps)
    torch().cuda.synchronize()
    assert out.guards_intact()
    return out.host()


def reload_ok(op, plan):
    if plan.chunks > 8:
        return False
    return not (op.startswith("layernorm") and plan.chunks >= 7 and plan.threads > 512)


@pytest.mark.parametrize("width", [3, 100, 257, 1000, 4096, 8192])
@pytest.mark.parametrize("op", CASES)
def test_reload_matches_resident_bitwise(op, width):
    rows = 41
    x, r = inputs("layernorm_residual" if op == "layernorm_residual" else op, rows, width, seed=7 * width + 3)
    ref = oracle_of(op, x, r)
    shift = 1 if width % 4 else 0
    xd = shifted_input(x, shift)
    rd = shifted_input(r, shift) if r is not None else None
    n = 0
    for plan in all_plans((width + 6) // 4):
        if plan.policy not in (0, 7) or not reload_ok(op, plan):
            continue
        print_case(op, width, plan)
        y0 = run(op, xd, rd, plan, rows, width, shift)
        plan_r = R.Plan(plan.lanes_per_row, 0, plan.chunks, plan.threads, 0, policy=plan.policy | R.ROWRED_POLICY_RELOAD)
        y1 = run(op, xd, rd, plan_r, rows, width, shift)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32)), f"{op} {width} {plan}"
        assert_close(y1, ref, f"{op} {width} {plan_r}")
        n += 1
    assert n >= 1


@pytest.mark.parametrize("case", [synthetic.CORE_WORKLOADS[4][0], synthetic.CORE_WORKLOADS[5][0]], ids=lambda c: c.name)
def test_reload_full_size(case):
    """The chooser's geometry with the reload bit at a full workload shape:
    bitwise the resident result (the register kernel of that geometry -- for
    exchange and LDS-stripe plans one 1024-lane workgroup per row -- with two
    softmax collectives: the reload kernels have no LDS-stripe, exchange or
    one-collective form)."""
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
    xd = shifted_input(x, 0)
    rd = shifted_input(r, 0) if r is not None else None
    q = R.rowred_plan_query(case.op, xd, rd, Guarded(case.rows, case.width, 0).y)
    L, C, T, pol = q.lanes_per_row, q.chunks, q.threads, q.policy & ~R.ROWRED_POLICY_ONLINE
    if pol & (R.ROWRED_POLICY_EXCHANGE | R.ROWRED_POLICY_LDS_STRIPE):  # one 1024-lane workgroup per row
        L = T = 1024
        C = -(-q.window // 1024)
        pol &= R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP
    p = R.Plan(L, 0, C, T, 0, policy=pol)
    y0 = run(case.op, xd, rd, p, case.rows, case.width, 0)
    pr = R.Plan(p.lanes_per_row, 0, p.chunks, p.threads, 0, policy=p.policy | R.ROWRED_POLICY_RELOAD)
    y1 = run(case.op, xd, rd, pr, case.rows, case.width, 0)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
