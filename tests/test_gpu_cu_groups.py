"""Workgroups-per-CU caps (policy bits 12-15) on the register kernels: the
launch reserves LDS so that at most n workgroups share a CU.  Occupancy
changes no arithmetic, so every capped result is bitwise the uncapped one,
and within the oracle's bar."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch
from tests.test_gpu_parity import inputs, oracle_of

pytestmark = pytest.mark.gpu

CAP = R.ROWRED_POLICY_CU_GROUPS


def run(op, xd, rd, plan, rows, width, shift):
    out = Guarded(rows, width, shift)
    R.rowred_run_plan(op, xd, rd, out.y, plan, eps=synthetic.EPS.get(op, 0.0))
    torch().cuda.synchronize()
    assert out.guards_intact(), f"{op} {rows}x{width} {plan} wrote outside y"
    return out.host()


@pytest.mark.parametrize("op", ["layernorm_residual", "rmsnorm", "softmax"])
@pytest.mark.parametrize("width,L,C,T", [(257, 32, 3, 256), (1024, 128, 3, 256), (4096, 256, 5, 512)])
def test_caps_change_nothing(op, width, L, C, T):
    rows = 300
    x, r = inputs(op, rows, width, seed=width + 3)
    ref = oracle_of(op, x, r)
    for shift in (0, 1):
        xd = shifted_input(x, shift)
        rd = shifted_input(r, shift) if r is not None else None
        pols = [3, 7] + ([11] if width <= 256 * 4 and shift else [])
        for pol in pols:
            base = run(op, xd, rd, R.Plan(L, 0, C, T, 0, policy=pol), rows, width, shift)
            assert_close(base, ref, f"{op} {width} {pol}")
            for n in (1, 2, 3, 5, 8, 14):
                plan = R.Plan(L, 0, C, T, 0, policy=pol | CAP(n))
                print_case("cap", op, width, shift, plan)
                y = run(op, xd, rd, plan, rows, width, shift)
                assert np.array_equal(y.view(np.uint32), base.view(np.uint32)), (op, width, shift, plan)


def test_row_reductions_with_caps():
    rows, width = 500, 1000
    x = synthetic.random_matrix(77, rows, width, "normal")
    xd = shifted_input(x, 0)
    outs = []
    for n in (0, 4):
        s = torch().empty(rows, device="cuda")
        lo, hi = torch().empty(rows, device="cuda"), torch().empty(rows, device="cuda")
        plan = R.Plan(256, 0, 1, 512, 0, policy=3 | CAP(n))
        R.rowred_row_reduce_run_plan("row_sum", xd, s, None, plan)
        R.rowred_row_reduce_run_plan("row_minmax", xd, lo, hi, plan)
        torch().cuda.synchronize()
        outs.append((s.cpu().numpy(), lo.cpu().numpy(), hi.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    assert np.array_equal(outs[0][1], x.min(axis=1)) and np.array_equal(outs[0][2], x.max(axis=1))


def test_capped_full_size_layernorm():
    """131072 x 1024 residual LayerNorm (16-byte aligned rows) with a cap:
    sampled rows against the oracle."""
    rows, width = 131072, 1024
    x = synthetic.random_matrix(5, rows, width, "uniform")
    r = synthetic.random_matrix(6, rows, width, "uniform", tensor="r")
    xd, rd = shifted_input(x, 0), shifted_input(r, 0)
    plan = R.Plan(128, 0, 2, 256, 0, policy=7 | CAP(5))
    y = run("layernorm_residual", xd, rd, plan, rows, width, 0)
    pick = np.unique(np.concatenate([np.arange(3), rows - 1 - np.arange(3),
                                     np.random.default_rng(1).integers(0, rows, 100)]))
    assert_close(y[pick], oracle_of("layernorm_residual", x[pick], r[pick]), "capped 131072x1024")
