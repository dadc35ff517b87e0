"""The chooser's plans for large calls, at full size, through the plain entry
points: every width band of the aligned-row rules (geometry and
workgroups-per-CU cap), the three-slot rule for RMSNorm / softmax rows off
16-byte boundaries, and the large-call exchange rule (segments of 1024 or
2048 granules, words in y's rows).  Sampled rows
against the FP64 oracle (atol = rtol = 1e-5), every element finite, guard
bands intact; the plan the chooser reports is checked to be the band's."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, assert_close, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

CAP = R.ROWRED_POLICY_CU_GROUPS
ON = R.ROWRED_POLICY_ONLINE

# (op, rows, width): (lanes, chunks, threads, cap) the chooser must take
BANDS = {
    ("rmsnorm", 262144, 512): (64, 2, 128, 10),
    ("softmax", 131072, 1024): (128, 2, 256, 6),
    ("rmsnorm", 65536, 2048): (256, 2, 256, 6),
    ("softmax", 32768, 4096): (128, 8, 256, 2),
    ("layernorm_residual", 32768, 4096): (256, 4, 512, 2),
    # large calls of LayerNorm rows beyond 2048 granules and RMSNorm / softmax
    # rows beyond 4096: the exchange kernels with words in y's rows
    ("layernorm_residual", 8192, 16384): (256, 8, 256, 0),
    ("layernorm_residual", 4096, 32768): (256, 8, 256, 0),
    ("layernorm_residual", 6553, 20480): (256, 4, 256, 0),
    ("rmsnorm", 6553, 20480): (256, 4, 256, 0),
    ("softmax", 8192, 32768): (128, 8, 128, 0),
    ("softmax", 4480, 30001): (128, 8, 128, 0),
    ("softmax", 2048, 16384): (256, 8, 256, 0),
    ("rmsnorm", 4096, 16384): (256, 8, 256, 0),
    ("layernorm", 131072, 1024): (128, 2, 128, 10),
    ("rmsnorm", 65568, 2047): (256, 3, 256, 6),
    ("softmax", 32776, 4095): (512, 3, 512, 0),
    ("softmax", 16386, 8191): (1024, 3, 1024, 0),
}


@pytest.mark.parametrize("op,rows,width", list(BANDS), ids=lambda v: str(v))
def test_band_full_size(op, rows, width):
    L, C, T, cap = BANDS[(op, rows, width)]
    print_case("band", op, rows, width)
    dist = "normal" if op == "softmax" else "uniform"
    x = synthetic.random_matrix(rows + width, rows, width, dist)
    r = synthetic.random_matrix(rows + width + 1, rows, width, dist, tensor="r") \
        if op == "layernorm_residual" else None
    xd = shifted_input(x, 0)
    rd = shifted_input(r, 0) if r is not None else None
    out = Guarded(rows, width)
    kop = "layernorm_residual" if op == "layernorm" else op
    p = R.rowred_plan_query(kop, xd, rd, out.y)
    assert (p.lanes_per_row, p.chunks, p.threads, (p.policy >> 12) & 15) == (L, C, T, cap), p
    exchange = (op, width) in (("layernorm_residual", 16384), ("layernorm_residual", 32768),
                               ("layernorm_residual", 20480), ("rmsnorm", 20480), ("softmax", 32768),
                               ("softmax", 30001), ("softmax", 16384), ("rmsnorm", 16384))
    assert bool(p.policy & R.ROWRED_POLICY_EXCHANGE) == exchange, p
    eps = synthetic.EPS.get(op, 0.0)
    if op in ("layernorm", "layernorm_residual"):
        R.rowred_layernorm(xd, rd, None, None, out.y, eps=eps)
    elif op == "rmsnorm":
        R.rowred_rmsnorm(xd, out.y, eps=eps)
    else:
        R.rowred_softmax(xd, out.y)
    torch().cuda.synchronize()
    assert out.guards_intact()
    y = out.host()
    assert np.isfinite(y).all()
    pick = np.unique(np.concatenate([np.arange(3), rows - 1 - np.arange(3),
                                     np.random.default_rng(rows ^ width).integers(0, rows, 100)]))
    ref = oracle.run_op(op, x[pick], r[pick] if r is not None else None, eps=synthetic.EPS.get(op))
    assert_close(y[pick], ref, f"{op} {rows}x{width} {p}")
