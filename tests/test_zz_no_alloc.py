"""rowred_static_ws: the _ws entry points on the library's static workspace
(a device array per GPU; nothing allocated per call).  Its results must be
bitwise those of the matching _ws entry point with a caller workspace, and
within the oracle's bar (|y - ref| <= 1e-5 + 1e-5 |ref|).  Two calls in a row
share the array: the second, on a smaller input, must not see the first's
leftovers.  A call that needs more workspace than the array holds is refused
before anything runs."""
import numpy as np
import pytest

import row_wise_reduction_amd as R
from tests.gpu_util import assert_close, print_case, shifted_input, torch
from tests.test_gpu_split import c_op, make_inputs, reference

pytestmark = pytest.mark.gpu

EPS = {"layernorm_residual": 1e-5, "layernorm": 1e-5, "layernorm_affine": 1e-5, "rmsnorm": 1e-6}

# (op, first shape, second shape): each first shape splits rows across
# workgroups (exchange or three split kernels), so the workspace is used.
CASES = [
    ("softmax", (64, 65536), (8, 40003)),
    ("rmsnorm", (32, 131072), (5, 70001)),
    ("layernorm_residual", (16, 65536), (3, 50001)),
    ("layernorm_affine", (8, 65540), (2, 40001)),
    ("row_sum", (16, 1048576), (4, 300001)),
    ("row_minmax", (8, 1048576), (3, 200003)),
    ("softmax", (256, 4096), (7, 1537)),  # rows that fit: no workspace touched
]


def call(op, xd, rd, gd, bd, static, ws=None):
    """Run `op` on the GPU: through rowred_static_ws or the _ws entry point."""
    t = torch()
    rows, width = xd.shape
    eps = EPS.get(op, 0.0)
    k = "layernorm_residual" if op.startswith("layernorm") else op
    if op in ("row_sum", "row_minmax"):
        o0 = t.full((rows,), float("nan"), device="cuda")
        o1 = t.full((rows,), float("nan"), device="cuda") if op == "row_minmax" else None
        if static:
            R.rowred_static_ws(k, xd, None, None, None, o0, o1)
        elif op == "row_sum":
            R.rowred_row_sum_ws(xd, o0, ws)
        else:
            R.rowred_row_minmax_ws(xd, o0, o1, ws)
        t.cuda.synchronize()
        return (o0.cpu().numpy(), o1.cpu().numpy()) if o1 is not None else o0.cpu().numpy()
    y = t.full((rows, width), float("nan"), device="cuda")
    if static:
        R.rowred_static_ws(k, xd, rd, gd, bd, y, None, eps=eps)
    elif op.startswith("layernorm"):
        R.rowred_layernorm_ws(xd, rd, gd, bd, y, ws, eps=eps)
    elif op == "rmsnorm":
        R.rowred_rmsnorm_ws(xd, y, ws, eps=eps)
    else:
        R.rowred_softmax_ws(xd, y, ws)
    t.cuda.synchronize()
    return y.cpu().numpy()


def same_bits(a, b):
    if isinstance(a, tuple):
        return all(same_bits(u, v) for u, v in zip(a, b))
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


@pytest.mark.parametrize("op,first,second", CASES, ids=[f"{c[0]}-{c[1][0]}x{c[1][1]}" for c in CASES])
def test_static_matches_ws(op, first, second):
    """Two static calls in a row (the second on a smaller input), then the
    same two through the _ws entry point with a caller workspace."""
    t = torch()
    k = "layernorm_residual" if op.startswith("layernorm") else op
    inputs, static_out = [], []
    for i, (rows, width) in enumerate((first, second)):
        x, r, g, b = make_inputs(op, rows, width, seed=7001 + 13 * i + width % 97)
        shift = i % 2
        dev = (shifted_input(x, shift), shifted_input(r, shift) if r is not None else None,
               t.from_numpy(g).cuda() if g is not None else None, t.from_numpy(b).cuda() if b is not None else None)
        inputs.append(((x, r, g, b), dev))
        print_case("static ws", op, rows, width, "call", i + 1)
        static_out.append(call(op, *dev, static=True))
    for ((x, r, g, b), dev), got in zip(inputs, static_out):
        rows, width = x.shape
        ws = t.empty(max(16, R.rowred_workspace_size(c_op(k), rows, width)), dtype=t.uint8, device="cuda")
        ws.fill_(0x5A)
        print_case("caller ws", op, rows, width)
        want = call(op, *dev, static=False, ws=ws)
        assert same_bits(got, want), f"{op} {rows}x{width}: static workspace differs from caller workspace"
        ref = reference(op, x, r, g, b)
        if op == "row_minmax":
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        else:
            assert_close(got, ref, f"{op} {rows}x{width} static")


def test_static_refuses_beyond_its_size():
    """Row min/max over 2047 rows of 1048577 floats runs the three split
    kernels with 257 segments per row: 2047 * 258 * 16 bytes of records, more
    than the static array holds.  Refused with ROWRED_ERR_UNSUPPORTED before
    anything runs (the outputs keep their fill)."""
    t = torch()
    rows, width = 2047, 1048577
    need = R.rowred_workspace_size(R.ROWRED_OP_ROW_MINMAX, rows, width)
    assert need > R.ROWRED_STATIC_WORKSPACE_BYTES
    x = t.empty((rows, width), dtype=t.float32, device="cuda")  # contents unused: the call is refused
    o0 = t.full((rows,), 7.0, device="cuda")
    o1 = t.full((rows,), 7.0, device="cuda")
    print_case("static ws refused", rows, width, need)
    with pytest.raises(R.RowRedError) as e:
        R.rowred_static_ws("row_minmax", x, None, None, None, o0, o1)
    assert e.value.status == R.ROWRED_ERR_UNSUPPORTED
    t.cuda.synchronize()
    assert bool((o0 == 7.0).all()) and bool((o1 == 7.0).all())
    del x
    t.cuda.empty_cache()
