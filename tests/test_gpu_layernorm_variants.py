"""Plain and affine LayerNorm (r, gamma, beta each optional) through the C
ABI against the FP64 oracle at atol = rtol = 1e-5."""
import numpy as np
import pytest

import oracle
import row_wise_reduction_amd as R
import synthetic
from tests.gpu_util import Guarded, all_plans, assert_close, dev, print_case, shifted_input, torch

pytestmark = pytest.mark.gpu

VARIANTS = {  # name: (residual, gamma, beta)
    "plain": (False, False, False),
    "residual": (True, False, False),
    "affine": (False, True, True),
    "residual_affine": (True, True, True),
    "gamma_only": (False, True, False),
    "beta_only": (True, False, True),
}


def make(rows, width, seed, variant):
    use_r, use_g, use_b = VARIANTS[variant]
    x = synthetic.random_matrix(seed, rows, width, "normal")
    r = synthetic.random_matrix(seed + 1, rows, width, "uniform", tensor="r") if use_r else None
    g = (1 + 0.1 * synthetic.random_matrix(seed + 2, 1, width, "normal", tensor="gamma")[0]).astype(np.float32) \
        if use_g else None
    b = (0.1 * synthetic.random_matrix(seed + 3, 1, width, "normal", tensor="beta")[0]).astype(np.float32) \
        if use_b else None
    return x, r, g, b


def run(x, r, g, b, shift=(0, 0, 0, 0), plan=None, eps=1e-5):
    rows, width = x.shape
    xd = shifted_input(x, shift[0])
    rd = shifted_input(r, shift[1]) if r is not None else None
    gd = shifted_input(g.reshape(1, -1), shift[3]).reshape(-1) if g is not None else None
    bd = shifted_input(b.reshape(1, -1), shift[3]).reshape(-1) if b is not None else None
    out = Guarded(rows, width, shift[2])
    if plan is None:
        R.rowred_layernorm(xd, rd, gd, bd, out.y, eps=eps)
    else:
        R.rowred_layernorm_run_plan(xd, rd, gd, bd, out.y, plan, eps=eps)
    torch().cuda.synchronize()
    assert out.guards_intact()
    return out.host()


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("width", [1, 3, 4, 5, 64, 127, 128, 257, 1000, 1537, 4096, 8192, 24576])
def test_variants_widths(variant, width):
    rows = max(2, min(300, (1 << 20) // width))
    print_case(variant, rows, width)
    x, r, g, b = make(rows, width, 17 * width, variant)
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g, beta=b)
    assert_close(run(x, r, g, b), ref, f"{variant} {rows}x{width}")


@pytest.mark.parametrize("variant", ["plain", "residual_affine", "gamma_only"])
@pytest.mark.parametrize("shift", [(1, 1, 1, 0), (0, 0, 0, 1), (2, 3, 1, 3), (0, 0, 0, 0)])
@pytest.mark.parametrize("width", [6, 129, 4096])
def test_variants_alignment(variant, shift, width):
    """gamma/beta 16-byte aligned with aligned rows (granule path) or at
    another phase than the rows (16-byte loads from 4-byte boundaries); x,
    r, y at every phase."""
    x, r, g, b = make(45, width, 5 * width + sum(shift), variant)
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g, beta=b)
    print_case(variant, shift, width)
    assert_close(run(x, r, g, b, shift=shift), ref, f"{variant} shift {shift} width {width}")


@pytest.mark.parametrize("variant,gshift", [("plain", 1), ("residual_affine", 1), ("residual_affine", 0)],
                         ids=["plain", "residual_affine-gamma_4B", "residual_affine-gamma_16B"])
@pytest.mark.parametrize("width", [100, 1000, 4096])
def test_variants_every_plan(variant, width, gshift):
    """Rows one float past 16-byte boundaries; gamma/beta at the rows' phase
    or 16-byte aligned, read 16 bytes at a time from 4-byte boundaries
    (the first and last slots of a row element by element)."""
    rows = 67
    x, r, g, b = make(rows, width, 3 * width, variant)
    ref = oracle.layernorm(x, r, eps=1e-5, gamma=g, beta=b)
    n = 0
    for plan in all_plans((width + 6) // 4):
        if g is not None and (plan.chunks > 12 or (plan.chunks >= 7 and plan.threads > 512)):
            continue
        print_case(variant, width, gshift, plan)
        assert_close(run(x, r, g, b, shift=(1, 1, 1, gshift), plan=plan), ref, f"{variant} {width} {plan}")
        n += 1
    assert n >= 3


@pytest.mark.parametrize("case", [c for cfg in sorted(synthetic.NEXT_WORKLOADS) for c in synthetic.NEXT_WORKLOADS[cfg]
                                  if c.op in ("layernorm", "layernorm_affine")], ids=lambda c: c.name)
def test_next_workloads_full_size(case):
    print_case(case.name)
    x = synthetic.case_input(case, "x")
    g, b = synthetic.affine_vectors(case) if case.op == "layernorm_affine" else (None, None)
    out = Guarded(case.rows, case.width)
    R.rowred_layernorm(dev(x), None, dev(g) if g is not None else None, dev(b) if b is not None else None, out.y,
                       eps=case.eps)
    torch().cuda.synchronize()
    assert out.guards_intact()
    y = out.host()
    blk = max(1, (1 << 24) // case.width)
    for s in range(0, case.rows, blk):
        t = min(case.rows, s + blk)
        ref = oracle.layernorm(x[s:t], None, eps=case.eps, gamma=g, beta=b)
        assert_close(y[s:t], ref, f"{case.name} rows {s}:{t}")


@pytest.mark.parametrize("width,xshift", [(8191, 0), (8192, 1), (4097, 3)])
def test_misaligned_affine_full_size(width, xshift):
    """Affine LayerNorm at full size on rows off 16-byte boundaries (odd width,
    or the matrix one or three floats past a boundary), gamma / beta on
    16-byte boundaries and one float past: the chooser's own plan, sampled
    rows against the oracle, every element checked for finiteness and the
    guards."""
    rows = 16384
    print_case("affine misaligned", rows, width, xshift)
    x = synthetic.random_matrix(91 + width, rows, width, "uniform")
    g = (1 + 0.1 * synthetic.random_matrix(92 + width, 1, width, "normal", tensor="gamma")[0]).astype(np.float32)
    b = (0.1 * synthetic.random_matrix(93 + width, 1, width, "normal", tensor="beta")[0]).astype(np.float32)
    xd = shifted_input(x, xshift)
    pick = np.unique(np.concatenate([np.arange(4), rows - 1 - np.arange(4),
                                     np.random.default_rng(width).integers(0, rows, 120)]))
    ref = oracle.layernorm(x[pick], None, eps=1e-5, gamma=g, beta=b)
    for gshift in (0, 1):
        gd = shifted_input(g.reshape(1, -1), gshift).reshape(-1)
        bd = shifted_input(b.reshape(1, -1), gshift).reshape(-1)
        out = Guarded(rows, width, xshift)
        R.rowred_layernorm(xd, None, gd, bd, out.y, eps=1e-5)
        torch().cuda.synchronize()
        assert out.guards_intact()
        y = out.host()
        assert np.isfinite(y).all()
        assert_close(y[pick], ref, f"affine {rows}x{width} shift {xshift} gamma shift {gshift}")
