"""Pins for the FP64 oracle that do not come from the oracle itself.

Each operator is fixed from outside the oracle by
  * worked rows whose exact result follows by hand (derivation beside each),
  * invariants of the mathematics (sum to one, zero mean, unit variance at
    eps = 0, shift/scale invariance, symmetry of x and r),
  * special cases (constant rows, -inf entries, huge offsets),
  * 40-digit ``decimal`` brute force on tiny random rows.
The definitions pinned are: residual LayerNorm from "Residual LayerNorm
shared-Tile materialization search" (section "Structural finding"); RMSNorm
and softmax phases from "Immutable input reuse in Metal reductions" (section
"What the transformation actually preserves"), with the plain formulas.
"""
import math
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import synthetic

f32 = np.float32


def row(*v):
    return np.array([v], dtype=np.float32)


# --------------------------------------------------------------------------
# Worked rows (exact by hand)
# --------------------------------------------------------------------------

def test_layernorm_worked_rows():
    # x = [1,2,3,4]: mean 5/2, centred [-3/2,-1/2,1/2,3/2], biased variance
    # (9/4+1/4+1/4+9/4)/4 = 5/4.  eps = 11/4 makes var+eps = 4, sqrt = 2:
    # y = [-3/4, -1/4, 1/4, 3/4] exactly.
    y = oracle.layernorm(row(1, 2, 3, 4), None, eps=2.75)
    assert np.array_equal(y, [[-0.75, -0.25, 0.25, 0.75]])
    # [-1, 1]: mean 0, biased variance 1; eps 3 -> sqrt(4) = 2 -> +-1/2.
    # (Unbiased variance 2 would give 1/sqrt(5); eps outside the root 1/4.)
    y = oracle.layernorm(row(-1, 1), None, eps=3.0)
    assert np.array_equal(y, [[-0.5, 0.5]])
    # eps = 0: y = centred / sqrt(5/4) = [-3,-1,1,3] / sqrt(5)
    y = oracle.layernorm(row(1, 2, 3, 4), None, eps=0.0)
    s5 = math.sqrt(5.0)
    np.testing.assert_allclose(y, [[-3 / s5, -1 / s5, 1 / s5, 3 / s5]], rtol=1e-15)


def test_layernorm_residual_worked_rows():
    # The residual is added, not subtracted: x = 0, r = [1,2,3,4] is the row
    # [1,2,3,4] (x - r would flip every sign; dropping r gives a zero row).
    y = oracle.layernorm_residual(row(0, 0, 0, 0), row(1, 2, 3, 4), eps=2.75)
    assert np.array_equal(y, [[-0.75, -0.25, 0.25, 0.75]])
    # x = [1,2,3,4], r = 10: the combined row is shifted by 10 -> same output.
    y = oracle.layernorm_residual(row(1, 2, 3, 4), row(10, 10, 10, 10), eps=2.75)
    assert np.array_equal(y, [[-0.75, -0.25, 0.25, 0.75]])
    # Split across x and r: x = [1,0,3,0], r = [0,2,0,4].
    y = oracle.layernorm_residual(row(1, 0, 3, 0), row(0, 2, 0, 4), eps=2.75)
    assert np.array_equal(y, [[-0.75, -0.25, 0.25, 0.75]])


def test_layernorm_constant_row_is_zero():
    # combined constant -> centred all zero -> 0 / sqrt(0 + eps) = 0.
    for c in (0.0, 1.0, -3.5, 1024.0):
        y = oracle.layernorm(np.full((3, 7), c, np.float32), None, eps=1e-5)
        assert np.array_equal(y, np.zeros((3, 7)))


def test_layernorm_eps_zero_constant_row_is_nan():
    y = oracle.layernorm(np.full((1, 4), 2.0, np.float32), None, eps=0.0)
    assert np.isnan(y).all()


def test_rmsnorm_worked_rows():
    # [3, 4]: mean square (9+16)/2 = 25/2; eps 7/2 -> 16 -> sqrt 4 -> [3/4, 1].
    assert np.array_equal(oracle.rmsnorm(row(3, 4), eps=3.5), [[0.75, 1.0]])
    # [1,-1,1,-1], eps 0: mean square 1 -> unchanged.
    assert np.array_equal(oracle.rmsnorm(row(1, -1, 1, -1), eps=0.0), [[1, -1, 1, -1]])
    # [2, 2, 2, 2], eps 0: mean square 4 -> all ones (mean of x would be 2
    # too, but [2, -2, 2, -2] tells x^2 from x: its mean is 0).
    assert np.array_equal(oracle.rmsnorm(row(2, -2, 2, -2), eps=0.0), [[1, -1, 1, -1]])
    # Zero row -> 0 / sqrt(eps) = 0.
    assert np.array_equal(oracle.rmsnorm(np.zeros((2, 5), np.float32), eps=1e-6), np.zeros((2, 5)))
    # [3, 4] with the FP32 eps 1e-6: 3/sqrt(12.5 + eps), 4/sqrt(12.5 + eps)
    e = float(f32(1e-6))
    d = math.sqrt(12.5 + e)
    np.testing.assert_allclose(oracle.rmsnorm(row(3, 4), eps=1e-6), [[3 / d, 4 / d]], rtol=1e-15)


def test_softmax_worked_rows():
    assert np.array_equal(oracle.softmax(row(0, 0, 0, 0)), [[0.25] * 4])
    # A huge gap: exp(-1000) underflows to 0 in FP64, so [0, 1000] -> [0, 1];
    # without max subtraction exp(1000) = inf and the row would be NaN.
    assert np.array_equal(oracle.softmax(row(0, 1000)), [[0.0, 1.0]])
    assert np.array_equal(oracle.softmax(row(-1000, -1000)), [[0.5, 0.5]])
    # -inf entries get weight exactly 0.
    assert np.array_equal(oracle.softmax(row(0, -np.inf)), [[1.0, 0.0]])
    assert np.array_equal(oracle.softmax(row(5, 5, -np.inf)), [[0.5, 0.5, 0.0]])
    # exp(ln k) = k: [0, ln 2, ln 3] -> [1, 2, 3] / 6 (up to FP32 input rounding,
    # which moves each log by < 2^-24 relative, i.e. < 1e-7 relative in y).
    y = oracle.softmax(row(0.0, math.log(2.0), math.log(3.0)))
    np.testing.assert_allclose(y, [[1 / 6, 2 / 6, 3 / 6]], rtol=2e-7)
    # Uneven row: [1, 2, 3] -> e^k / (e + e^2 + e^3)
    e1, e2, e3 = math.e, math.e ** 2, math.e ** 3
    s = e1 + e2 + e3
    np.testing.assert_allclose(oracle.softmax(row(1, 2, 3)), [[e1 / s, e2 / s, e3 / s]], rtol=1e-14)


def test_softmax_all_neg_inf_row_is_nan():
    y = oracle.softmax(row(-np.inf, -np.inf, -np.inf))
    assert np.isnan(y).all()


def test_row_sum_and_minmax_worked():
    x = np.array([[1, 2, 3, 4], [-1, 0.5, -7, 2]], dtype=np.float32)
    assert np.array_equal(oracle.row_sum(x), [10.0, -5.5])
    lo, hi = oracle.row_minmax(x)
    assert np.array_equal(lo, [1.0, -7.0]) and np.array_equal(hi, [4.0, 2.0])
    lo, hi = oracle.row_minmax(np.zeros((2, 0), np.float32))
    assert np.array_equal(lo, [np.inf, np.inf]) and np.array_equal(hi, [-np.inf, -np.inf])
    # NaN entries are skipped (minNum/maxNum); an all-NaN row is like the empty row
    nan = np.nan
    lo, hi = oracle.row_minmax(np.array([[nan, 3, -2, nan], [nan, nan, nan, nan]], np.float32))
    assert np.array_equal(lo, [-2.0, np.inf]) and np.array_equal(hi, [3.0, -np.inf])


# --------------------------------------------------------------------------
# Invariants on seeded random rows
# --------------------------------------------------------------------------

def dyadic(seed, rows, width, scale=1024):
    """Random multiples of 1/scale in [-1, 1]: sums of two and shifts by small
    powers of two stay exact in FP32."""
    rng = np.random.default_rng(seed)
    return (rng.integers(-scale, scale + 1, size=(rows, width)) / scale).astype(np.float32)


@pytest.mark.parametrize("width", [1, 2, 3, 7, 64, 127, 257, 1000])
def test_softmax_invariants(width):
    x = synthetic.random_matrix(11, 33, width, "normal") * np.float32(4)
    y = oracle.softmax(x)
    np.testing.assert_allclose(y.sum(axis=1), 1.0, rtol=0, atol=1e-14 * max(1, width))
    assert (y >= 0).all() and (y <= 1).all()
    # order preserving
    for i in range(x.shape[0]):
        o = np.argsort(x[i], kind="stable")
        assert (np.diff(y[i][o]) >= 0).all()
    # shift invariance: x + 8 is exact for dyadic inputs
    xd = dyadic(3, 17, width)
    np.testing.assert_allclose(oracle.softmax(xd + np.float32(8)), oracle.softmax(xd), rtol=1e-13, atol=0)
    # argmax gets the largest weight, ties equal
    xt = np.zeros((1, width), np.float32)
    np.testing.assert_allclose(oracle.softmax(xt), 1.0 / width, rtol=1e-15)


@pytest.mark.parametrize("width", [2, 3, 8, 127, 257, 4096])
def test_layernorm_invariants(width):
    x = synthetic.random_matrix(21, 19, width, "uniform")
    r = synthetic.random_matrix(22, 19, width, "uniform", tensor="r")
    # eps = 0: zero mean and unit (biased) variance
    y = oracle.layernorm_residual(x, r, eps=0.0)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)
    # symmetry of x and r (x + r commutes)
    assert np.array_equal(oracle.layernorm_residual(x, r, 1e-5), oracle.layernorm_residual(r, x, 1e-5))
    # LN(x, r) = LN(x + r) when the FP32 sum is exact (dyadic inputs)
    xd, rd = dyadic(5, 19, width), dyadic(6, 19, width)
    assert np.array_equal(oracle.layernorm_residual(xd, rd, 1e-5), oracle.layernorm(xd + rd, None, eps=1e-5))
    # shift invariance: adding 4 to every element (exact for dyadic rows)
    np.testing.assert_allclose(oracle.layernorm(xd + np.float32(4), None, eps=1e-5),
                               oracle.layernorm(xd, None, eps=1e-5), rtol=1e-12, atol=1e-12)
    # scale invariance at eps = 0 (doubling is exact)
    np.testing.assert_allclose(oracle.layernorm(xd * np.float32(2), None, eps=0.0),
                               oracle.layernorm(xd, None, eps=0.0), rtol=1e-13, atol=1e-13)
    # With eps > 0 the output's mean square is var / (var + eps) < 1, and the
    # output is the eps = 0 output times sqrt(var / (var + eps)).
    eps = float(f32(1e-5))
    c = x.astype(np.float64) + r.astype(np.float64)
    var = c.var(axis=1, keepdims=True)
    ratio = np.sqrt(var / (var + eps))
    np.testing.assert_allclose(oracle.layernorm_residual(x, r, 1e-5), y * ratio, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("width", [1, 2, 5, 127, 1537])
def test_rmsnorm_invariants(width):
    x = synthetic.random_matrix(31, 23, width, "normal")
    y = oracle.rmsnorm(x, eps=0.0)
    np.testing.assert_allclose((y * y).mean(axis=1), 1.0, rtol=1e-13)
    # y / x is one constant per row
    ratio = y / x.astype(np.float64)
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones_like(ratio), rtol=1e-15)
    # scale invariance at eps = 0
    np.testing.assert_allclose(oracle.rmsnorm(x * np.float32(4), eps=0.0), y, rtol=1e-14)
    # sign symmetry
    assert np.array_equal(oracle.rmsnorm(-x, eps=1e-6), -oracle.rmsnorm(x, eps=1e-6))


def test_row_sum_minmax_invariants():
    x = synthetic.random_matrix(41, 50, 333, "normal")
    s = oracle.row_sum(x)
    exact = np.array([math.fsum(map(float, x[i])) for i in range(x.shape[0])])
    np.testing.assert_allclose(s, exact, rtol=1e-13, atol=1e-12)
    lo, hi = oracle.row_minmax(x)
    assert np.array_equal(lo, x.min(axis=1).astype(np.float64))
    assert np.array_equal(hi, x.max(axis=1).astype(np.float64))


def test_threads_do_not_change_results():
    x = synthetic.random_matrix(51, 101, 129, "normal")
    r = synthetic.random_matrix(52, 101, 129, "normal", tensor="r")
    for op in ("layernorm_residual", "rmsnorm", "softmax"):
        a = oracle.run_op(op, x, r, threads=1)
        b = oracle.run_op(op, x, r, threads=7)
        assert np.array_equal(a, b)


# --------------------------------------------------------------------------
# 40-digit brute force
# --------------------------------------------------------------------------

def _dec_ln(row_x, row_r, eps):
    c = [Decimal(float(a)) + (Decimal(float(b)) if row_r is not None else 0) for a, b in
         zip(row_x, row_r if row_r is not None else row_x)]
    n = Decimal(len(c))
    mu = sum(c) / n
    var = sum((v - mu) ** 2 for v in c) / n
    d = (var + Decimal(eps)).sqrt()
    return [(v - mu) / d for v in c]


def _dec_rms(row_x, eps):
    c = [Decimal(float(a)) for a in row_x]
    d = (sum(v * v for v in c) / Decimal(len(c)) + Decimal(eps)).sqrt()
    return [v / d for v in c]


def _dec_softmax(row_x):
    c = [Decimal(float(a)) for a in row_x]
    m = max(c)
    e = [(v - m).exp() for v in c]
    s = sum(e)
    return [v / s for v in e]


def _close(y, ref, rel=1e-13):
    for a, b in zip(y, ref):
        b = float(b)
        assert abs(a - b) <= rel * abs(b) + 1e-300, (a, b)


@pytest.mark.parametrize("width", [1, 2, 3, 5, 8, 13, 16])
def test_bruteforce_decimal(width):
    getcontext().prec = 40
    x = synthetic.random_matrix(61, 12, width, "normal") * np.float32(3)
    r = synthetic.random_matrix(62, 12, width, "uniform", tensor="r")
    e5, e6 = float(f32(1e-5)), float(f32(1e-6))
    yl = oracle.layernorm_residual(x, r, eps=1e-5)
    yr = oracle.rmsnorm(x, eps=1e-6)
    ys = oracle.softmax(x)
    for i in range(x.shape[0]):
        _close(yr[i], _dec_rms(x[i], e6))
        _close(ys[i], _dec_softmax(x[i]))
        if width >= 2:
            _close(yl[i], _dec_ln(x[i], r[i], e5), rel=1e-12)


# --------------------------------------------------------------------------
# Independent library implementations in float64 (torch CPU)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(5, 1), (9, 33), (17, 257), (4, 4096)])
def test_against_torch_float64(shape):
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    x = synthetic.random_matrix(71, *shape, "normal")
    r = synthetic.random_matrix(72, *shape, "uniform", tensor="r")
    tx = torch.from_numpy(x).double()
    tr = torch.from_numpy(r).double()
    e5, e6 = float(f32(1e-5)), float(f32(1e-6))
    ref_sm = torch.softmax(tx, dim=1).numpy()
    ref_ln = F.layer_norm(tx + tr, (shape[1],), eps=e5).numpy()
    ref_rms = F.rms_norm(tx, (shape[1],), eps=e6).numpy()
    np.testing.assert_allclose(oracle.softmax(x), ref_sm, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.layernorm_residual(x, r, eps=1e-5), ref_ln, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.rmsnorm(x, eps=1e-6), ref_rms, rtol=1e-12, atol=1e-15)
    # affine LayerNorm
    g = synthetic.random_matrix(73, 1, shape[1], "normal", tensor="gamma")[0]
    b = synthetic.random_matrix(74, 1, shape[1], "normal", tensor="beta")[0]
    ref_aff = F.layer_norm(tx, (shape[1],), weight=torch.from_numpy(g).double(),
                           bias=torch.from_numpy(b).double(), eps=e5).numpy()
    np.testing.assert_allclose(oracle.layernorm(x, None, eps=1e-5, gamma=g, beta=b), ref_aff,
                               rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# The comparison rule itself
# --------------------------------------------------------------------------

def test_within_tolerance_rule():
    ref = np.array([0.0, 1.0, -2.0, np.nan, -np.inf])
    ok, _, _ = oracle.within_tolerance(ref + np.array([1e-5, 2e-5 - 1e-12, -3e-5 + 1e-12, 0, 0]), ref)
    assert ok
    ok, _, idx = oracle.within_tolerance(ref + np.array([0, 2.1e-5, 0, 0, 0]), ref)
    assert not ok and idx == (1,)
    ok, _, _ = oracle.within_tolerance(np.array([0.0, 1.0, -2.0, 0.0, -np.inf]), ref)
    assert not ok  # NaN must sit where the reference has NaN
    ok, _, _ = oracle.within_tolerance(np.array([0.0, 1.0, -2.0, np.nan, 0.0]), ref)
    assert not ok  # infinities must match
