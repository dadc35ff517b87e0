"""Plant plausible mistakes in a copy of the oracle (CPU only) and check that
the pins catch every one of them.

Each mutant is the oracle's C source with one textual change (a dropped term,
a wrong sign, a wrong index or divisor, a misplaced eps, a missing max
subtraction ...), built with gcc into a temporary library.  The battery below
re-runs a compact selection of the pins from ``test_oracle_pins.py``
(worked rows, invariants and 40-digit brute force) against the mutant; a
mutant that passes every pin would mean the pins cannot tell it from the
definition.
"""
import math
import os
import subprocess
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import synthetic

SRC = os.path.join(os.path.dirname(oracle.__file__), "rowred_oracle.c")


def _nth_replace(src, old, new, occurrence):
    idx = -1
    for _ in range(occurrence + 1):
        idx = src.find(old, idx + 1)
        assert idx >= 0, f"mutation anchor not found: {old!r} #{occurrence}"
    return src[:idx] + new + src[idx + len(old):]


# (name, anchor, replacement, occurrence)
MUTANTS = [
    ("ln_unbiased_variance", "double var = sq / (double)width;", "double var = sq / (double)(width - 1);", 0),
    ("ln_eps_outside_sqrt", "double denom = sqrt(var + eps);", "double denom = sqrt(var) + eps;", 0),
    ("ln_residual_subtracted", "(double)xi[j] + (ri ?", "(double)xi[j] - (ri ?", 0),
    ("ln_residual_dropped", "(ri ? (double)ri[j] : 0.0)", "0.0", 0),
    ("ln_no_centering", "yi[j] = yi[j] - mean;", "yi[j] = yi[j];", 0),
    ("ln_mean_drops_first", "for (int64_t j = 0; j < width; ++j) sum += yi[j];",
     "for (int64_t j = 1; j < width; ++j) sum += yi[j];", 0),
    ("ln_var_drops_last", "for (int64_t j = 0; j < width; ++j) sq += yi[j] * yi[j];",
     "for (int64_t j = 0; j + 1 < width; ++j) sq += yi[j] * yi[j];", 0),
    ("ln_multiplies_by_denom", "double v = yi[j] / denom;", "double v = yi[j] * denom;", 0),
    ("ln_row_stride", "const float *xi = x + i * width;", "const float *xi = x + i;", 0),
    ("rms_sum_not_mean", "double ms = sq / (double)width;", "double ms = sq;", 0),
    ("rms_eps_outside_sqrt", "double denom = sqrt(ms + eps);", "double denom = sqrt(ms) + eps;", 0),
    ("rms_drops_first", "for (int64_t j = 0; j < width; ++j) sq += (double)xi[j] * (double)xi[j];",
     "for (int64_t j = 1; j < width; ++j) sq += (double)xi[j] * (double)xi[j];", 0),
    ("rms_abs_not_square", "sq += (double)xi[j] * (double)xi[j];", "sq += fabs((double)xi[j]);", 0),
    ("rms_row_stride", "const float *xi = x + i * width;", "const float *xi = x + i;", 1),
    ("sm_no_max_subtraction", "yi[j] = exp((double)xi[j] - m);", "yi[j] = exp((double)xi[j]);", 0),
    ("sm_min_not_max", "m = fmax(m, (double)xi[j]);", "m = fmin(m, (double)xi[j]);", 0),
    ("sm_no_normalise", "for (int64_t j = 0; j < width; ++j) yi[j] = yi[j] / s;",
     "for (int64_t j = 0; j < width; ++j) yi[j] = yi[j];", 0),
    ("sm_reversed_index", "yi[j] = exp((double)xi[j] - m);", "yi[j] = exp((double)xi[width - 1 - j] - m);", 0),
    ("sm_sum_drops_last", "s += yi[j];", "s += (j + 1 < width) ? yi[j] : 0.0;", 0),
    ("sm_wrong_sign", "yi[j] = exp((double)xi[j] - m);", "yi[j] = exp(m - (double)xi[j]);", 0),
    ("sum_drops_first", "for (int64_t j = 0; j < width; ++j) s += (double)xi[j];",
     "for (int64_t j = 1; j < width; ++j) s += (double)xi[j];", 0),
    ("minmax_swapped", "out_min[i] = lo;", "out_min[i] = hi;", 0),
]


def _row(*v):
    return np.array([v], dtype=np.float32)


def _dec_softmax(xr):
    c = [Decimal(float(a)) for a in xr]
    m = max(c)
    e = [(v - m).exp() for v in c]
    s = sum(e)
    return [float(v / s) for v in e]


def _dec_ln(xr, rr, eps):
    c = [Decimal(float(a)) + Decimal(float(b)) for a, b in zip(xr, rr)]
    n = Decimal(len(c))
    mu = sum(c) / n
    var = sum((v - mu) ** 2 for v in c) / n
    d = (var + Decimal(eps)).sqrt()
    return [float((v - mu) / d) for v in c]


def _dec_rms(xr, eps):
    c = [Decimal(float(a)) for a in xr]
    d = (sum(v * v for v in c) / Decimal(len(c)) + Decimal(eps)).sqrt()
    return [float(v / d) for v in c]


def battery():
    """Run the pin selection; return the names of the pins that fail."""
    getcontext().prec = 40
    failed = []

    def check(name, fn):
        try:
            with np.errstate(all="ignore"):
                ok = bool(fn())
        except Exception:
            ok = False
        if not ok:
            failed.append(name)

    check("ln_worked", lambda: np.array_equal(oracle.layernorm(_row(1, 2, 3, 4), None, eps=2.75),
                                              [[-0.75, -0.25, 0.25, 0.75]]))
    check("ln_res_worked", lambda: np.array_equal(
        oracle.layernorm_residual(_row(0, 0, 0, 0), _row(1, 2, 3, 4), eps=2.75), [[-0.75, -0.25, 0.25, 0.75]]))
    check("ln_pm1", lambda: np.array_equal(oracle.layernorm(_row(-1, 1), None, eps=3.0), [[-0.5, 0.5]]))
    check("rms_worked", lambda: np.array_equal(oracle.rmsnorm(_row(3, 4), eps=3.5), [[0.75, 1.0]]))
    check("rms_pm", lambda: np.array_equal(oracle.rmsnorm(_row(2, -2, 2, -2), eps=0.0), [[1, -1, 1, -1]]))
    check("sm_gap", lambda: np.array_equal(oracle.softmax(_row(0, 1000)), [[0.0, 1.0]]))
    check("sm_uniform", lambda: np.array_equal(oracle.softmax(_row(0, 0, 0, 0)), [[0.25] * 4]))
    check("sum_worked", lambda: np.array_equal(oracle.row_sum(_row(1, 2, 3, 4)), [10.0]))
    check("minmax_worked", lambda: [list(a) for a in oracle.row_minmax(_row(-1, 5, 2))] == [[-1.0], [5.0]])

    x = synthetic.random_matrix(81, 6, 5, "normal") * np.float32(3)
    r = synthetic.random_matrix(82, 6, 5, "uniform", tensor="r")
    e5, e6 = float(np.float32(1e-5)), float(np.float32(1e-6))

    def close(a, b):
        return all(abs(p - q) <= 1e-12 * abs(q) + 1e-300 for p, q in zip(a, b))

    check("brute_sm", lambda: all(close(oracle.softmax(x)[i], _dec_softmax(x[i])) for i in range(6)))
    check("brute_ln", lambda: all(close(oracle.layernorm_residual(x, r, 1e-5)[i], _dec_ln(x[i], r[i], e5))
                                  for i in range(6)))
    check("brute_rms", lambda: all(close(oracle.rmsnorm(x, 1e-6)[i], _dec_rms(x[i], e6)) for i in range(6)))
    check("sum_fsum", lambda: np.allclose(oracle.row_sum(x), [math.fsum(map(float, v)) for v in x],
                                          rtol=1e-13, atol=1e-13))
    return failed


def test_unmutated_oracle_passes_battery(monkeypatch):
    monkeypatch.setattr(oracle, "default_threads", lambda: 1)
    assert battery() == []


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, occ, tmp_path, monkeypatch):
    src = open(SRC).read()
    mutated = _nth_replace(src, old, new, occ)
    assert mutated != src
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so), str(c),
                    "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(str(so)))
    # one thread, so multi-row calls go through the row stride
    monkeypatch.setattr(oracle, "default_threads", lambda: 1)
    failed = battery()
    assert failed, f"mutant {name} passed every pin"
