"""FP64 CPU oracle for the fused row reductions.

TEST INFRASTRUCTURE ONLY.  The test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers allowed.  The product path
(the HIP library and its Python binding) never imports this module, and this
module imports nothing from the product path.

The arithmetic lives in ``rowred_oracle.c`` (plain sequential FP64 loops, one
row at a time, see that file for the definitions and the pages each follows).
This wrapper only compiles it with gcc, marshals numpy arrays and splits the
row range over threads: rows are independent, so a split changes no
floating-point operation.

Input arrays are float32 (the precision the method works in); outputs are
float64.  ``eps`` is taken as the float32 value the kernels use, widened
exactly to double.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rowred_oracle.c")
_LIB = os.path.join(_HERE, "librowred_oracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc into ``oracle/librowred_oracle.so``.

    -O2 without -ffast-math: no reassociation, contraction or reordering of
    the FP64 loops (``-ffp-contract=off`` keeps every multiply and add
    separately rounded, exactly as written)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path: str):
    """Open a compiled oracle library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.rowred_oracle_layernorm.argtypes = [f32p, f32p, f32p, f32p, f64p, i64, i64, ctypes.c_double]
    lib.rowred_oracle_rmsnorm.argtypes = [f32p, f64p, i64, i64, ctypes.c_double]
    lib.rowred_oracle_softmax.argtypes = [f32p, f64p, i64, i64]
    lib.rowred_oracle_row_sum.argtypes = [f32p, f64p, i64, i64]
    lib.rowred_oracle_row_minmax.argtypes = [f32p, f64p, f64p, i64, i64]
    for fn in (lib.rowred_oracle_layernorm, lib.rowred_oracle_rmsnorm, lib.rowred_oracle_softmax,
               lib.rowred_oracle_row_sum, lib.rowred_oracle_row_minmax):
        fn.restype = None
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = load_library(_LIB)
    return _lib


def default_threads() -> int:
    """Cores in this process's affinity mask, capped at 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _f32(a, name):
    a = np.ascontiguousarray(a, dtype=np.float32)
    if a.ndim != 2:
        raise ValueError(f"{name} must be 2-D (rows, width), got shape {a.shape}")
    return a


def _ptr(a, ctype, offset_elems=0):
    if a is None:
        return None
    return ctypes.cast(a.ctypes.data + offset_elems * a.itemsize, ctypes.POINTER(ctype))


def _split(rows: int, threads: int):
    threads = max(1, min(threads, rows))
    step = -(-rows // threads) if rows else 0
    return [(s, min(rows, s + step)) for s in range(0, rows, step)] if rows else []


def _run_rows(fn, rows, threads):
    blocks = _split(rows, threads)
    if len(blocks) <= 1:
        for b in blocks:
            fn(*b)
        return
    with ThreadPoolExecutor(max_workers=len(blocks)) as ex:
        list(ex.map(lambda b: fn(*b), blocks))


def layernorm(x, r=None, eps=1e-5, gamma=None, beta=None, threads=None):
    """Residual LayerNorm (``r`` given) or plain LayerNorm (``r=None``), no
    affine unless ``gamma``/``beta`` (1-D, length width) are given."""
    lib = _load()
    x = _f32(x, "x")
    rows, width = x.shape
    if r is not None:
        r = _f32(r, "r")
        if r.shape != x.shape:
            raise ValueError("r must have the shape of x")
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32).reshape(-1)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float32).reshape(-1)
    for v, nm in ((g, "gamma"), (b, "beta")):
        if v is not None and v.shape[0] != width:
            raise ValueError(f"{nm} must have length width")
    y = np.empty((rows, width), dtype=np.float64)
    e = float(np.float32(eps))

    def run(s, t):
        lib.rowred_oracle_layernorm(
            _ptr(x, ctypes.c_float, s * width),
            _ptr(r, ctypes.c_float, s * width) if r is not None else None,
            _ptr(g, ctypes.c_float), _ptr(b, ctypes.c_float),
            _ptr(y, ctypes.c_double, s * width), t - s, width, e)

    _run_rows(run, rows, threads or default_threads())
    return y


def layernorm_residual(x, r, eps=1e-5, threads=None):
    """y = (x + r - mean) / sqrt(var + eps), biased two-pass variance."""
    if r is None:
        raise ValueError("residual LayerNorm needs r")
    return layernorm(x, r, eps=eps, threads=threads)


def rmsnorm(x, eps=1e-6, threads=None):
    """y = x / sqrt(mean(x^2) + eps)."""
    lib = _load()
    x = _f32(x, "x")
    rows, width = x.shape
    y = np.empty((rows, width), dtype=np.float64)
    e = float(np.float32(eps))

    def run(s, t):
        lib.rowred_oracle_rmsnorm(_ptr(x, ctypes.c_float, s * width),
                                  _ptr(y, ctypes.c_double, s * width), t - s, width, e)

    _run_rows(run, rows, threads or default_threads())
    return y


def softmax(x, threads=None):
    """y = exp(x - max) / sum(exp(x - max)) per row."""
    lib = _load()
    x = _f32(x, "x")
    rows, width = x.shape
    y = np.empty((rows, width), dtype=np.float64)

    def run(s, t):
        lib.rowred_oracle_softmax(_ptr(x, ctypes.c_float, s * width),
                                  _ptr(y, ctypes.c_double, s * width), t - s, width)

    _run_rows(run, rows, threads or default_threads())
    return y


def row_sum(x, threads=None):
    """out[i] = sum_j x[i, j] (float64, shape (rows,))."""
    lib = _load()
    x = _f32(x, "x")
    rows, width = x.shape
    out = np.empty((rows,), dtype=np.float64)

    def run(s, t):
        lib.rowred_oracle_row_sum(_ptr(x, ctypes.c_float, s * width),
                                  _ptr(out, ctypes.c_double, s), t - s, width)

    _run_rows(run, rows, threads or default_threads())
    return out


def row_minmax(x, threads=None):
    """(min_j x[i, j], max_j x[i, j]) per row, float64 arrays of shape (rows,)."""
    lib = _load()
    x = _f32(x, "x")
    rows, width = x.shape
    lo = np.empty((rows,), dtype=np.float64)
    hi = np.empty((rows,), dtype=np.float64)

    def run(s, t):
        lib.rowred_oracle_row_minmax(_ptr(x, ctypes.c_float, s * width),
                                     _ptr(lo, ctypes.c_double, s), _ptr(hi, ctypes.c_double, s),
                                     t - s, width)

    _run_rows(run, rows, threads or default_threads())
    return lo, hi


def run_op(op: str, x, r=None, eps=None, threads=None, gamma=None, beta=None):
    """Dispatch by operator name: 'layernorm_residual', 'layernorm' (r, gamma,
    beta optional), 'layernorm_affine', 'rmsnorm', 'softmax'."""
    if op == "layernorm_residual":
        return layernorm_residual(x, r, eps=1e-5 if eps is None else eps, threads=threads)
    if op in ("layernorm", "layernorm_affine"):
        return layernorm(x, r, eps=1e-5 if eps is None else eps, gamma=gamma, beta=beta, threads=threads)
    if op == "rmsnorm":
        return rmsnorm(x, eps=1e-6 if eps is None else eps, threads=threads)
    if op == "row_sum":
        return row_sum(x, threads=threads)
    if op == "row_minmax":
        return row_minmax(x, threads=threads)
    if op == "softmax":
        return softmax(x, threads=threads)
    raise ValueError(f"unknown op {op!r}")


def within_tolerance(y, ref, atol=1e-5, rtol=1e-5):
    """Element-wise |y - ref| <= atol + rtol*|ref|, NaN exactly where ref is
    NaN, and infinities equal.  Returns (ok, worst_excess, index)."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    nan_ref = np.isnan(ref)
    nan_y = np.isnan(y)
    if not np.array_equal(nan_ref, nan_y):
        idx = np.argwhere(nan_ref != nan_y)[0]
        return False, float("inf"), tuple(int(i) for i in idx)
    inf_ref = np.isinf(ref)
    if not np.array_equal(y[inf_ref], ref[inf_ref]):
        idx = np.argwhere(inf_ref & (y != ref))[0]
        return False, float("inf"), tuple(int(i) for i in idx)
    fin = ~(nan_ref | inf_ref)
    if not fin.any():
        return True, 0.0, None
    with np.errstate(invalid="ignore"):
        err = np.where(fin, np.abs(y - ref) - (atol + rtol * np.abs(ref)), -np.inf)
    worst = int(np.argmax(err))
    excess = float(err.reshape(-1)[worst])
    return excess <= 0.0, excess, tuple(int(i) for i in np.unravel_index(worst, err.shape))
