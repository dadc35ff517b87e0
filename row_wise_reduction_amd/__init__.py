"""Python binding of ``librowred.so``: fused FP32 row reductions on MI355X.

Argument marshalling only -- every step of every reduction runs in the HIP
kernels behind the C ABI declared in ``include/rowred.h``.  There is no
fallback: if the library is not built, or a call fails, an exception is
raised.

Each C entry point has a Python function of the same name.  Matrix
arguments may be torch tensors (CUDA, float32, row-major contiguous; the
last dimension is the row width and leading dimensions are rows) or raw
device addresses (ints, then ``rows`` and ``width`` are required).  With
tensors the call is enqueued on torch's current stream unless ``stream`` (a
raw ``hipStream_t`` as int) is given.  Torch is used for device memory and
streams only.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librowred.so")

ROWRED_OK = 0
ROWRED_ERR_INVALID_ARG = 1
ROWRED_ERR_ALIAS = 2
ROWRED_ERR_UNSUPPORTED = 3
ROWRED_ERR_HIP = 4

ROWRED_POLICY_NT_LOADS = 1
ROWRED_POLICY_NT_STORES = 2
ROWRED_POLICY_XCD_REMAP = 4
ROWRED_POLICY_STAGE_STORES = 8
ROWRED_POLICY_RELOAD = 16
ROWRED_POLICY_REVERSE = 32
ROWRED_POLICY_LOOPED = 64
ROWRED_POLICY_EXCHANGE = 128
ROWRED_POLICY_LDS_STRIPE = 256
ROWRED_POLICY_FLAT = 512
ROWRED_POLICY_ONLINE = 1024
ROWRED_POLICY_CU_GROUPS_SHIFT = 12


def ROWRED_POLICY_CU_GROUPS(n: int) -> int:
    """Policy bits capping the workgroups per compute unit at n (1-14)."""
    return int(n) << ROWRED_POLICY_CU_GROUPS_SHIFT


ROWRED_MAX_WIDTH = 2146435071  # widest row any entry point takes (2^31 - 2^20 - 1)

ROWRED_OP_LAYERNORM_RESIDUAL = 0
ROWRED_OP_RMSNORM = 1
ROWRED_OP_SOFTMAX = 2
ROWRED_OP_ROW_SUM = 3
ROWRED_OP_ROW_MINMAX = 4
OPS = {"layernorm_residual": ROWRED_OP_LAYERNORM_RESIDUAL, "rmsnorm": ROWRED_OP_RMSNORM,
       "softmax": ROWRED_OP_SOFTMAX, "row_sum": ROWRED_OP_ROW_SUM, "row_minmax": ROWRED_OP_ROW_MINMAX}


class RowRedError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({rowred_status_string(status)})")


class _Plan(ctypes.Structure):
    _fields_ = [("lanes_per_row", ctypes.c_int32), ("rows_per_group", ctypes.c_int32),
                ("chunks", ctypes.c_int32), ("threads", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("vector_io", ctypes.c_int32), ("window", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


@dataclass
class Plan:
    lanes_per_row: int
    rows_per_group: int
    chunks: int
    threads: int
    grid: int
    vector_io: int = 0
    window: int = 0
    policy: int = 0
    reserved: int = 0

    def _c(self) -> _Plan:
        return _Plan(self.lanes_per_row, self.rows_per_group, self.chunks, self.threads, self.grid,
                     self.vector_io, self.window, self.policy, self.reserved)


class _SplitPlan(ctypes.Structure):
    _fields_ = [("threads", ctypes.c_int32), ("chunks", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("window", ctypes.c_int32), ("block_rows", ctypes.c_int64), ("segments", ctypes.c_int64),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64), ("wait_polls", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


@dataclass
class SplitPlan:
    threads: int = 0
    chunks: int = 0
    policy: int = 0
    window: int = 0
    block_rows: int = 0
    segments: int = 0
    grid: int = 0
    workspace_bytes: int = 0
    wait_polls: int = 0
    reserved: int = 0

    def _c(self) -> _SplitPlan:
        return _SplitPlan(self.threads, self.chunks, self.policy, self.window, self.block_rows, self.segments,
                          self.grid, self.workspace_bytes, self.wait_polls, self.reserved)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64


def lib():
    """The loaded ``librowred.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m row_wise_reduction_amd.build`")
        # torch ships its own copy of the HIP runtime under the same soname.
        # Loaded first, it is the one this library binds to; loaded after
        # this library, it would be a second runtime in the process, and
        # torch's streams would be invalid handles to ours.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "rowred_layernorm_residual": [_P, _P, _P, _I64, _I64, ctypes.c_float, _P],
            "rowred_rmsnorm": [_P, _P, _I64, _I64, ctypes.c_float, _P],
            "rowred_layernorm": [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P],
            "rowred_layernorm_run_plan": [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, ctypes.POINTER(_Plan), _P],
            "rowred_softmax": [_P, _P, _I64, _I64, _P],
            "rowred_plan_query": [ctypes.c_int, _P, _P, _P, _I64, _I64, ctypes.POINTER(_Plan)],
            "rowred_layernorm_plan_query": [_P, _P, _P, _P, _P, _I64, _I64, ctypes.POINTER(_Plan)],
            "rowred_run_plan": [ctypes.c_int, _P, _P, _P, _I64, _I64, ctypes.c_float, ctypes.POINTER(_Plan), _P],
            "rowred_copy": [_P, _P, _I64, _P],
            "rowred_row_sum": [_P, _P, _I64, _I64, _P],
            "rowred_row_minmax": [_P, _P, _P, _I64, _I64, _P],
            "rowred_row_reduce_run_plan": [ctypes.c_int, _P, _P, _P, _I64, _I64, ctypes.POINTER(_Plan), _P],
            "rowred_workspace_size": [ctypes.c_int, _I64, _I64, ctypes.POINTER(ctypes.c_size_t)],
            "rowred_layernorm_ws": [_P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P, ctypes.c_size_t, _P],
            "rowred_rmsnorm_ws": [_P, _P, _I64, _I64, ctypes.c_float, _P, ctypes.c_size_t, _P],
            "rowred_softmax_ws": [_P, _P, _I64, _I64, _P, ctypes.c_size_t, _P],
            "rowred_row_sum_ws": [_P, _P, _I64, _I64, _P, ctypes.c_size_t, _P],
            "rowred_row_minmax_ws": [_P, _P, _P, _I64, _I64, _P, ctypes.c_size_t, _P],
            "rowred_split_plan_query": [ctypes.c_int, _P, _I64, _I64, ctypes.POINTER(_SplitPlan)],
            "rowred_split_run_plan": [ctypes.c_int, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float,
                                      ctypes.POINTER(_SplitPlan), _P, ctypes.c_size_t, _P],
            "rowred_static_ws": [ctypes.c_int, _P, _P, _P, _P, _P, _P, _I64, _I64, ctypes.c_float, _P],
        }
        for name, argtypes in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        L.rowred_status_string.argtypes = [ctypes.c_int]
        L.rowred_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def rowred_status_string(status: int) -> str:
    return lib().rowred_status_string(int(status)).decode()


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _is_tensor(a) -> bool:
    return hasattr(a, "data_ptr") and hasattr(a, "dtype")


def _matrix(a, name, rows=None, width=None):
    """(address, rows, width) of a tensor or raw address."""
    if a is None:
        return None, rows, width
    if _is_tensor(a):
        import torch
        if a.dtype != torch.float32:
            raise TypeError(f"{name} must be float32, got {a.dtype}")
        if not a.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        if not a.is_contiguous():
            raise ValueError(f"{name} must be row-major contiguous")
        if a.dim() == 0:
            return a.data_ptr(), 1, 1
        r = 1
        for d in a.shape[:-1]:
            r *= int(d)
        return a.data_ptr(), r, int(a.shape[-1])
    return int(a), rows, width


def _shape(pairs, rows, width):
    """Check that every tensor argument agrees on (rows, width)."""
    for name, (addr, r, w) in pairs:
        if addr is None:
            continue
        if rows is None:
            rows, width = r, w
        elif (r, w) != (rows, width):
            raise ValueError(f"{name} has shape ({r}, {w}), expected ({rows}, {width})")
    if rows is None or width is None:
        raise ValueError("rows and width are required with raw addresses")
    return int(rows), int(width)


def _stream(stream, *args):
    if stream is not None:
        return int(stream)
    if any(_is_tensor(a) for a in args):
        import torch
        return torch.cuda.current_stream().cuda_stream
    return 0


def _check(status, what):
    if status != ROWRED_OK:
        raise RowRedError(status, what)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def rowred_layernorm_residual(x, r, y, rows=None, width=None, eps=1e-5, stream=None):
    """y = (x + r - mean) / sqrt(var + eps) per row (biased variance, no affine)."""
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    st = lib().rowred_layernorm_residual(mx[0], mr[0], my[0], rows, width, float(eps), _stream(stream, x, r, y))
    _check(st, "rowred_layernorm_residual")


def _vector(v, name, width):
    """Address of a length-`width` vector (tensor or raw address), or None."""
    if v is None:
        return None
    if _is_tensor(v):
        addr, r, w = _matrix(v, name)
        if r * w != width:
            raise ValueError(f"{name} must hold width={width} floats")
        return addr
    return int(v)


def rowred_layernorm(x, r, gamma, beta, y, rows=None, width=None, eps=1e-5, stream=None):
    """LayerNorm with optional residual r and affine gamma/beta (each may be None)."""
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    st = lib().rowred_layernorm(mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width), my[0],
                                rows, width, float(eps), _stream(stream, x, r, gamma, beta, y))
    _check(st, "rowred_layernorm")


def rowred_layernorm_run_plan(x, r, gamma, beta, y, plan: "Plan", rows=None, width=None, eps=1e-5, stream=None):
    """rowred_layernorm with an explicit launch plan."""
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    c = plan._c()
    st = lib().rowred_layernorm_run_plan(mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width),
                                         my[0], rows, width, float(eps), ctypes.byref(c),
                                         _stream(stream, x, r, gamma, beta, y))
    _check(st, "rowred_layernorm_run_plan")


def rowred_layernorm_plan_query(x, r, gamma, beta, y, rows=None, width=None) -> "Plan":
    """The plan rowred_layernorm would launch (host only; no device work)."""
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    p = _Plan()
    st = lib().rowred_layernorm_plan_query(mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width),
                                           my[0], rows, width, ctypes.byref(p))
    _check(st, "rowred_layernorm_plan_query")
    return Plan(p.lanes_per_row, p.rows_per_group, p.chunks, p.threads, p.grid, p.vector_io, p.window, p.policy,
                p.reserved)


def _row_vector(v, name, rows):
    if v is None:
        return None
    if _is_tensor(v):
        addr, r, w = _matrix(v, name)
        if r * w != rows:
            raise ValueError(f"{name} must hold rows={rows} floats")
        return addr
    return int(v)


def rowred_row_sum(x, out, rows=None, width=None, stream=None):
    """out[i] = sum_j x[i, j] (FP64 accumulation, FP32 result)."""
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    st = lib().rowred_row_sum(mx[0], _row_vector(out, "out", rows), rows, width, _stream(stream, x, out))
    _check(st, "rowred_row_sum")


def rowred_row_minmax(x, out_min, out_max, rows=None, width=None, stream=None):
    """out_min[i] = min_j x[i, j], out_max[i] = max_j x[i, j] (NaN skipped)."""
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    st = lib().rowred_row_minmax(mx[0], _row_vector(out_min, "out_min", rows), _row_vector(out_max, "out_max", rows),
                                 rows, width, _stream(stream, x, out_min, out_max))
    _check(st, "rowred_row_minmax")


def rowred_row_reduce_run_plan(op, x, out0, out1, plan: "Plan", rows=None, width=None, stream=None):
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    c = plan._c()
    st = lib().rowred_row_reduce_run_plan(_op_id(op), mx[0], _row_vector(out0, "out0", rows),
                                          _row_vector(out1, "out1", rows), rows, width, ctypes.byref(c),
                                          _stream(stream, x, out0, out1))
    _check(st, "rowred_row_reduce_run_plan")


def rowred_rmsnorm(x, y, rows=None, width=None, eps=1e-6, stream=None):
    """y = x / sqrt(mean(x^2) + eps) per row (no weight)."""
    mx, my = _matrix(x, "x", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("y", my)], rows, width)
    st = lib().rowred_rmsnorm(mx[0], my[0], rows, width, float(eps), _stream(stream, x, y))
    _check(st, "rowred_rmsnorm")


def rowred_softmax(x, y, rows=None, width=None, stream=None):
    """y = exp(x - max) / sum(exp(x - max)) per row."""
    mx, my = _matrix(x, "x", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("y", my)], rows, width)
    st = lib().rowred_softmax(mx[0], my[0], rows, width, _stream(stream, x, y))
    _check(st, "rowred_softmax")


def _op_id(op):
    return OPS[op] if isinstance(op, str) else int(op)


def rowred_plan_query(op, x, r, y, rows=None, width=None) -> Plan:
    """The plan the entry point would launch (host only; no device work).
    For row_sum / row_minmax, y is the (first) output vector and r the
    row-max vector of row_minmax."""
    op = _op_id(op)
    if op in (OPS["row_sum"], OPS["row_minmax"]):
        mx = _matrix(x, "x", rows, width)
        rows, width = _shape([("x", mx)], rows, width)
        ar, ay = _row_vector(r, "out_max", rows), _row_vector(y, "out", rows)
    else:
        mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
        rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
        ar, ay = mr[0], my[0]
    p = _Plan()
    st = lib().rowred_plan_query(op, mx[0], ar, ay, rows, width, ctypes.byref(p))
    _check(st, "rowred_plan_query")
    return Plan(p.lanes_per_row, p.rows_per_group, p.chunks, p.threads, p.grid, p.vector_io, p.window, p.policy,
                p.reserved)


def rowred_run_plan(op, x, r, y, plan: Plan, rows=None, width=None, eps=0.0, stream=None):
    """Run `op` with an explicit launch plan."""
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    c = plan._c()
    st = lib().rowred_run_plan(_op_id(op), mx[0], mr[0], my[0], rows, width, float(eps), ctypes.byref(c),
                               _stream(stream, x, r, y))
    _check(st, "rowred_run_plan")


# ----------------------------------------------------------------------------
# any width / split rows (caller-provided workspace)
# ----------------------------------------------------------------------------

def _workspace(ws):
    """(address, bytes) of a workspace tensor, or (address, bytes) passed as
    a pair of ints."""
    if ws is None:
        return None, 0
    if _is_tensor(ws):
        if not ws.is_cuda or not ws.is_contiguous():
            raise TypeError("workspace must be a contiguous CUDA (HIP) tensor")
        return ws.data_ptr(), ws.numel() * ws.element_size()
    addr, nbytes = ws
    return int(addr), int(nbytes)


def rowred_workspace_size(op, rows, width) -> int:
    """Workspace bytes the _ws entry point of `op` needs at this shape."""
    n = ctypes.c_size_t()
    _check(lib().rowred_workspace_size(_op_id(op), int(rows), int(width), ctypes.byref(n)), "rowred_workspace_size")
    return n.value


def new_workspace(op, rows, width):
    """A torch uint8 CUDA tensor of rowred_workspace_size bytes (at least 16).
    torch allocations are 256-byte aligned."""
    import torch
    return torch.empty(max(16, rowred_workspace_size(op, rows, width)), dtype=torch.uint8, device="cuda")


def rowred_layernorm_ws(x, r, gamma, beta, y, workspace, rows=None, width=None, eps=1e-5, stream=None):
    mx, mr, my = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
    wa, wn = _workspace(workspace)
    st = lib().rowred_layernorm_ws(mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width), my[0],
                                   rows, width, float(eps), wa, wn, _stream(stream, x, r, gamma, beta, y))
    _check(st, "rowred_layernorm_ws")


def rowred_rmsnorm_ws(x, y, workspace, rows=None, width=None, eps=1e-6, stream=None):
    mx, my = _matrix(x, "x", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("y", my)], rows, width)
    wa, wn = _workspace(workspace)
    _check(lib().rowred_rmsnorm_ws(mx[0], my[0], rows, width, float(eps), wa, wn, _stream(stream, x, y)),
           "rowred_rmsnorm_ws")


def rowred_softmax_ws(x, y, workspace, rows=None, width=None, stream=None):
    mx, my = _matrix(x, "x", rows, width), _matrix(y, "y", rows, width)
    rows, width = _shape([("x", mx), ("y", my)], rows, width)
    wa, wn = _workspace(workspace)
    _check(lib().rowred_softmax_ws(mx[0], my[0], rows, width, wa, wn, _stream(stream, x, y)), "rowred_softmax_ws")


def rowred_row_sum_ws(x, out, workspace, rows=None, width=None, stream=None):
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    wa, wn = _workspace(workspace)
    _check(lib().rowred_row_sum_ws(mx[0], _row_vector(out, "out", rows), rows, width, wa, wn, _stream(stream, x, out)),
           "rowred_row_sum_ws")


def rowred_row_minmax_ws(x, out_min, out_max, workspace, rows=None, width=None, stream=None):
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    wa, wn = _workspace(workspace)
    _check(lib().rowred_row_minmax_ws(mx[0], _row_vector(out_min, "out_min", rows),
                                      _row_vector(out_max, "out_max", rows), rows, width, wa, wn,
                                      _stream(stream, x, out_min, out_max)), "rowred_row_minmax_ws")


def rowred_split_plan_query(op, x, rows=None, width=None, plan: SplitPlan = None) -> SplitPlan:
    """The split plan the _ws entry points use (plan None), or `plan` checked
    and completed."""
    mx = _matrix(x, "x", rows, width)
    rows, width = _shape([("x", mx)], rows, width)
    c = (plan or SplitPlan())._c()
    _check(lib().rowred_split_plan_query(_op_id(op), mx[0], rows, width, ctypes.byref(c)), "rowred_split_plan_query")
    return SplitPlan(c.threads, c.chunks, c.policy, c.window, c.block_rows, c.segments, c.grid, c.workspace_bytes,
                     c.wait_polls, c.reserved)


def rowred_split_run_plan(op, x, r, gamma, beta, y, y2, plan: SplitPlan, workspace, rows=None, width=None, eps=0.0,
                          stream=None):
    """The split kernels with an explicit plan.  For row_sum / row_minmax, y
    (and y2) are row vectors."""
    op = _op_id(op)
    mx, mr = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width)
    if op in (ROWRED_OP_ROW_SUM, ROWRED_OP_ROW_MINMAX):
        rows, width = _shape([("x", mx)], rows, width)
        ay, ay2 = _row_vector(y, "y", rows), _row_vector(y2, "y2", rows)
    else:
        my = _matrix(y, "y", rows, width)
        rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
        ay, ay2 = my[0], _row_vector(y2, "y2", rows)
    wa, wn = _workspace(workspace)
    c = plan._c()
    st = lib().rowred_split_run_plan(op, mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width),
                                     ay, ay2, rows, width, float(eps), ctypes.byref(c), wa, wn,
                                     _stream(stream, x, r, gamma, beta, y, y2, workspace))
    _check(st, "rowred_split_run_plan")


ROWRED_STATIC_WORKSPACE_BYTES = 8 << 20  # the library's static workspace per GPU (rowred_static_ws)


def rowred_static_ws(op, x, r, gamma, beta, y, y2=None, rows=None, width=None, eps=0.0, stream=None):
    """The _ws entry point of `op` on the library's static workspace (no
    workspace argument; nothing allocated).  For row_sum / row_minmax, y
    (and y2) are row vectors."""
    op = _op_id(op)
    mx, mr = _matrix(x, "x", rows, width), _matrix(r, "r", rows, width)
    if op in (ROWRED_OP_ROW_SUM, ROWRED_OP_ROW_MINMAX):
        rows, width = _shape([("x", mx)], rows, width)
        ay, ay2 = _row_vector(y, "y", rows), _row_vector(y2, "y2", rows)
    else:
        my = _matrix(y, "y", rows, width)
        rows, width = _shape([("x", mx), ("r", mr), ("y", my)], rows, width)
        ay, ay2 = my[0], _row_vector(y2, "y2", rows)
    st = lib().rowred_static_ws(op, mx[0], mr[0], _vector(gamma, "gamma", width), _vector(beta, "beta", width),
                                ay, ay2, rows, width, float(eps), _stream(stream, x, r, gamma, beta, y, y2))
    _check(st, "rowred_static_ws")


def rowred_copy(x, y, n=None, stream=None):
    """y[:n] = x[:n] with the library's streaming 16-byte copy (measurement aid)."""
    if _is_tensor(x):
        n = x.numel() if n is None else n
    st = lib().rowred_copy(_matrix(x, "x")[0] if _is_tensor(x) else int(x),
                           _matrix(y, "y")[0] if _is_tensor(y) else int(y), int(n), _stream(stream, x, y))
    _check(st, "rowred_copy")


# Short aliases over tensors (allocate the output with torch when not given).

def layernorm_residual(x, r, out=None, eps=1e-5):
    import torch
    out = torch.empty_like(x) if out is None else out
    rowred_layernorm_residual(x, r, out, eps=eps)
    return out


def rmsnorm(x, out=None, eps=1e-6):
    import torch
    out = torch.empty_like(x) if out is None else out
    rowred_rmsnorm(x, out, eps=eps)
    return out


def softmax(x, out=None):
    import torch
    out = torch.empty_like(x) if out is None else out
    rowred_softmax(x, out)
    return out


def run_op(op: str, x, r, y, eps=None):
    """Dispatch by operator name with the pages' eps defaults (1e-5 LN, 1e-6 RMS)."""
    if op == "layernorm_residual":
        rowred_layernorm_residual(x, r, y, eps=1e-5 if eps is None else eps)
    elif op == "rmsnorm":
        rowred_rmsnorm(x, y, eps=1e-6 if eps is None else eps)
    elif op == "softmax":
        rowred_softmax(x, y)
    else:
        raise ValueError(f"unknown op {op!r}")
