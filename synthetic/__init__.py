"""Seeded synthetic inputs for the row-reduction workloads.

This module only draws random numbers; it holds none of the reductions'
arithmetic.  Both the HIP path (tests, benchmark) and the FP64 oracle are fed
the same float32 arrays produced here.

Every array comes from numpy's PCG64 seeded by
``SeedSequence([20260905, cfg, op_id, tensor_id, rows, width])``, drawn in
float64 in row blocks and rounded to float32.

Workloads (rows x width, FP32, row-major, stride = width):

=====  ==========================================  ======================  =========================
cfg    operators                                   shapes                  distribution
=====  ==========================================  ======================  =========================
1      residual LayerNorm (eps 1e-5)               17x257, 1x127           x, r i.i.d. U[-1, 1]
2      softmax, RMSNorm (1e-6), res. LN (1e-5)     1024x4096               i.i.d. U[-1, 1]
3      RMSNorm, softmax                            131072 x {127,257,1537}  i.i.d. N(0, 1)
4      residual LN, RMSNorm, softmax               16384x8192              i.i.d. U[-1, 1]
5      softmax                                     8192x32768              stress (below)
=====  ==========================================  ======================  =========================

The stress distribution draws ``8 * N(0, 1) + off_i`` with one offset
``off_i ~ U[-80, 80]`` per row, then sets each entry to -inf with probability
0.01 (Bernoulli); a row that came out entirely -inf gets column 0 redrawn as
its finite value, so no row is all -inf.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass
from typing import Iterator

import numpy as np

SEED_ROOT = 20260905
OP_IDS = {"layernorm_residual": 0, "rmsnorm": 1, "softmax": 2, "layernorm": 3,
          "row_sum": 4, "row_minmax": 5, "layernorm_affine": 6}
TENSOR_IDS = {"x": 0, "r": 1, "gamma": 2, "beta": 3}
EPS = {"layernorm_residual": 1e-5, "layernorm": 1e-5, "layernorm_affine": 1e-5, "rmsnorm": 1e-6}

_BLOCK_ELEMS = 1 << 24  # float64 elements drawn per block (128 MiB)


@dataclass(frozen=True)
class Case:
    cfg: int
    op: str
    rows: int
    width: int
    dist: str

    @property
    def eps(self):
        return EPS.get(self.op)

    @property
    def inputs(self):
        return ("x", "r") if self.op == "layernorm_residual" else ("x",)

    @property
    def name(self):
        return f"cfg{self.cfg}-{self.op}-{self.rows}x{self.width}"


CORE_WORKLOADS = {
    1: [Case(1, "layernorm_residual", 17, 257, "uniform"),
        Case(1, "layernorm_residual", 1, 127, "uniform")],
    2: [Case(2, op, 1024, 4096, "uniform") for op in ("softmax", "rmsnorm", "layernorm_residual")],
    3: [Case(3, op, 131072, w, "normal") for w in (127, 257, 1537) for op in ("rmsnorm", "softmax")],
    4: [Case(4, op, 16384, 8192, "uniform") for op in ("layernorm_residual", "rmsnorm", "softmax")],
    5: [Case(5, "softmax", 8192, 32768, "stress")],
}


# Workloads of the next steps beyond the three core operators: plain
# LayerNorm at the shape the pages time it (1024x4096) and at the wide-row
# shape, affine LayerNorm (gamma ~ 1 + 0.1 N(0,1), beta ~ 0.1 N(0,1)), and
# the row sum / paired min-max reductions at a wide and a short ragged shape,
# rows beyond one workgroup's registers (1M, 128K, 256K and 4M columns) plus
# the pages' few-row shape 7x1537 through the workspace entry points, and
# many wide rows (64K and 128K columns) through the plain entry points and,
# at the same shapes, through the workspace entry points.
NEXT_WORKLOADS = {
    6: [Case(6, "layernorm", 1024, 4096, "uniform"), Case(6, "layernorm", 16384, 8192, "uniform")],
    7: [Case(7, "layernorm_affine", 1024, 4096, "uniform"), Case(7, "layernorm_affine", 16384, 8192, "uniform")],
    8: [Case(8, "row_sum", 16384, 8192, "uniform"), Case(8, "row_minmax", 16384, 8192, "uniform"),
        Case(8, "row_sum", 131072, 257, "normal"), Case(8, "row_minmax", 131072, 257, "normal")],
    9: [Case(9, "softmax", 64, 1 << 20, "normal"), Case(9, "rmsnorm", 1024, 1 << 17, "uniform"),
        Case(9, "layernorm_residual", 256, 1 << 18, "uniform"), Case(9, "row_sum", 16, 1 << 22, "uniform"),
        Case(9, "softmax", 7, 1537, "normal")],
    10: [Case(10, "softmax", 4096, 1 << 16, "normal"), Case(10, "rmsnorm", 2048, 1 << 17, "uniform"),
         Case(10, "layernorm_residual", 1024, 1 << 16, "uniform"), Case(10, "row_sum", 2048, 1 << 17, "uniform")],
    11: [Case(11, "softmax", 4096, 1 << 16, "normal"), Case(11, "rmsnorm", 2048, 1 << 17, "uniform"),
         Case(11, "layernorm_residual", 1024, 1 << 16, "uniform"), Case(11, "row_sum", 2048, 1 << 17, "uniform")],
}


def all_cases() -> Iterator[Case]:
    for cfg in sorted(CORE_WORKLOADS):
        yield from CORE_WORKLOADS[cfg]


def affine_vectors(case: Case):
    """(gamma, beta) for an affine LayerNorm case, float32 vectors of length width."""
    g = draw("normal", 1, case.width, seed_sequence(case.cfg, "layernorm", "gamma", 1, case.width))[0]
    b = draw("normal", 1, case.width, seed_sequence(case.cfg, "layernorm", "beta", 1, case.width))[0]
    return (np.float32(1.0) + np.float32(0.1) * g).astype(np.float32), (np.float32(0.1) * b).astype(np.float32)


def seed_sequence(cfg: int, op: str, tensor: str, rows: int, width: int) -> np.random.SeedSequence:
    return np.random.SeedSequence([SEED_ROOT, int(cfg), OP_IDS[op], TENSOR_IDS[tensor], int(rows), int(width)])


def draw(dist: str, rows: int, width: int, seed: np.random.SeedSequence) -> np.ndarray:
    """Draw a (rows, width) float32 matrix from ``dist`` with PCG64(seed)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((rows, width), dtype=np.float32)
    if rows == 0 or width == 0:
        return out
    blk = max(1, _BLOCK_ELEMS // max(1, width))
    for s in range(0, rows, blk):
        t = min(rows, s + blk)
        n = t - s
        if dist == "uniform":
            v = rng.uniform(-1.0, 1.0, size=(n, width))
        elif dist == "normal":
            v = rng.standard_normal(size=(n, width))
        elif dist == "stress":
            off = rng.uniform(-80.0, 80.0, size=(n, 1))
            v = 8.0 * rng.standard_normal(size=(n, width)) + off
            hole = rng.random(size=(n, width)) < 0.01
            v[hole] = -np.inf
            dead = hole.all(axis=1)
            if dead.any():
                v[dead, 0] = 8.0 * rng.standard_normal(size=int(dead.sum())) + off[dead, 0]
        else:
            raise ValueError(f"unknown distribution {dist!r}")
        out[s:t] = v.astype(np.float32)
    return out


def case_input(case: Case, tensor: str = "x") -> np.ndarray:
    return draw(case.dist, case.rows, case.width,
                seed_sequence(case.cfg, case.op, tensor, case.rows, case.width))


def random_matrix(seed: int, rows: int, width: int, dist: str = "uniform", tensor: str = "x") -> np.ndarray:
    """Ad-hoc test matrix: config id 0 with a caller-chosen seed folded in."""
    ss = np.random.SeedSequence([SEED_ROOT, 0, int(seed), TENSOR_IDS[tensor], int(rows), int(width)])
    return draw(dist, rows, width, ss)


def fingerprint(a: np.ndarray) -> str:
    """SHA-256 of the first and last MiB of an array's bytes (for run records)."""
    b = np.ascontiguousarray(a).view(np.uint8).reshape(-1)
    h = hashlib.sha256()
    h.update(b[: 1 << 20].tobytes())
    h.update(b[-(1 << 20):].tobytes())
    return h.hexdigest()
