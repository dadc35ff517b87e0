"""Write ``oracle_small.txt``: FP64 oracle outputs on a few tiny seeded rows.

Run from the repository root:  python tests/golden/make_oracle_small.py

It calls only ``oracle/`` (and the seeded generator in ``synthetic/``); the
file guards the oracle against unintended changes and gives the GPU smoke
check a fixed expectation.  Inputs and outputs are stored as float.hex so the
round trip is exact.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small.txt")

CASES = [
    # name, op, rows, width, dist, seed
    ("ln_res_3x5", "layernorm_residual", 3, 5, "uniform", 1),
    ("ln_res_2x9", "layernorm_residual", 2, 9, "uniform", 2),
    ("rms_3x7", "rmsnorm", 3, 7, "normal", 3),
    ("rms_1x13", "rmsnorm", 1, 13, "normal", 4),
    ("sm_3x6", "softmax", 3, 6, "normal", 5),
    ("sm_stress_2x11", "softmax", 2, 11, "stress", 6),
]


def case_arrays(op, rows, width, dist, seed):
    x = synthetic.random_matrix(1000 + seed, rows, width, dist)
    r = synthetic.random_matrix(2000 + seed, rows, width, dist, tensor="r") if op == "layernorm_residual" else None
    return x, r


def hexrow(a):
    return " ".join(float(v).hex() for v in np.asarray(a, dtype=np.float64).reshape(-1))


def main():
    lines = ["# FP64 oracle outputs on tiny seeded inputs; written by make_oracle_small.py (calls only oracle/).",
             "# case <name> <op> <rows> <width> <eps-or-none> ; then lines x:, r: (optional), y: as float.hex"]
    for name, op, rows, width, dist, seed in CASES:
        x, r = case_arrays(op, rows, width, dist, seed)
        eps = synthetic.EPS.get(op)
        y = oracle.run_op(op, x, r, eps=eps, threads=1)
        lines.append(f"case {name} {op} {rows} {width} {eps if eps is not None else 'none'}")
        lines.append("x: " + hexrow(x))
        if r is not None:
            lines.append("r: " + hexrow(r))
        lines.append("y: " + hexrow(y))
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
