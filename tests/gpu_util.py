"""Helpers shared by the GPU tests: device upload, guarded outputs, comparison
with the oracle at atol = rtol = 1e-5 (|y - ref| <= 1e-5 + 1e-5 |ref|, NaN
only where the oracle has NaN)."""
import numpy as np

import oracle

ATOL = 1e-5
RTOL = 1e-5
GUARD = 64  # sentinel floats before and after each output
SENTINEL_BITS = np.uint32(0x7FC0DEAD)  # a quiet NaN no kernel produces


def torch():
    import torch as t
    return t


def dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


class Guarded:
    """A device output of shape (rows, width) at `shift` floats past a 256-byte
    aligned base, with GUARD sentinel floats on each side."""

    def __init__(self, rows, width, shift=0):
        t = torch()
        self.n = rows * width
        self.shift = shift
        self.buf = t.empty(GUARD + shift + self.n + GUARD, dtype=t.int32, device="cuda")
        self.buf.fill_(int(SENTINEL_BITS.view(np.int32)))
        self.y = self.buf[GUARD + shift: GUARD + shift + self.n].view(t.float32).view(rows, width)

    def guards_intact(self):
        b = self.buf.cpu().numpy().view(np.uint32)
        head = b[: GUARD + self.shift]
        tail = b[GUARD + self.shift + self.n:]
        return bool((head == SENTINEL_BITS).all() and (tail == SENTINEL_BITS).all())

    def host(self):
        return self.y.cpu().numpy()


def shifted_input(a, shift):
    """Upload `a` so that its first element sits `shift` floats past a 256-byte
    aligned allocation (shift 0..3 sets the address modulo 16)."""
    t = torch()
    flat = t.empty(a.size + shift + 4, dtype=t.float32, device="cuda")
    v = flat[shift: shift + a.size].view(a.shape)
    v.copy_(t.from_numpy(np.ascontiguousarray(a)))
    return v


def assert_close(y, ref, what=""):
    ok, excess, idx = oracle.within_tolerance(y, ref, ATOL, RTOL)
    if not ok:
        yv = float(np.asarray(y)[idx]) if idx is not None else None
        rv = float(np.asarray(ref)[idx]) if idx is not None else None
        raise AssertionError(f"{what}: mismatch at {idx}: gpu={yv!r} oracle={rv!r} (excess {excess:.3g})")


def print_case(*parts):
    print("CASE", *parts, flush=True)


def all_plans(window):
    """Every explicit plan (lanes, chunks, threads, policy) that covers a row
    window of `window` granules without a wholly idle lane group."""
    import row_wise_reduction_amd as R
    chunks_set = (1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16)
    for L in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        for C in chunks_set:
            if L * C < window or (L > 1 and L * C >= 2 * window + 4 * L):
                continue
            for T in sorted({max(64, L), 256, 1024 if C <= 8 else 512}):
                if T < L or T % L or T > (1024 if C <= 8 else 512):
                    continue
                for policy in (0, 3, 4, 7, 8, 11, 15):
                    if policy & R.ROWRED_POLICY_STAGE_STORES and (C > 4 or T > 512):
                        continue
                    yield R.Plan(lanes_per_row=L, rows_per_group=0, chunks=C, threads=T, grid=0, policy=policy)
