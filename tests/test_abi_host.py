"""Host-side checks of the C ABI (no GPU, no device work).

* the library loads and exports every function ``include/rowred.h`` declares;
* the plan chooser's geometry covers every row and respects the limits;
* every argument error is reported before anything touches the GPU.

Pointers here are fake addresses: the checked paths never dereference them.
"""
import ctypes
import os
import re

import pytest

import row_wise_reduction_amd as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rowred.h")

CHUNKS = {1, 2, 3, 4, 5, 6, 7, 8, 10, 12, 16}


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rowred_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("rowred_layernorm_residual", "rowred_rmsnorm", "rowred_softmax", "rowred_plan_query",
              "rowred_run_plan", "rowred_status_string", "rowred_copy"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(R.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_library_exports_nothing_else():
    # -fvisibility=hidden: only the C ABI is visible.
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", R.LIB_PATH], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {n for n in exported if n.startswith("rowred_")} == set(declared_functions())


def test_status_strings():
    for s in range(5):
        assert R.rowred_status_string(s)
    assert R.rowred_status_string(99) == "unknown status"


X, RR, Y = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000  # 16-byte aligned, far apart


def window(x, rows, width):
    off0 = (x >> 2) & 3
    return max((width + ((off0 + i * width) & 3) + 3) // 4 for i in range(min(rows, 4)))


@pytest.mark.parametrize("op", ["layernorm_residual", "rmsnorm", "softmax"])
@pytest.mark.parametrize("width", [1, 2, 3, 4, 5, 7, 8, 31, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 1023,
                                   1024, 1025, 1537, 2048, 4095, 4096, 4097, 8191, 8192, 16384, 32764, 32765])
@pytest.mark.parametrize("mis", [0, 1, 2, 3])
def test_plan_covers_rows_and_respects_limits(op, width, mis):
    for rows in (1, 3, 17, 1024, 131072):
        x, y = X + 4 * mis, Y + 4 * mis
        r = RR + 4 * mis
        p = R.rowred_plan_query(op, x, r, y, rows=rows, width=width)
        L, T = p.lanes_per_row, p.threads
        if p.policy & R.ROWRED_POLICY_FLAT:
            # short rows off 16-byte boundaries (RMSNorm, softmax): rows_per_group
            # rows as one run of threads * chunks granules at any phase, and
            # lanes_per_row lanes fold each row
            assert op in ("rmsnorm", "softmax") and width >= 4 and p.policy & ~R.ROWRED_POLICY_FLAT == 3
            P = p.rows_per_group
            assert (T, p.chunks) in ((512, 2), (256, 4)) and P == min(T, (4 * T * p.chunks - 3) // width) >= 1
            assert P * width + 3 <= 4 * T * p.chunks
            assert L & (L - 1) == 0 and 1 <= L <= 64 and L * P <= T and (L == 64 or 2 * L * P > T)
            assert p.grid == -(-rows // P) and p.window == window(x, rows, width) and p.vector_io == 1
            continue
        assert L & (L - 1) == 0 and 1 <= L <= 1024
        assert T % 64 == 0 and 64 <= T <= 1024 and T % L == 0
        assert p.chunks in CHUNKS
        assert T <= (1024 if p.chunks <= 8 else 512)
        assert p.rows_per_group == T // L
        assert p.grid == -(-rows // p.rows_per_group)
        assert p.grid * p.rows_per_group >= rows
        assert p.vector_io == 1  # same alignment everywhere
        assert p.window == window(x, rows, width)
        assert L * p.chunks >= p.window
        # stripe within the private budget: <= 64 floats per lane
        assert 4 * p.chunks <= 64
        lds, on = R.ROWRED_POLICY_LDS_STRIPE, R.ROWRED_POLICY_ONLINE
        cap = (p.policy >> R.ROWRED_POLICY_CU_GROUPS_SHIFT) & 15
        assert 0 <= p.policy & ~(lds | on | R.ROWRED_POLICY_CU_GROUPS(15)) < 16 and p.reserved == 0
        if p.policy & lds:  # RMSNorm / softmax, 1024 lanes, 5-8 slots (RMSNorm up to 2048 x 8192 granules), 9-16 slots
            assert op in ("rmsnorm", "softmax") and L == T == 1024 and 5 <= p.chunks <= 16
            assert p.chunks > 8 or op == "softmax" or rows * p.window <= 2048 * 8192
            assert not p.policy & R.ROWRED_POLICY_STAGE_STORES
        if p.policy & on:  # softmax only, across 1024 lanes
            assert op == "softmax" and L == 1024
        if cap:  # large calls only, even caps; off 16-byte boundaries RMSNorm / softmax at 256 lanes
            assert rows * width * 4 > 64 << 20 and cap in (2, 6, 10)
            assert (mis == 0 and width % 4 == 0) or (op != "layernorm_residual" and L == T == 256 and cap == 6)


def test_plan_for_workload_shapes():
    # the shapes of the five workloads, aligned buffers
    nl, ns, rm = R.ROWRED_POLICY_NT_LOADS, R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_XCD_REMAP
    st = R.ROWRED_POLICY_STAGE_STORES
    # short ragged rows: flat plans (256 lanes x 4 granules for softmax;
    # lanes_per_row is the lanes that fold one row)
    fl = R.ROWRED_POLICY_FLAT
    lds, on = R.ROWRED_POLICY_LDS_STRIPE, R.ROWRED_POLICY_ONLINE
    cases = {(131072, 127): (8, 4, fl | nl | ns), (131072, 257): (16, 4, fl | nl | ns),
             (131072, 1537): (256, 2, nl | ns), (1024, 4096): (128, 8, nl | ns), (64, 4096): (256, 4, nl | ns),
             (16384, 8192): (256, 8, nl | ns | rm | R.ROWRED_POLICY_CU_GROUPS(2)),
             (8192, 32768): (1024, 8, nl | ns | rm | lds | on),
             (17, 257): (64, 2, nl), (7, 1537): (256, 2, nl), (512, 32768): (1024, 8, nl | ns | lds | on),
             (2048, 32768): (1024, 8, nl | ns | rm | lds | on),
             (1024, 50257): (1024, 13, nl | ns | lds | on),
             (4096, 65536): (1024, 16, nl | ns | rm | lds | on),
             (131072, 1024): (128, 2, nl | ns | rm | R.ROWRED_POLICY_CU_GROUPS(6)),
             (8192, 16384): (1024, 4, nl | ns | rm | on)}
    for (rows, width), (L, C, pol) in cases.items():
        p = R.rowred_plan_query("softmax", X, None, Y, rows=rows, width=width)
        assert (p.lanes_per_row, p.chunks, p.policy) == (L, C, pol), (rows, width, p)


def test_plan_memory_policy():
    nl, ns, rm = R.ROWRED_POLICY_NT_LOADS, R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_XCD_REMAP
    st = R.ROWRED_POLICY_STAGE_STORES
    # small, every row on a 16-byte boundary: streaming, no remap, no staging
    assert R.rowred_plan_query("rmsnorm", X, None, Y, rows=64, width=4096).policy == nl | ns
    # short rows share boundary lines: RMSNorm and softmax read them as one
    # run of granules (flat), streaming; LayerNorm stages its outputs in LDS,
    # with streaming stores and cached loads (each boundary granule is read twice)
    assert R.rowred_plan_query("rmsnorm", X, None, Y, rows=16384, width=127).policy == \
        R.ROWRED_POLICY_FLAT | nl | ns
    assert R.rowred_plan_query("layernorm_residual", X, RR, Y, rows=16384, width=127).policy == ns | st
    # longer ragged rows (> 256 granules): unstaged, streaming
    assert R.rowred_plan_query("rmsnorm", X + 4, None, Y + 4, rows=64, width=4096).policy == nl | ns
    assert R.rowred_plan_query("rmsnorm", X, None, Y, rows=2048, width=2049).policy == nl | ns
    # beyond 64 MiB: three slots per lane, at most 6 workgroups per CU at 256 lanes
    p = R.rowred_plan_query("rmsnorm", X, None, Y, rows=65536, width=2049)
    assert (p.lanes_per_row, p.chunks, p.threads, p.policy) == (256, 3, 256, nl | ns | R.ROWRED_POLICY_CU_GROUPS(6))
    p = R.rowred_plan_query("softmax", X, None, Y, rows=32768, width=4095)
    assert (p.lanes_per_row, p.chunks, p.threads, p.policy) == (512, 3, 512, nl | ns)
    # shared lines but y at another phase (no staging), > 2 slots per lane: cached stores
    assert R.rowred_plan_query("rmsnorm", X, None, Y + 4, rows=16384, width=127).policy == nl
    # large aligned matrix: streaming + remap, at most 2 workgroups per CU
    assert R.rowred_plan_query("rmsnorm", X, None, Y, rows=65536, width=4096).policy == \
        nl | ns | rm | R.ROWRED_POLICY_CU_GROUPS(2)


def test_plan_for_latency_bound_calls():
    """At most 2^19 elements in rows of at most 512 granules: 2 slots per
    lane, L the smallest power of two >= half the window, one wavefront per
    workgroup up to 2^16 elements (256 threads beyond), streaming loads,
    nothing staged.  Row reductions and affine LayerNorm keep their rules."""
    nl = R.ROWRED_POLICY_NT_LOADS
    for op, rows, width, want in (("softmax", 7, 1537, (256, 2, 256, nl)), ("softmax", 1, 127, (16, 2, 64, nl)),
                                  ("rmsnorm", 4096, 127, (32, 2, 256, nl)), ("softmax", 256, 2048, (256, 2, 256, nl)),
                                  ("layernorm_residual", 17, 257, (64, 2, 64, nl)),
                                  ("layernorm_residual", 1, 5, (8, 1, 64, nl)),
                                  ("rmsnorm", 1024, 512, (64, 2, 256, nl))):
        r = RR if op == "layernorm_residual" else None
        p = R.rowred_plan_query(op, X, r, Y, rows=rows, width=width)
        assert (p.lanes_per_row, p.chunks, p.threads, p.policy) == want, (op, rows, width, p)
    # affine LayerNorm: one slot per lane up to 256 granules, then two
    G, B = RR + (1 << 30), RR + (1 << 31)
    for rows, width, want in ((64, 257, (128, 1, 128)), (1024, 127, (64, 1, 256)), (7, 1537, (256, 2, 256))):
        p = R.rowred_layernorm_plan_query(X, None, G, B, Y, rows, width)
        assert (p.lanes_per_row, p.chunks, p.threads, p.policy) == (*want, nl), (rows, width, p)
    # row sum and min/max keep their geometry, in 256-thread workgroups
    p = R.rowred_plan_query("row_sum", X, None, Y, rows=1, width=4096)
    assert (p.lanes_per_row, p.chunks, p.threads) == (256, 4, 256)
    assert R.rowred_plan_query("row_sum", X, None, Y, rows=16384, width=8192).threads == 512
    # beyond either bound the general rules apply
    assert R.rowred_plan_query("softmax", X, None, Y, rows=4097, width=128).policy != nl
    assert R.rowred_plan_query("softmax", X, None, Y, rows=64, width=4096).lanes_per_row == 256
    assert R.rowred_plan_query("row_sum", X, None, Y, rows=7, width=1537).policy & R.ROWRED_POLICY_NT_LOADS


def test_plan_reports_4byte_io_on_mixed_alignment():
    p = R.rowred_plan_query("rmsnorm", X, None, Y + 4, rows=10, width=100)
    assert p.vector_io == 0 and p.window == 25
    p = R.rowred_plan_query("layernorm_residual", X, RR + 8, Y, rows=10, width=100)
    assert p.vector_io == 0
    p = R.rowred_plan_query("layernorm_residual", X + 4, RR + 4, Y + 4, rows=10, width=100)
    assert p.vector_io == 1 and p.window == 26


def test_pages_stripe_arithmetic():
    # At 4096 columns with 512 lanes of 4-element slots, one row needs
    # 2 slots per lane: an eight-float stripe per input, the RMSNorm figure in
    # "Immutable input reuse in Metal reductions" (section "What the
    # transformation actually preserves").  A 512-lane, 2-chunk plan is
    # accepted and its window is exactly covered.
    plan = R.Plan(lanes_per_row=512, rows_per_group=1, chunks=2, threads=512, grid=0)
    st = R.lib().rowred_run_plan(1, 0, 0, 0, 0, 4096, ctypes.c_float(1e-6), ctypes.byref(plan._c()), None)
    assert st == R.ROWRED_OK  # rows == 0: validated, nothing launched
    p = R.rowred_plan_query("rmsnorm", X, None, Y, rows=1024, width=4096)
    assert p.window == 4096 // 4 == 512 * 2


def raw(fn, *args):
    return getattr(R.lib(), fn)(*args)


def f(v):
    return ctypes.c_float(v)


def test_size_errors():
    assert raw("rowred_rmsnorm", X, Y, -1, 4, f(1e-6), None) == R.ROWRED_ERR_INVALID_ARG
    assert raw("rowred_rmsnorm", X, Y, 4, -1, f(1e-6), None) == R.ROWRED_ERR_INVALID_ARG
    # empty matrices: OK with nothing launched, even with NULL pointers
    assert raw("rowred_rmsnorm", None, None, 0, 4, f(1e-6), None) == R.ROWRED_OK
    assert raw("rowred_softmax", None, None, 7, 0, None) == R.ROWRED_OK
    assert raw("rowred_layernorm_residual", None, None, None, 0, 0, f(1e-5), None) == R.ROWRED_OK
    # rows wider than one register-resident pass: softmax and RMSNorm hold up
    # to 16384 granules in registers and LDS, wider rows (and LayerNorm) loop
    lp, lds = R.ROWRED_POLICY_LOOPED, R.ROWRED_POLICY_LDS_STRIPE
    for op, xx, yy, w, want in (("softmax", X, Y, 32769, lds), ("softmax", X + 4, Y + 4, 32768, lds),
                                ("rmsnorm", X, Y, 65536, lds), ("softmax", X + 4, Y + 4, 65536, lp | lds),
                                ("softmax", X, Y, 1 << 20, lp | lds)):
        p = R.rowred_plan_query(op, xx, None, yy, rows=4, width=w)
        assert p.policy & (lp | lds) == want, (op, w, p)
        assert p.lanes_per_row == p.threads == 1024 and p.grid == 4 and p.rows_per_group == 1
    # LayerNorm holds x and r of its first 8192 granules; row sum loops
    p = R.rowred_plan_query("layernorm_residual", X, None, Y, rows=4, width=32769)
    assert p.policy & (lp | lds) == lp | lds and p.chunks == 8
    p = R.rowred_plan_query("row_sum", X, None, Y, rows=4, width=65537)
    assert p.policy & lp and not p.policy & lds
    # widths beyond 32-bit element indices within a row
    assert raw("rowred_rmsnorm", X, Y, 1, 1 << 40, f(1e-6), None) == R.ROWRED_ERR_UNSUPPORTED


def test_max_width():
    """ROWRED_MAX_WIDTH leaves 2^20 elements of headroom below 2^31 for the
    kernels' 32-bit element and granule indices (a last tile or segment runs
    up to 16384 granules past the row); one more element is refused before
    anything launches, by every family of entry points."""
    M = R.ROWRED_MAX_WIDTH
    assert M == 2**31 - 2**20 - 1
    assert M + 3 + 4 * 16384 * 4 < 2**31
    for w, want in ((M + 1, R.ROWRED_ERR_UNSUPPORTED), (2**31 - 1, R.ROWRED_ERR_UNSUPPORTED)):
        assert raw("rowred_rmsnorm", X, Y, 1, w, f(1e-6), None) == want
        assert raw("rowred_softmax_ws", X, Y, 1, w, RR + (1 << 36), 1 << 30, None) == want
        assert raw("rowred_row_sum", X, Y, 1, w, None) == want
        assert raw("rowred_layernorm_residual", X, RR, Y, 1, w, f(1e-5), None) == want
    for op in ("softmax", "rmsnorm", "layernorm_residual", "row_sum"):
        p = R.rowred_plan_query(op, X, None, Y, rows=1, width=M)
        assert p.grid == 1 and p.policy & R.ROWRED_POLICY_LOOPED, (op, p)


def test_pointer_errors():
    assert raw("rowred_rmsnorm", None, Y, 4, 4, f(1e-6), None) == R.ROWRED_ERR_INVALID_ARG
    assert raw("rowred_rmsnorm", X, None, 4, 4, f(1e-6), None) == R.ROWRED_ERR_INVALID_ARG
    assert raw("rowred_layernorm_residual", X, None, Y, 4, 4, f(1e-5), None) == R.ROWRED_ERR_INVALID_ARG
    assert raw("rowred_softmax", X + 2, Y, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG  # not 4-byte aligned
    assert raw("rowred_softmax", X, Y + 1, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG


def test_eps_errors():
    for eps in (float("nan"), float("inf"), -1e-6):
        assert raw("rowred_rmsnorm", X, Y, 4, 4, f(eps), None) == R.ROWRED_ERR_INVALID_ARG
        assert raw("rowred_layernorm_residual", X, RR, Y, 4, 4, f(eps), None) == R.ROWRED_ERR_INVALID_ARG


def test_alias_errors():
    n = 16 * 64 * 4
    assert raw("rowred_softmax", X, X, 16, 64, None) == R.ROWRED_ERR_ALIAS
    assert raw("rowred_softmax", X, X + n - 4, 16, 64, None) == R.ROWRED_ERR_ALIAS
    assert raw("rowred_rmsnorm", X + n - 4, X, 16, 64, f(1e-6), None) == R.ROWRED_ERR_ALIAS
    assert raw("rowred_layernorm_residual", X, RR, RR + 64, 16, 64, f(1e-5), None) == R.ROWRED_ERR_ALIAS
    # x and r may overlap each other (both only read); checked before launch,
    # so use rows=0 to stop right after the argument checks.
    assert raw("rowred_layernorm_residual", X, X, Y, 0, 64, f(1e-5), None) == R.ROWRED_OK


def bad_plan(**kw):
    base = dict(lanes_per_row=64, rows_per_group=0, chunks=4, threads=256, grid=0, vector_io=0, window=0)
    base.update(kw)
    return R.Plan(**base)


@pytest.mark.parametrize("kw", [
    dict(lanes_per_row=48),           # not a power of two
    dict(lanes_per_row=2048, threads=1024),
    dict(threads=1056),               # over the 1024-thread workgroup limit
    dict(threads=96),                 # not a whole number of wavefronts
    dict(lanes_per_row=512, threads=256),   # row wider than the workgroup
    dict(chunks=9),                   # no kernel instantiated for 9 chunks
    dict(chunks=16, threads=1024, lanes_per_row=1024),  # 16 chunks compiled for <= 512 threads
    dict(chunks=1),                   # 64 lanes x 1 slot does not cover 1024 slots
    dict(policy=16),                  # unknown policy bit
    dict(policy=8, chunks=16, lanes_per_row=64, threads=256),  # staging compiled for <= 4 chunks only
    dict(policy=8, lanes_per_row=1024, chunks=1, threads=1024),  # staging needs <= 512 threads
    dict(reserved=1),
])
def test_run_plan_rejects_bad_plans(kw):
    c = bad_plan(**kw)._c()
    st = R.lib().rowred_run_plan(1, X, None, Y, 8, 4096, f(1e-6), ctypes.byref(c), None)
    assert st == R.ROWRED_ERR_INVALID_ARG, kw


def test_reload_policy_preconditions():
    m = R.ROWRED_POLICY_RELOAD
    lib = R.lib()
    # reload kernels exist for the matrix operators at <= 8 chunks
    c10 = bad_plan(lanes_per_row=64, chunks=10, threads=256, policy=m)._c()
    assert lib.rowred_run_plan(1, X, None, Y, 8, 2500, f(1e-6), ctypes.byref(c10), None) == R.ROWRED_ERR_INVALID_ARG
    # not for the scalar-output reductions, nor affine LayerNorm
    c2 = bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=m)._c()
    O1 = 0x7F4000000000
    assert lib.rowred_row_reduce_run_plan(3, X, O1, None, 8, 127, ctypes.byref(c2), None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm_run_plan(X, None, O1, None, Y, 8, 127, f(1e-5), ctypes.byref(c2), None) == \
        R.ROWRED_ERR_INVALID_ARG
    # LayerNorm at 7-8 chunks: at most 512 threads
    c8 = bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=m)._c()
    assert lib.rowred_run_plan(0, X, X, Y, 8, 32768, f(1e-5), ctypes.byref(c8), None) == R.ROWRED_ERR_INVALID_ARG
    # unknown policy bits stay rejected
    c32 = bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=32)._c()
    assert lib.rowred_run_plan(1, X, None, Y, 8, 127, f(1e-6), ctypes.byref(c32), None) == R.ROWRED_ERR_INVALID_ARG


def test_lds_stripe_preconditions():
    """ROWRED_POLICY_LDS_STRIPE: RMSNorm and softmax, 1024 lanes and threads,
    5-8 chunks, without staging or reloading."""
    m = R.ROWRED_POLICY_LDS_STRIPE
    lib = R.lib()
    ok = bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=m)._c()
    for op in (1, 2):  # zero rows: checked, nothing launched
        assert lib.rowred_run_plan(op, X, None, Y, 0, 32768, f(1e-6), ctypes.byref(ok), None) == R.ROWRED_OK
    wide = bad_plan(lanes_per_row=1024, chunks=16, threads=1024, policy=m)._c()  # 8 register + 8 LDS slots
    assert lib.rowred_run_plan(2, X, None, Y, 0, 65536, f(0), ctypes.byref(wide), None) == R.ROWRED_OK
    for kw in (dict(chunks=4, policy=m), dict(chunks=17, policy=m), dict(lanes_per_row=512, chunks=16, threads=512, policy=m),
               dict(lanes_per_row=512, threads=1024, chunks=16, policy=m),
               dict(policy=m | R.ROWRED_POLICY_RELOAD), dict(policy=m | R.ROWRED_POLICY_LOOPED),
               dict(policy=m | R.ROWRED_POLICY_STAGE_STORES)):
        base = dict(lanes_per_row=1024, chunks=8, threads=1024)
        base.update(kw)
        c = bad_plan(**base)._c()
        assert lib.rowred_run_plan(2, X, None, Y, 8, 32768, f(0), ctypes.byref(c), None) == R.ROWRED_ERR_INVALID_ARG, kw
    # LayerNorm (residual, plain, affine) and the row reductions have no LDS-stripe kernel
    assert lib.rowred_run_plan(0, X, X + (1 << 30), Y, 8, 32768, f(1e-5), ctypes.byref(ok), None) == \
        R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm_run_plan(X, None, None, None, Y, 8, 32768, f(1e-5), ctypes.byref(ok), None) == \
        R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_reduce_run_plan(3, X, 0x7F4000000000, None, 8, 32768, ctypes.byref(ok), None) == \
        R.ROWRED_ERR_INVALID_ARG


def test_head_tail_plan_preconditions():
    """ROWRED_POLICY_LDS_STRIPE | ROWRED_POLICY_LOOPED: 1024 lanes and threads;
    RMSNorm and softmax with 16 chunks (the held head), rows wider than 16384
    granules; LayerNorm with 8, rows wider than 8192."""
    m = R.ROWRED_POLICY_LDS_STRIPE | R.ROWRED_POLICY_LOOPED
    lib = R.lib()
    ok = bad_plan(lanes_per_row=1024, chunks=16, threads=1024, policy=m)._c()
    assert lib.rowred_run_plan(2, X, None, Y, 0, 100000, f(0), ctypes.byref(ok), None) == R.ROWRED_OK
    ln = bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=m)._c()  # LayerNorm: x and r of 8 slots
    assert lib.rowred_run_plan(0, X, X + (1 << 32), Y, 0, 40000, f(1e-5), ctypes.byref(ln), None) == R.ROWRED_OK
    # REVERSE orders the second walk (last tail tile first, head last)
    rev = bad_plan(lanes_per_row=1024, chunks=16, threads=1024, policy=m | R.ROWRED_POLICY_REVERSE)._c()
    assert lib.rowred_run_plan(1, X, None, Y, 0, 100000, f(1e-6), ctypes.byref(rev), None) == R.ROWRED_OK
    for op, width, kw in ((2, 65536, {}),                       # not wider than the head
                          (2, 100000, dict(chunks=8)), (2, 100000, dict(lanes_per_row=512, threads=512)),
                          (2, 100000, dict(policy=m | R.ROWRED_POLICY_STAGE_STORES)),
                          (0, 100000, {}),                      # LayerNorm takes 8 chunks
                          (0, 32768, dict(chunks=8))):          # LayerNorm row not wider than its head
        base = dict(lanes_per_row=1024, chunks=16, threads=1024, policy=m)
        base.update(kw)
        c = bad_plan(**base)._c()
        r = X + (1 << 32) if op == 0 else None
        assert lib.rowred_run_plan(op, X, r, Y, 4, width, f(1e-5), ctypes.byref(c), None) == \
            R.ROWRED_ERR_INVALID_ARG, (op, width, kw)


def test_row_exchange_plan_preconditions():
    """ROWRED_POLICY_EXCHANGE on a row plan: LayerNorm, RMSNorm and softmax
    rows in segments of threads * chunks granules (lanes_per_row == threads),
    only the memory bits and LDS_STRIPE beside it, the split plans' geometry
    limits, and the row's exchange words (2 S + 1 for LayerNorm, S + 1
    otherwise, 8 bytes each, from the row's first 16-byte boundary) ending
    inside segment 0's outputs and inside the row.  Valid plans pass the
    checks (on a host without a device the run then reports the missing
    residency, never an argument error)."""
    E, LDS = R.ROWRED_POLICY_EXCHANGE, R.ROWRED_POLICY_LDS_STRIPE
    lib = R.lib()

    def st(op, width, **kw):
        c = bad_plan(**kw)._c()
        if op == "affine":
            return lib.rowred_layernorm_run_plan(X, None, RR, None, Y, 8, width, f(1e-5), ctypes.byref(c), None)
        if op == "row_sum":
            return lib.rowred_row_reduce_run_plan(3, X, RR, None, 8, width, ctypes.byref(c), None)
        return lib.rowred_run_plan(op, X, RR if op == 0 else None, Y, 8, width, f(1e-5), ctypes.byref(c), None)

    g = dict(lanes_per_row=256, threads=256, chunks=8)
    for op, width, kw in ((1, 100000, dict(g, policy=E | 3)), (2, 1 << 20, dict(g, chunks=16, policy=E | 3 | LDS)),
                          (0, 65536, dict(g, policy=E | LDS)), ("affine", 65536, dict(g, policy=E | 3 | LDS)),
                          (0, 40000, dict(lanes_per_row=1024, threads=1024, chunks=4, policy=E)),
                          (1, 16377, dict(lanes_per_row=64, threads=64, chunks=1, policy=E))):  # 64 segments
        assert st(op, width, **kw) != R.ROWRED_ERR_INVALID_ARG, (op, width, kw)
    for op, width, kw in ((1, 100000, dict(g, lanes_per_row=128, policy=E)),       # lanes != threads
                          (1, 100000, dict(g, policy=E | R.ROWRED_POLICY_XCD_REMAP)),
                          (2, 100000, dict(g, policy=E | R.ROWRED_POLICY_ONLINE)),
                          (2, 100000, dict(g, policy=E | R.ROWRED_POLICY_LOOPED)),
                          (2, 100000, dict(g, chunks=4, policy=E | R.ROWRED_POLICY_STAGE_STORES)),
                          (2, 100000, dict(g, policy=E | R.ROWRED_POLICY_RELOAD)),
                          (2, 100000, dict(g, policy=E, reserved=1)),
                          ("row_sum", 100000, dict(g, policy=E)),                  # matrix operators only
                          (0, 100000, dict(g, policy=E)),                         # LayerNorm: 8 slots need LDS
                          (2, 4 * 1024 * 4 * 128 + 4, dict(lanes_per_row=1024, threads=1024, chunks=4,
                                                           policy=E)),            # 129 segments
                          (0, 16377, dict(lanes_per_row=64, threads=64, chunks=1, policy=E)),  # 129 words > 1012 B
                          (2, 5, dict(lanes_per_row=64, threads=64, chunks=1, policy=E))):     # row < its words
        assert st(op, width, **kw) == R.ROWRED_ERR_INVALID_ARG, (op, width, kw)


def test_stage_policy_preconditions():
    m = R.ROWRED_POLICY_STAGE_STORES
    ok = bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=m)._c()
    assert R.lib().rowred_run_plan(1, X, None, Y, 0, 127, f(1e-6), ctypes.byref(ok), None) == R.ROWRED_OK
    # y at another 16-byte phase than x
    assert R.lib().rowred_run_plan(1, X, None, Y + 4, 8, 127, f(1e-6), ctypes.byref(ok), None) == \
        R.ROWRED_ERR_INVALID_ARG
    # more than 512 threads
    big = bad_plan(lanes_per_row=32, chunks=2, threads=1024, policy=m)._c()
    assert R.lib().rowred_run_plan(1, X, None, Y, 8, 127, f(1e-6), ctypes.byref(big), None) == \
        R.ROWRED_ERR_INVALID_ARG


def test_run_plan_coverage_depends_on_x_alignment():
    # 4096 columns from a 16-byte aligned x span 1024 granules (64 x 16 covers
    # them); shifted by one float they span 1025, which 64 x 16 does not.
    c = bad_plan(lanes_per_row=64, chunks=16, threads=256)._c()
    assert R.lib().rowred_run_plan(1, X, None, Y, 0, 4096, f(1e-6), ctypes.byref(c), None) == R.ROWRED_OK
    assert R.lib().rowred_run_plan(1, X + 4, None, Y, 8, 4096, f(1e-6), ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG


def test_copy_argument_errors():
    assert raw("rowred_copy", X, Y, 6, None) == R.ROWRED_ERR_INVALID_ARG       # not a multiple of 4
    assert raw("rowred_copy", X + 4, Y, 8, None) == R.ROWRED_ERR_INVALID_ARG   # not 16-byte aligned
    assert raw("rowred_copy", X, X + 16, 64, None) == R.ROWRED_ERR_ALIAS
    assert raw("rowred_copy", None, None, 0, None) == R.ROWRED_OK


def test_python_binding_shape_checks():
    with pytest.raises(ValueError):
        R.rowred_softmax(X, Y)  # raw addresses need rows/width
    with pytest.raises(R.RowRedError) as e:
        R.rowred_softmax(X, X, rows=4, width=4)
    assert e.value.status == R.ROWRED_ERR_ALIAS


def test_xcd_block_remap_is_a_bijection():
    # Workgroup b runs on XCD b % 8 as that XCD's (b // 8)-th block; the
    # kernel maps it to row block x*q + min(x, rem) + i.  Every grid size must
    # give a permutation of [0, G) in which each XCD's blocks are contiguous.
    for G in list(range(1, 130)) + [4096, 4097, 32768, 131071]:
        q, rem = divmod(G, 8)
        seen = []
        per_xcd = {}
        for b in range(G):
            x, i = b % 8, b // 8
            blk = x * q + min(x, rem) + i
            seen.append(blk)
            per_xcd.setdefault(x, []).append(blk)
        assert sorted(seen) == list(range(G)), G
        for blks in per_xcd.values():
            assert blks == list(range(blks[0], blks[0] + len(blks)))


def test_layernorm_entry_argument_checks():
    lib = R.lib()
    G = 0x7F3000000000
    # plain LayerNorm: r may be NULL (rows = 0 stops after the checks)
    assert lib.rowred_layernorm(X, None, None, None, Y, 0, 64, f(1e-5), None) == R.ROWRED_OK
    assert lib.rowred_layernorm(X, None, G + 2, None, Y, 4, 64, f(1e-5), None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm(X, None, None, G + 1, Y, 4, 64, f(1e-5), None) == R.ROWRED_ERR_INVALID_ARG
    # gamma overlapping y
    assert lib.rowred_layernorm(X, None, Y + 64, None, Y, 4, 64, f(1e-5), None) == R.ROWRED_ERR_ALIAS
    assert lib.rowred_layernorm(X, None, None, Y + 4 * 255, Y, 4, 64, f(1e-5), None) == R.ROWRED_ERR_ALIAS
    assert lib.rowred_layernorm(X, None, None, None, Y, 4, 64, f(-1.0), None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm(X, None, None, None, Y, 0, 32768, f(1e-5), None) == R.ROWRED_OK
    # explicit plans: affine kernels of >= 7 chunks need <= 512 threads, 16 chunks do not exist
    c = bad_plan(lanes_per_row=1024, chunks=8, threads=1024)._c()
    assert lib.rowred_layernorm_run_plan(X, None, G, None, Y, 2, 24576, f(1e-5), ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG
    c = bad_plan(lanes_per_row=512, chunks=16, threads=512)._c()
    assert lib.rowred_layernorm_run_plan(X, None, G, None, Y, 2, 24576, f(1e-5), ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG
    c = bad_plan(lanes_per_row=512, chunks=12, threads=512)._c()
    assert lib.rowred_layernorm_run_plan(X, None, G, None, Y, 0, 24576, f(1e-5), ctypes.byref(c), None) == R.ROWRED_OK


def test_plan_query_layernorm_without_residual():
    p = R.rowred_plan_query("layernorm_residual", X, None, Y, rows=1024, width=4096)
    assert (p.lanes_per_row, p.chunks) == (128, 8)


def test_row_reduce_argument_checks():
    lib = R.lib()
    O1, O2 = 0x7F4000000000, 0x7F5000000000
    assert lib.rowred_row_sum(X, O1, 0, 64, None) == R.ROWRED_OK            # nothing to do
    assert lib.rowred_row_sum(X, O1, 4, 0, None) == R.ROWRED_ERR_INVALID_ARG  # rows need an element
    assert lib.rowred_row_sum(X, O1, -1, 4, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_sum(X, None, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_sum(X, O1 + 2, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_sum(X, X + 8, 4, 4, None) == R.ROWRED_ERR_ALIAS   # out inside x
    assert lib.rowred_row_minmax(X, O1, None, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_minmax(X, O1, O1 + 8, 4, 4, None) == R.ROWRED_ERR_ALIAS  # min and max overlap
    assert lib.rowred_row_minmax(X, O1, X, 4, 4, None) == R.ROWRED_ERR_ALIAS
    p = R.rowred_plan_query("row_sum", X, None, O1, rows=4, width=32769)
    assert p.policy & R.ROWRED_POLICY_LOOPED and p.grid == 4
    # staging does not apply to scalar outputs
    c = bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=R.ROWRED_POLICY_STAGE_STORES)._c()
    assert lib.rowred_row_reduce_run_plan(3, X, O1, None, 8, 127, ctypes.byref(c), None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_reduce_run_plan(1, X, O1, None, 8, 127, ctypes.byref(c), None) == R.ROWRED_ERR_INVALID_ARG
    p = R.rowred_plan_query("row_minmax", X, O2, O1, rows=1024, width=4096)
    assert p.lanes_per_row * p.chunks >= p.window and p.policy & R.ROWRED_POLICY_STAGE_STORES == 0


# ---------------------------------------------------------------------------
# any width / split rows
# ---------------------------------------------------------------------------

SPLIT_OPS = ["layernorm_residual", "rmsnorm", "softmax", "row_sum", "row_minmax"]


@pytest.mark.parametrize("op", SPLIT_OPS)
@pytest.mark.parametrize("rows,width", [(1, 1), (7, 1537), (3, 32769), (64, 1 << 20), (1024, 131072), (1, 100003),
                                        (16384, 8192), (5, 255)])
def test_workspace_size_covers_every_alignment(op, rows, width):
    need = R.rowred_workspace_size(op, rows, width)
    for mis in range(4):
        p = R.rowred_split_plan_query(op, X + 4 * mis, rows, width)
        G = p.threads * p.chunks
        assert p.window == window(X + 4 * mis, rows, width)
        assert p.segments == -(-p.window // G) and p.grid == rows * p.segments
        assert p.workspace_bytes == (p.grid + rows) * 16 <= need
        assert p.threads in (64, 128, 256, 512, 1024)
        if p.policy & R.ROWRED_POLICY_EXCHANGE:
            # LayerNorm, RMSNorm and softmax rows of at most 64 segments
            # (LayerNorm's 8 + 8 LDS-stripe segments: 128)
            assert op in ("layernorm_residual", "rmsnorm", "softmax")
            assert p.segments <= (128 if op == "layernorm_residual" and p.chunks == 16 else 64)
            if p.policy & R.ROWRED_POLICY_LDS_STRIPE:
                assert p.threads == 256 and p.chunks in ((8, 16) if op == "layernorm_residual" else (8, 12, 16))
            else:
                assert p.chunks in ((1, 2, 4) if op == "layernorm_residual" else (1, 2, 4, 8))
        else:
            assert p.chunks in (1, 2, 4)
            if op in ("layernorm_residual", "rmsnorm", "softmax"):
                # no exchange geometry fits
                assert p.window > (128 if op == "layernorm_residual" else 64) * 4096
        # the chooser never cuts a row into segments wider than the row, unless
        # the smallest one already is
        assert G <= max(p.window + 3, 64)


def test_workspace_size_empty_and_errors():
    assert R.rowred_workspace_size("softmax", 0, 100) == 0
    assert R.rowred_workspace_size("softmax", 100, 0) == 0
    n = ctypes.c_size_t()
    assert R.lib().rowred_workspace_size(7, 4, 4, ctypes.byref(n)) == R.ROWRED_ERR_INVALID_ARG
    assert R.lib().rowred_workspace_size(1, -1, 4, ctypes.byref(n)) == R.ROWRED_ERR_INVALID_ARG
    assert R.lib().rowred_workspace_size(1, 4, 4, None) == R.ROWRED_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(threads=96), dict(threads=32), dict(threads=2048), dict(chunks=3),
                                dict(chunks=8), dict(policy=R.ROWRED_POLICY_STAGE_STORES),
                                dict(policy=R.ROWRED_POLICY_XCD_REMAP)])
def test_split_plan_rejects(kw):
    base = dict(threads=256, chunks=2, policy=0)
    base.update(kw)
    with pytest.raises(R.RowRedError) as e:
        R.rowred_split_plan_query("softmax", X, 8, 100000, plan=R.SplitPlan(**base))
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG


@pytest.mark.parametrize("op,width,kw", [
    ("row_sum", 100000, {}), ("row_minmax", 100000, {}),                    # matrix operators only
    ("softmax", 100000, dict(policy=R.ROWRED_POLICY_EXCHANGE | R.ROWRED_POLICY_REVERSE)),
    ("softmax", 4 * 1024 * 4 * 128 + 4, dict(threads=1024, chunks=4)),       # S = 129 > 128
    ("rmsnorm", 4 * 64 * 2 * 70, dict(threads=64, chunks=2)),                # S = 70 > 64 threads
    ("rmsnorm", 100000, dict(policy=R.ROWRED_POLICY_XCD_REMAP)),              # no XCD remap
    ("softmax", 100000, dict(threads=1024, chunks=8)),                       # 8 slots: <= 512 threads
    ("layernorm_residual", 100000, dict(threads=256, chunks=8)),             # LayerNorm: <= 4 slots
])
def test_exchange_plan_rejects(op, width, kw):
    base = dict(threads=256, chunks=2, policy=0)
    base.update(kw)
    base["policy"] |= R.ROWRED_POLICY_EXCHANGE
    with pytest.raises(R.RowRedError) as e:
        R.rowred_split_plan_query(op, X, 8, width, plan=R.SplitPlan(**base))
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG


def test_lds_stripe_split_plans():
    """LDS-stripe exchange plans: 256 threads, 8, 12 or 16 slots (4 + 4,
    8 + 4, 8 + 8) for every matrix operator; only with EXCHANGE."""
    E, L = R.ROWRED_POLICY_EXCHANGE, R.ROWRED_POLICY_LDS_STRIPE
    for op, chunks in (("layernorm_residual", 8), ("layernorm_residual", 12), ("layernorm_residual", 16),
                       ("rmsnorm", 8), ("rmsnorm", 12), ("softmax", 16)):
        p = R.rowred_split_plan_query(op, X, 8, 100000, plan=R.SplitPlan(threads=256, chunks=chunks, policy=E | L))
        assert p.segments == -(-p.window // (256 * chunks))
    for op, kw in (("softmax", dict(threads=256, chunks=8, policy=L)),          # without EXCHANGE
                   ("softmax", dict(threads=512, chunks=8, policy=E | L)),      # 256 threads only
                   ("softmax", dict(threads=256, chunks=4, policy=E | L)),
                   ("layernorm_residual", dict(threads=256, chunks=10, policy=E | L)),
                   ("row_sum", dict(threads=256, chunks=8, policy=E | L))):
        with pytest.raises(R.RowRedError) as e:
            R.rowred_split_plan_query(op, X, 8, 100000, plan=R.SplitPlan(**kw))
        assert e.value.status == R.ROWRED_ERR_INVALID_ARG, (op, kw)


@pytest.mark.parametrize("op", ["layernorm_residual", "rmsnorm", "softmax"])
@pytest.mark.parametrize("T,C", [(64, 1), (256, 2), (1024, 4), (512, 8)])
def test_exchange_plan_limits(op, T, C):
    """The largest row an exchange plan takes: 128 segments, at most one per
    thread."""
    if C == 8 and op == "layernorm_residual":
        return
    S = min(128, T)
    width = 4 * T * C * S - 3  # worst phase: window = S * T * C granules
    plan = R.rowred_split_plan_query(op, X, 8, width, plan=R.SplitPlan(threads=T, chunks=C,
                                                                         policy=R.ROWRED_POLICY_EXCHANGE))
    assert plan.segments == S
    # the exchange words fit the workspace the three-kernel path needs
    assert (1 + 2 * 8 * S) * 8 <= plan.workspace_bytes


@pytest.mark.parametrize("op,rows,width,want", [
    ("softmax", 4096, 1 << 16, (256, 8, 8, 0)), ("rmsnorm", 2048, 1 << 17, (256, 8, 16, 0)),
    ("layernorm_residual", 1024, 1 << 16, (256, 8, 8, 1)), ("layernorm_residual", 256, 1 << 18, (256, 8, 32, 1)),
    # RMSNorm / softmax beyond 16 segments of 256 x 8: 8 + 8 LDS-stripe segments
    ("rmsnorm", 1024, 1 << 18, (256, 16, 16, 1)), ("rmsnorm", 64, 1 << 19, (256, 16, 32, 1)),
    ("rmsnorm", 64, 600000, (256, 16, 37, 1)), ("softmax", 64, 1 << 20, (256, 16, 64, 1)),
    ("softmax", 512, 1 << 17, (256, 8, 16, 0)),
    # LayerNorm beyond 32 segments of 4 + 4: 8 + 8 up to 128 segments
    ("layernorm_residual", 16, 1 << 20, (256, 16, 64, 1)), ("layernorm_residual", 16, 1 << 21, (256, 16, 128, 1)),
    ("layernorm_residual", 64, 1 << 18, (256, 8, 32, 1)), ("softmax", 7, 1537, (64, 2, 4, 0)),
    # no more (row, segment) workgroups than CUs: the segment is halved
    ("softmax", 16, 32768, (256, 4, 8, 0)), ("layernorm_residual", 8, 1 << 16, (256, 4, 16, 0)),
    ("softmax", 32, 1 << 16, (256, 4, 16, 0)), ("softmax", 33, 1 << 16, (256, 8, 8, 0)),
])
def test_ws_split_plan_choice(op, rows, width, want):
    """The _ws entry points' split plans: exchange geometries from the sweep
    (the last field: part of each segment in LDS); one phase off 16 bytes, a
    row of 2^20 floats spans 262145 granules, one more than 64 segments of
    4096 hold, and falls back to the three kernels."""
    p = R.rowred_split_plan_query(op, X, rows, width)
    T, C, S, lds = want
    assert (p.threads, p.chunks, p.segments) == (T, C, S)
    assert p.policy == R.ROWRED_POLICY_EXCHANGE | R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | \
        (R.ROWRED_POLICY_LDS_STRIPE if lds else 0)
    if width == 1 << 20 and op != "layernorm_residual":
        q = R.rowred_split_plan_query(op, X + 4, rows, width)
        assert not q.policy & R.ROWRED_POLICY_EXCHANGE and q.segments > 64


def test_ws_entry_argument_checks():
    lib = R.lib()
    W = 0x7F6000000000  # a workspace address far from the operands
    rows, width = 4, 40000  # beyond the register-resident window: needs the split kernels
    need = R.rowred_workspace_size("rmsnorm", rows, width)
    # nothing to do
    assert lib.rowred_rmsnorm_ws(X, Y, 0, width, f(1e-6), None, 0, None) == R.ROWRED_OK
    # no, misaligned or short workspace
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(1e-6), None, 0, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(1e-6), W + 8, need, None) == R.ROWRED_ERR_INVALID_ARG
    chosen = R.rowred_split_plan_query("rmsnorm", X, rows, width).workspace_bytes
    assert chosen <= need
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(1e-6), W, chosen - 16, None) == R.ROWRED_ERR_INVALID_ARG
    # workspace inside x, inside y
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(1e-6), X + 4096, need, None) == R.ROWRED_ERR_ALIAS
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(1e-6), Y, need, None) == R.ROWRED_ERR_ALIAS
    # y inside x, bad eps
    assert lib.rowred_rmsnorm_ws(X, X + 16, rows, width, f(1e-6), W, need, None) == R.ROWRED_ERR_ALIAS
    assert lib.rowred_rmsnorm_ws(X, Y, rows, width, f(-1.0), W, need, None) == R.ROWRED_ERR_INVALID_ARG
    # row sum needs an element per row; min/max needs both outputs
    O1, O2 = 0x7F4000000000, 0x7F5000000000
    assert lib.rowred_row_sum_ws(X, O1, rows, 0, W, need, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_minmax_ws(X, O1, None, rows, width, W, need, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_row_minmax_ws(X, O1, O2, rows, width, O2, need, None) == R.ROWRED_ERR_ALIAS
    # gamma/beta overlapping y
    assert lib.rowred_layernorm_ws(X, None, Y + 64, None, Y, rows, width, f(1e-5), W, need, None) == \
        R.ROWRED_ERR_ALIAS
    # residual / affine only with LayerNorm; y2 only with min/max
    p = R.SplitPlan(threads=256, chunks=2, policy=0)._c()
    assert lib.rowred_split_run_plan(1, X, RR, None, None, Y, None, rows, width, f(1e-6), ctypes.byref(p), W, need,
                                     None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_split_run_plan(2, X, None, RR, None, Y, None, rows, width, f(0), ctypes.byref(p), W, need,
                                     None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_split_run_plan(0, X, None, None, None, Y, O1, rows, width, f(1e-5), ctypes.byref(p), W, need,
                                     None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_split_run_plan(3, X, RR, None, None, O1, None, rows, width, f(0), ctypes.byref(p), W, need,
                                     None) == R.ROWRED_ERR_INVALID_ARG
    bad = R.SplitPlan(threads=256, chunks=3, policy=0)._c()
    assert lib.rowred_split_run_plan(1, X, None, None, None, Y, None, rows, width, f(1e-6), ctypes.byref(bad), W,
                                     need, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_split_run_plan(1, X, None, None, None, Y, None, rows, width, f(1e-6), None, W, need,
                                     None) == R.ROWRED_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(lanes_per_row=512, threads=1024), dict(lanes_per_row=1024, threads=1024, chunks=3),
                                dict(lanes_per_row=1024, threads=1024, chunks=8),
                                dict(lanes_per_row=96, threads=96, chunks=2),
                                dict(lanes_per_row=1024, threads=1024, chunks=2,
                                     policy=R.ROWRED_POLICY_LOOPED | R.ROWRED_POLICY_STAGE_STORES),
                                dict(lanes_per_row=1024, threads=1024, chunks=2,
                                     policy=R.ROWRED_POLICY_LOOPED | R.ROWRED_POLICY_REVERSE)])
def test_looped_plan_rejects(kw):
    base = dict(lanes_per_row=1024, rows_per_group=0, chunks=4, threads=1024, grid=0,
                policy=R.ROWRED_POLICY_LOOPED)
    base.update(kw)
    c = R.Plan(**base)._c()
    assert R.lib().rowred_run_plan(1, X, None, Y, 4, 100000, f(1e-6), ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG


def test_looped_layernorm_needs_two_chunks():
    c = R.Plan(lanes_per_row=1024, rows_per_group=0, chunks=4, threads=1024, grid=0,
               policy=R.ROWRED_POLICY_LOOPED)._c()
    assert R.lib().rowred_run_plan(0, X, RR, Y, 4, 100000, f(1e-5), ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG
    c2 = R.Plan(lanes_per_row=1024, rows_per_group=0, chunks=2, threads=1024, grid=0,
                policy=R.ROWRED_POLICY_LOOPED)._c()
    assert R.lib().rowred_run_plan(0, X, RR, Y, 0, 100000, f(1e-5), ctypes.byref(c2), None) == R.ROWRED_OK
    # the entry point holds x and r of the first 8192 granules instead
    p = R.rowred_plan_query("layernorm_residual", X, RR, Y, rows=4, width=100000)
    assert p.chunks == 8 and p.policy & R.ROWRED_POLICY_LOOPED and p.policy & R.ROWRED_POLICY_LDS_STRIPE



@pytest.mark.parametrize("rows,width,want", [
    ((16384, 8192, (256, 8, 256))), ((32768, 4096, (128, 8, 256))), ((65536, 2048, (128, 4, 256))),
    ((131072, 1024, (128, 2, 256))), ((1024, 4096, (256, 4, 256))), ((512, 8192, (512, 4, 512))),
    ((8192, 16384, (1024, 4, 1024))),
])
def test_layernorm_plan_query_affine(rows, width, want):
    """Affine LayerNorm's own geometry rule (256-thread workgroups, 4 slots,
    8 for rows of 1024-2048 granules beyond 32 MiB, 2 for rows of at most 256)
    on aligned rows; plain LayerNorm keeps the general rules; misaligned affine
    rows take 5 slots per lane beyond 32 MiB when gamma and beta sit on 16-byte
    boundaries, else plain LayerNorm's geometry (without its XCD remap)."""
    G, B = 0x7F4000000000, 0x7F5000000000
    p = R.rowred_layernorm_plan_query(X, None, G, B, Y, rows=rows, width=width)
    assert (p.lanes_per_row, p.chunks, p.threads) == want
    assert p.lanes_per_row * p.chunks >= p.window
    q = R.rowred_layernorm_plan_query(X, None, None, None, Y, rows=rows, width=width)
    assert q == R.rowred_plan_query("layernorm_residual", X, None, Y, rows=rows, width=width)
    n = R.rowred_layernorm_plan_query(X + 4, None, None, None, Y + 4, rows=rows, width=width - 1)
    for g, b in ((G, B), (G + 4, B + 4)):
        m = R.rowred_layernorm_plan_query(X + 4, None, g, b, Y + 4, rows=rows, width=width - 1)
        if rows * width * 4 > 32 << 20 and m.window <= 2560:
            L = 1
            while 5 * L < m.window:
                L *= 2
            assert (m.lanes_per_row, m.chunks, m.threads) == (L, -(-m.window // L), max(128 if L <= 64 else 256, L))
        else:
            assert (m.lanes_per_row, m.chunks, m.threads) == (n.lanes_per_row, n.chunks, n.threads)
        assert m.policy == n.policy & ~R.ROWRED_POLICY_XCD_REMAP


def test_layernorm_plan_query_errors():
    lib = R.lib()
    p = R._Plan()
    # gamma overlapping y; misaligned beta; no output
    assert lib.rowred_layernorm_plan_query(X, None, Y + 64, None, Y, 4, 4096, ctypes.byref(p)) == R.ROWRED_ERR_ALIAS
    assert lib.rowred_layernorm_plan_query(X, None, None, 0x7F5000000002, Y, 4, 4096, ctypes.byref(p)) == \
        R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm_plan_query(X, None, None, None, Y, 4, 4096, None) == R.ROWRED_ERR_INVALID_ARG
    assert lib.rowred_layernorm_plan_query(X, None, None, None, Y, 0, 4096, ctypes.byref(p)) == R.ROWRED_OK


def test_wide_row_remap_rule():
    """One workgroup per wide row: rows go over the XCDs in contiguous runs
    from 2048 rows that start on 16-byte boundaries (head+tail RMSNorm and
    softmax, looped row sum and min/max); LayerNorm's head+tail from 256 MiB
    per aligned input."""
    rem = R.ROWRED_POLICY_XCD_REMAP
    for op, rows, width, xx, want in (("rmsnorm", 2048, 131072, X, True), ("softmax", 4096, 65540, X, True),
                                      ("softmax", 1024, 131072, X, False), ("softmax", 512, 524288, X, False),
                                      ("rmsnorm", 2048, 131073, X, False), ("rmsnorm", 2048, 131072, X + 4, False),
                                      ("row_sum", 2048, 131072, X, True), ("row_minmax", 8192, 40000, X, True),
                                      ("row_sum", 512, 524288, X, False), ("row_sum", 4096, 65537, X, False),
                                      ("layernorm_residual", 1024, 65536, X, False),
                                      ("layernorm_residual", 2048, 40000, X, True)):
        r = RR if op in ("layernorm_residual", "row_minmax") else None
        p = R.rowred_plan_query(op, xx, r, Y, rows=rows, width=width)
        assert p.policy & R.ROWRED_POLICY_LOOPED, (op, rows, width, p)
        assert bool(p.policy & rem) == want, (op, rows, width, p)


@pytest.mark.parametrize("op", ["layernorm_residual", "rmsnorm", "softmax", "row_sum"])
def test_workspace_size_covers_every_chosen_plan(op):
    """rowred_workspace_size(op, rows, width) is enough for the plan a _ws
    call of that shape chooses at any 16-byte phase of x, including row
    counts on either side of the segment-halving rule."""
    for width in (32769, 40000, 65536, 98304, 100003, 262144, 1 << 20):
        for rows in (1, 7, 8, 16, 31, 32, 33, 63, 64, 65, 127, 255, 256):
            need = R.rowred_workspace_size(op, rows, width)
            for shift in (0, 4, 8, 12):
                p = R.rowred_split_plan_query(op, X + shift, rows, width)
                assert p.workspace_bytes <= need, (op, rows, width, shift, p, need)


def test_ragged_layernorm_rule():
    """LayerNorm on misaligned rows of more than 256 granules beyond 32 MiB:
    4 slots (5 beyond 1024 granules, 2 at 385-512), at most 512 lanes while
    that takes at most 8 slots, one row per workgroup, XCD remap (not
    affine).  Affine rows of up to 2560 granules: 5 slots per lane (128
    threads at 64 lanes).  RMSNorm rows of 513-3072 granules: 3 slots."""
    nl, ns, rm = R.ROWRED_POLICY_NT_LOADS, R.ROWRED_POLICY_NT_STORES, R.ROWRED_POLICY_XCD_REMAP
    G, B = RR + (1 << 30), RR + (1 << 31)
    shifted = {1023: (64, 5, 128), 1537: (128, 4, 256), 2047: (128, 5, 256), 4095: (256, 5, 256),
               8191: (512, 5, 512)}
    for width, want in ((1023, (128, 3, 256)), (1537, (256, 2, 256)), (2047, (256, 3, 256)), (4095, (256, 5, 256)),
                        (8191, (512, 5, 512)), (12287, (512, 7, 512)), (16383, (1024, 5, 1024))):
        rows = (1 << 27) // width
        for r in (None, RR):
            p = R.rowred_layernorm_plan_query(X, r, None, None, Y, rows, width)
            assert (p.lanes_per_row, p.chunks, p.threads, p.policy) == (*want, nl | ns | rm), (width, r, p)
        for g, b in ((G, B), (G + 4, B + 4)):
            a = R.rowred_layernorm_plan_query(X, None, g, b, Y, rows, width)
            assert (a.lanes_per_row, a.chunks, a.threads, a.policy) == (*shifted.get(width, want), nl | ns), (width, a)
    p = R.rowred_plan_query("rmsnorm", X, None, Y, rows=16386, width=8191)
    assert (p.lanes_per_row, p.chunks, p.threads) == (1024, 3, 1024)
    p = R.rowred_plan_query("rmsnorm", X, None, Y, rows=65536, width=2047)
    assert (p.lanes_per_row, p.chunks, p.threads) == (256, 3, 256)


def undefined_symbols():
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", R.LIB_PATH], capture_output=True, text=True).stdout
    return {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}


def test_library_reads_no_environment():
    """No entry point reads the environment (getenv racing a setenv on
    another thread is undefined behaviour, and the library is documented as
    safe to call from several threads)."""
    und = undefined_symbols()
    assert not {"getenv", "secure_getenv", "__secure_getenv"} & und


def test_library_never_allocates_device_memory():
    """The caller owns every buffer: the library references no HIP allocator."""
    und = undefined_symbols()
    alloc = {n for n in und if re.match(r"hip(Ext)?(Malloc|Free|MallocAsync|FreeAsync|HostMalloc|HostFree|"
                                        r"MallocManaged|MallocPitch|Malloc3D|MallocArray|MemPool)", n)}
    assert not alloc, alloc


@pytest.mark.parametrize("kw", [dict(wait_polls=-1), dict(reserved=1)])
def test_split_plan_rejects_bad_wait_fields(kw):
    base = dict(threads=256, chunks=8, policy=R.ROWRED_POLICY_EXCHANGE)
    base.update(kw)
    with pytest.raises(R.RowRedError) as e:
        R.rowred_split_plan_query("softmax", X, 8, 100000, plan=R.SplitPlan(**base))
    assert e.value.status == R.ROWRED_ERR_INVALID_ARG
    ok = R.rowred_split_plan_query("softmax", X, 8, 100000, plan=R.SplitPlan(threads=256, chunks=8,
                                                                               policy=R.ROWRED_POLICY_EXCHANGE,
                                                                               wait_polls=5))
    assert ok.wait_polls == 5 and ok.segments == 13


def test_online_policy_preconditions():
    """ROWRED_POLICY_ONLINE: softmax only, on the register kernels (not
    RELOAD) or LDS_STRIPE at 5-16 chunks; not with LOOPED or FLAT plans."""
    on = R.ROWRED_POLICY_ONLINE
    lds, lp, fl = R.ROWRED_POLICY_LDS_STRIPE, R.ROWRED_POLICY_LOOPED, R.ROWRED_POLICY_FLAT
    lib = R.lib()

    def st(op, plan, width, rows=8):  # the plan is checked before any device call
        return lib.rowred_run_plan(op, X, None, Y, rows, width, f(0), ctypes.byref(plan._c()), None)

    # accepted plans get past the checks (here the launch then fails: no GPU)
    for plan, width in ((bad_plan(lanes_per_row=256, policy=on | 3), 4096),
                        (bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=on | lds), 32768),
                        (bad_plan(lanes_per_row=1024, chunks=16, threads=1024, policy=on | lds), 65536),
                        (bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=on | 7), 32768),
                        (bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=on | 11), 127)):
        assert st(2, plan, width) != R.ROWRED_ERR_INVALID_ARG, plan
    for plan in (bad_plan(policy=on), bad_plan(lanes_per_row=256, policy=on | 3)):
        assert st(2, plan, 4096, rows=0) == R.ROWRED_OK  # zero rows: nothing to check or launch
    for op, plan, width in ((1, bad_plan(lanes_per_row=256, policy=on), 4096),  # RMSNorm
                            (0, bad_plan(lanes_per_row=256, policy=on), 4096),  # LayerNorm
                            (2, bad_plan(lanes_per_row=256, policy=on | R.ROWRED_POLICY_RELOAD), 4096),
                            (1, bad_plan(lanes_per_row=1024, chunks=8, threads=1024, policy=on | lds), 32768),
                            (2, bad_plan(lanes_per_row=1024, chunks=4, threads=1024, policy=on | lp), 65536),
                            (2, bad_plan(lanes_per_row=1024, chunks=16, threads=1024, policy=on | lp | lds), 131072),
                            (2, bad_plan(lanes_per_row=0, chunks=4, threads=256, policy=on | fl), 127)):
        assert st(op, plan, width) == R.ROWRED_ERR_INVALID_ARG, (op, plan)
    # not for the scalar-output reductions
    c = bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=on)._c()
    assert lib.rowred_row_reduce_run_plan(3, X, 0x7F4000000000, None, 8, 127, ctypes.byref(c), None) == \
        R.ROWRED_ERR_INVALID_ARG


def test_cu_groups_field():
    """Bits 12-15 of a row plan's policy: a cap of 1-14 workgroups per CU on
    the register kernels; 15 rejected, as is a cap on FLAT, LOOPED or
    LDS_STRIPE plans."""
    lib = R.lib()
    cap = R.ROWRED_POLICY_CU_GROUPS
    assert cap(5) == 5 << 12

    def st(op, plan, width, rows=8):
        return lib.rowred_run_plan(op, X, None, Y, rows, width, f(1e-6), ctypes.byref(plan._c()), None)

    for n in range(1, 15):
        for pol in (3, 3 | R.ROWRED_POLICY_STAGE_STORES):
            assert st(1, bad_plan(lanes_per_row=32, chunks=2, threads=256, policy=pol | cap(n)), 250) != \
                R.ROWRED_ERR_INVALID_ARG, n
    assert st(1, bad_plan(lanes_per_row=256, policy=3 | cap(15)), 4096) == R.ROWRED_ERR_INVALID_ARG
    for plan, width in ((bad_plan(lanes_per_row=1024, chunks=8, threads=1024,
                                  policy=R.ROWRED_POLICY_LDS_STRIPE | cap(2)), 32768),
                        (bad_plan(lanes_per_row=1024, chunks=4, threads=1024, policy=R.ROWRED_POLICY_LOOPED | cap(4)),
                         65536),
                        (bad_plan(lanes_per_row=0, chunks=4, threads=256, policy=R.ROWRED_POLICY_FLAT | cap(4)), 127)):
        assert st(1, plan, width) == R.ROWRED_ERR_INVALID_ARG, plan


def test_binding_constants_match_header():
    """Every ROWRED_POLICY_* / ROWRED_OP_* / ROWRED_ERR_* value the header
    defines has the same value in the binding."""
    import re
    text = open(HEADER).read()
    pairs = re.findall(r"\b(ROWRED_(?:POLICY|OP|ERR)_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)
    pairs += re.findall(r"#define\s+(ROWRED_POLICY_CU_GROUPS_SHIFT)\s+(\d+)", text)
    assert len(pairs) >= 20
    for name, value in pairs:
        assert getattr(R, name) == int(value), name
