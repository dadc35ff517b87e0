"""Checks on the gfx950 assembly of our own kernels (built here, no GPU).

* no private (scratch) segment and no register spills: the row stripes stay
  in VGPRs, so no hidden memory traffic;
* VGPR counts fit the workgroup sizes the kernels are launched with;
* 16-byte loads and stores are used; no MFMA (nothing here is a contraction);
* the non-temporal load policy selects its own copy of the row loads;
* no packed-FP32 VALU instructions;
* barriers only where cross-wave partials are folded or outputs are
  staged in LDS.
"""
import os
import re
import subprocess

import pytest

from row_wise_reduction_amd import build as B


@pytest.fixture(scope="module")
def asm():
    path = B.device_asm()
    return open(path).read()


def kernel_meta(asm):
    out = {}
    for m in re.finditer(r"\n  - \.agpr_count:\s+(\d+)(.*?)(?=\n  - \.agpr_count|\n\s*\.end_amdgpu_metadata)", asm, re.S):
        body = m.group(2)

        def g(k):
            mm = re.search(r"\." + k + r":\s+(\S+)", body)
            return mm.group(1) if mm else None

        name = g("name")
        out[name] = dict(agpr=int(m.group(1)), vgpr=int(g("vgpr_count")), sgpr=int(g("sgpr_count")),
                         private=int(g("private_segment_fixed_size")), vspill=int(g("vgpr_spill_count")),
                         sspill=int(g("sgpr_spill_count")), lds=int(g("group_segment_fixed_size")),
                         max_flat=int(g("max_flat_workgroup_size")))
    return out


def kernel_body(asm, name):
    m = re.search(r"\n" + re.escape(name) + r":(.*?)\n\s*s_endpgm", asm, re.S)
    assert m, name
    return m.group(1)


def kernel_function(asm, name):
    """The whole function (every exit), up to its end label."""
    m = re.search(r"\n" + re.escape(name) + r":(.*?)\.Lfunc_end", asm, re.S)
    assert m, name
    return m.group(1)


def demangle(n):
    return subprocess.run(["c++filt", n], capture_output=True, text=True).stdout.strip()


def test_every_kernel_is_spill_free(asm):
    meta = kernel_meta(asm)
    # five operators, affine LayerNorm (no 16-chunk kernel), the reload
    # variant of the three matrix operators at 1-8 chunks, copy; split rows:
    # statistics (5 operators x 3 chunk counts), apply (3 x 3), merge (5)
    # ... and the looped kernels (5 operators x 2 chunk counts, LayerNorm at 2 only),
    # the exchange kernels (3 operators x 4 chunk counts, LayerNorm not at 8)
    # and their two clear kernels (workspace words, words in y's rows), the LDS-stripe kernels (2 operators x 12 stripes,
    # and 5 with a walked tail: RMSNorm, softmax, LayerNorm plain and with
    # gamma/beta read 4 or 16 bytes at a time), the LDS-stripe exchange kernels (LayerNorm,
    # RMSNorm and softmax 3 each), the flat kernels (RMSNorm and softmax at
    # 1, 2, 4 chunks) and the affine LayerNorm kernels for rows off 16-byte
    # boundaries with 16-byte gamma/beta loads (10 chunk counts)
    assert len(meta) == 5 * 11 + 10 + 3 * 8 + 1 + 15 + 9 + 5 + 9 + 11 + 2 + 24 + 5 + 9 + 2 * 3 + 10
    for name, m in meta.items():
        # No scratch memory at all.  The 10/12/16-chunk kernels (reachable only
        # through an explicit plan) may park SGPRs in VGPR lanes.
        assert m["private"] == 0 and m["vspill"] == 0, (demangle(name), m)
        dn = demangle(name)
        wide = any(f", {c}>" in dn or f"<{c}>" in dn for c in (10, 12, 16))  # never picked by the chooser
        # LayerNorm exchange segments with 8 register slots of x and of r
        # (12 and 16 chunks), and the 8-slot RMSNorm / softmax exchange
        # kernels (with the count of words kept in y's rows), park a few SGPRs
        # in VGPR lanes as well: no memory.
        wide = wide or "seg_xlds_kernel<0, 8," in dn or "seg_exchange_kernel<1, 8>" in dn or \
            "seg_exchange_kernel<2, 8>" in dn
        if not wide:
            assert m["sspill"] == 0, (dn, m)


def test_vgprs_fit_launch_bounds(asm):
    for name, m in kernel_meta(asm).items():
        # 512 VGPRs per SIMD lane; a workgroup of max_flat threads puts
        # max_flat/256 waves on each SIMD.
        waves_per_simd = max(1, m["max_flat"] // 256)
        assert m["vgpr"] + m["agpr"] <= 512 // waves_per_simd, (demangle(name), m)


def test_row_kernels_use_16_byte_access_and_no_mfma(asm):
    assert "v_mfma" not in asm
    for name in kernel_meta(asm):
        if "rows_kernel" not in name:
            continue
        dn = demangle(name)
        body = kernel_body(asm, name)
        assert "global_load_dwordx4" in body, dn
        if not any(f"rows_kernel<{op}," in dn for op in (3, 4)):  # row sum / min-max store one float per row
            assert "global_store_dwordx4" in body, dn


def test_no_packed_fp32(asm):
    assert not re.search(r"v_pk_(add|mul|fma)_f32", asm)


def test_loads_are_issued_before_the_first_wait(asm):
    # RMSNorm, 5 chunks, 16-byte path: all five loads precede the first vmcnt wait.
    name = [n for n in kernel_meta(asm) if demangle(n).startswith("void rowred::(anonymous namespace)::rows_kernel<1, 5>")][0]
    body = kernel_body(asm, name)
    first_wait = body.find("s_waitcnt vmcnt")
    assert body[:first_wait].count("global_load_dwordx4") == 5


def x4_loads(body):
    """(non-temporal, cached) 16-byte global loads of a kernel body."""
    lines = [ln.strip() for ln in body.splitlines() if "global_load_dwordx4" in ln]
    nt = sum(1 for ln in lines if ln.endswith(" nt"))
    return nt, len(lines) - nt


def test_nt_load_policy_reaches_the_row_loads(asm):
    # Every row load exists twice, once with the non-temporal hint and once
    # without, selected by ROWRED_POLICY_NT_LOADS (affine LayerNorm adds its
    # cached gamma/beta loads).
    for name in kernel_meta(asm):
        dn = demangle(name)
        kind = "rows_kernel<" if "rows_kernel<" in dn else "reload_kernel<" if "reload_kernel<" in dn else None
        if not kind:
            continue
        op = int(dn.split(kind)[1].split(",")[0])
        chunks = int(dn.split(kind)[1].split(",")[1].split(">")[0])
        nt, cached = x4_loads(kernel_body(asm, name))
        assert nt > 0, dn
        extra = 2 * chunks if op == 5 else 0
        assert cached == nt + extra, (dn, nt, cached)


def test_reload_kernels_read_the_row_once_per_phase(asm):
    # With x 16-byte phase-aligned to y, RMSNorm reads the row twice,
    # softmax and LayerNorm three times (LayerNorm also reads r each time,
    # 16 bytes or 4 bytes at a time depending on its alignment).  Counted
    # in the non-temporal copy of the loads.
    for name in kernel_meta(asm):
        dn = demangle(name)
        if "reload_kernel<" not in dn:
            continue
        op = int(dn.split("reload_kernel<")[1].split(",")[0])
        chunks = int(dn.split("reload_kernel<")[1].split(",")[1].split(">")[0])
        phases = {0: 3, 1: 2, 2: 3}[op]
        nt, _ = x4_loads(kernel_body(asm, name))
        # x in every phase; LayerNorm adds r's 16-byte loads
        want = phases * chunks * (2 if op == 0 else 1)
        assert nt == want, (dn, nt, want)
        # the resident kernel of the same shape reads each granule once
        resident = name.replace("13reload_kernel", "11rows_kernel")  # mangled: length-prefixed names
        assert x4_loads(kernel_body(asm, resident))[0] == chunks * (2 if op == 0 else 1), dn


def test_barriers_only_where_partials_are_folded(asm):
    copy = [n for n in kernel_meta(asm) if "copy_kernel" in n][0]
    assert "s_barrier" not in kernel_body(asm, copy)
    for name in kernel_meta(asm):
        dn = demangle(name)
        kind = "rows_kernel<" if "rows_kernel<" in dn else "reload_kernel<" if "reload_kernel<" in dn else None
        if kind:
            # RMSNorm, row sum and paired min/max (one shared exchange) fold
            # once, softmax and LayerNorm twice; softmax row kernels also
            # carry the one-collective (ROWRED_POLICY_ONLINE) path, one more
            # fold; matrix-output kernels of at most 4 chunks add one for the
            # staged stores.  Reloading adds none.
            n = kernel_body(asm, name).count("s_barrier")
            op = int(dn.split(kind)[1].split(",")[0])
            chunks = int(dn.split(kind)[1].split(",")[1].split(">")[0])
            folds = {0: 2, 1: 1, 2: 2 if kind == "reload_kernel<" else 3, 3: 1, 4: 1, 5: 2}[op]
            staged = chunks <= 4 and op not in (3, 4)
            want = folds + (1 if staged else 0)
            assert n == want, (dn, n)


def test_split_kernels(asm):
    """Statistics kernels read with cached loads (the apply kernel reads the
    segment again and should find it in cache); apply kernels carry a
    non-temporal and a cached copy of their segment loads and no barrier; merge
    kernels work per wavefront, without barriers; statistics kernels fold
    across waves once per reduction (LayerNorm and softmax twice)."""
    seen = {"seg_stats_kernel": 0, "seg_apply_kernel": 0, "seg_merge_kernel": 0}
    for name in kernel_meta(asm):
        dn = demangle(name)
        kind = next((k for k in seen if k + "<" in dn), None)
        if not kind:
            continue
        seen[kind] += 1
        body = kernel_body(asm, name)
        nt, cached = x4_loads(body)
        op = int(dn.split(kind + "<")[1].split(",")[0].split(">")[0])
        if kind == "seg_stats_kernel":
            assert nt == 0 and cached > 0, dn
            assert body.count("s_barrier") == {0: 2, 1: 1, 2: 2, 3: 1, 4: 1}[op], dn
        elif kind == "seg_apply_kernel":
            # plus at most one cached 16-byte load (the row record), and for
            # LayerNorm one each of gamma and beta per slot
            C = int(dn.split(kind + "<")[1].split(",")[1].split(">")[0])
            extra = (0, 1, 2 * C, 2 * C + 1) if op == 0 else (0, 1)
            assert nt > 0 and cached - nt in extra, (dn, nt, cached)
            assert "s_barrier" not in body, dn
            assert "global_store_dwordx4" in body, dn
        else:
            assert "s_barrier" not in body and "global_load_dword" in body, dn
    assert seen == {"seg_stats_kernel": 15, "seg_apply_kernel": 9, "seg_merge_kernel": 5}


def test_looped_kernels(asm):
    """Looped kernels: no scratch; the statistics walk uses cached loads and
    the second walk (matrix outputs) has a non-temporal copy; one collective
    per statistic (LayerNorm and softmax two), no barrier in the loops."""
    seen = 0
    for name in kernel_meta(asm):
        dn = demangle(name)
        if "looped_kernel<" not in dn:
            continue
        seen += 1
        body = kernel_body(asm, name)
        op = int(dn.split("looped_kernel<")[1].split(",")[0])
        nt, cached = x4_loads(body)
        if op in (3, 4):
            assert nt == 0 and cached > 0, dn
        else:
            assert nt > 0 and cached > nt, (dn, nt, cached)
        assert body.count("s_barrier") == {0: 2, 1: 1, 2: 2, 3: 1, 4: 1}[op], dn
    assert seen == 9



def test_exchange_kernels(asm):
    """Exchange kernels: a non-temporal and a cached copy of the segment
    loads; the statistics leave and arrive through 8-byte agent-scope (sc1)
    stores and loads, with a sleep in the wait; no cache write-back or
    invalidate instruction (value and flag share one word, so relaxed atomics
    suffice); one cross-wave fold per reduction."""
    seen = 0
    for name in kernel_meta(asm):
        dn = demangle(name)
        if "seg_exchange_kernel<" not in dn:
            continue
        seen += 1
        body = kernel_body(asm, name)
        op = int(dn.split("seg_exchange_kernel<")[1].split(",")[0])
        nt, cached = x4_loads(body)
        assert nt > 0 and cached >= nt, (dn, nt, cached)
        lines = [ln.strip() for ln in body.splitlines()]
        assert any(ln.startswith("global_store_dwordx2") and ln.endswith("sc1") for ln in lines), dn
        assert any(ln.startswith("global_load_dwordx2") and ln.endswith("sc1") for ln in lines), dn
        assert "s_sleep" in body and "buffer_wbl2" not in body and "buffer_inv" not in body, dn
        # RMSNorm: segment sum + exchanged sum; softmax: max, sum, exchanged max
        # and sum; LayerNorm: sum, squares, exchanged sum and squares; RMSNorm
        # and softmax also segment 0's wait before it writes over words kept in
        # y's row (LayerNorm's row-completing workgroup stores those instead)
        nb = kernel_function(asm, name).count("s_barrier")
        assert nb == {0: 4, 1: 3, 2: 5}[op], (dn, nb)
    assert seen == 11


def test_lds_stripe_kernels(asm):
    """LDS-stripe kernels: 1..8 slots per lane loaded straight into LDS with
    16-byte LDS-writing loads (a non-temporal and a cached copy), 4 or 8
    register slots (16-byte loads, both copies), a full wait before the first
    LDS read, LDS sized for the slots, and registers for two 1024-thread
    workgroups per CU (at most 64 VGPRs) where 4 slots are in registers (the
    8-register-slot kernels take over 80 KiB of LDS: one workgroup per CU,
    up to 128 VGPRs)."""
    meta = kernel_meta(asm)
    seen = 0
    for name, m in meta.items():
        dn = demangle(name)
        if "wide_kernel<" not in dn:
            continue
        seen += 1
        _, cr, cl = (int(t) for t in dn.split("wide_kernel<")[1].split(">")[0].split(","))
        body = kernel_body(asm, name)
        lines = [ln.strip() for ln in body.splitlines()]
        lds_loads = [ln for ln in lines if ln.startswith("global_load_lds_dwordx4")]
        assert len(lds_loads) == 2 * cl and sum(ln.endswith(" nt") for ln in lds_loads) == cl, (dn, lds_loads)
        nt, cached = x4_loads(body)
        assert nt == cr and cached == cr, (dn, nt, cached)
        first_read = next(i for i, ln in enumerate(lines) if ln.startswith("ds_read_b128"))
        assert any(ln.startswith("s_waitcnt vmcnt(0)") for ln in lines[:first_read]), dn
        assert m["lds"] >= cl * 1024 * 16 and m["vgpr"] <= (64 if cr == 4 else 128), (dn, m)
    assert seen == 24


def test_lds_stripe_exchange_kernels(asm):
    """LDS-stripe exchange kernels: CL slots of x (and of r for LayerNorm)
    loaded straight into LDS, non-temporal and cached copies; the exchange's
    agent-scope words; a full wait before the first LDS read."""
    seen = 0
    for name, m in kernel_meta(asm).items():
        dn = demangle(name)
        if "seg_xlds_kernel<" not in dn:
            continue
        seen += 1
        op, cr, cl = (int(t) for t in dn.split("seg_xlds_kernel<")[1].split(">")[0].split(","))
        body = kernel_body(asm, name)
        lines = [ln.strip() for ln in body.splitlines()]
        lds_loads = [ln for ln in lines if ln.startswith("global_load_lds_dwordx4")]
        per_copy = cl * (2 if op == 0 else 1)
        assert len(lds_loads) == 2 * per_copy and sum(ln.endswith(" nt") for ln in lds_loads) == per_copy, dn
        assert any(ln.startswith("global_store_dwordx2") and ln.endswith("sc1") for ln in lines), dn
        first_read = next(i for i, ln in enumerate(lines) if ln.startswith("ds_read_b128"))
        assert any(ln.startswith("s_waitcnt vmcnt(0)") for ln in lines[:first_read]), dn
        assert m["lds"] >= cl * 256 * 16 * (2 if op == 0 else 1), (dn, m)
    assert seen == 9
