"""Checks on the gfx950 assembly of our own kernels (built here, no GPU).

* no private (scratch) segment and no register spills: the row stripes stay
  in VGPRs, so no hidden memory traffic;
* VGPR counts fit the workgroup sizes the kernels are launched with;
* 16-byte loads and stores are used; no MFMA (nothing here is a contraction);
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


def demangle(n):
    return subprocess.run(["c++filt", n], capture_output=True, text=True).stdout.strip()


def test_every_kernel_is_spill_free(asm):
    meta = kernel_meta(asm)
    assert len(meta) == 5 * 11 + 10 + 1  # five operators, affine LayerNorm (no 16-chunk kernel), copy
    for name, m in meta.items():
        # No scratch memory at all.  The 10/12/16-chunk kernels (reachable only
        # through an explicit plan) may park SGPRs in VGPR lanes.
        assert m["private"] == 0 and m["vspill"] == 0, (demangle(name), m)
        dn = demangle(name)
        wide = any(f", {c}>" in dn for c in (10, 12, 16))  # never picked by the chooser
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


def test_barriers_only_where_partials_are_folded(asm):
    copy = [n for n in kernel_meta(asm) if "copy_kernel" in n][0]
    assert "s_barrier" not in kernel_body(asm, copy)
    for name in kernel_meta(asm):
        if "rows_kernel" in name:
            # RMSNorm and row sum fold once, softmax, LayerNorm and min/max
            # twice; matrix-output kernels of at most 4 chunks add one for
            # the staged stores.
            n = kernel_body(asm, name).count("s_barrier")
            dn = demangle(name)
            op = int(dn.split("rows_kernel<")[1].split(",")[0])
            chunks = int(dn.split("rows_kernel<")[1].split(",")[1].split(">")[0])
            folds = {0: 2, 1: 1, 2: 2, 3: 1, 4: 2, 5: 2}[op]
            staged = chunks <= 4 and op not in (3, 4)
            want = folds + (1 if staged else 0)
            assert n == want, (dn, n)
