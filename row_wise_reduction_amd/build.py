"""Build ``librowred.so`` (gfx950 kernels + C ABI) in-tree with hipcc.

    python -m row_wise_reduction_amd.build          # build the library
    python -m row_wise_reduction_amd.build --asm    # also write the gfx950 assembly

hipcc cross-compiles for gfx950 without a GPU.  Packed FP32 instructions are
turned off for the device code (``-packed-fp32-ops``); hipcc's host pass warns
that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "librowred.so")
ASM = os.path.join(PKG, "_build", "rowred_kernels-gfx950.s")

DEVICE_SOURCES = [os.path.join(CSRC, "rowred_kernels.hip"), os.path.join(CSRC, "rowred_split.hip"),
                  os.path.join(CSRC, "rowred_looped.hip"), os.path.join(CSRC, "rowred_wide.hip"),
                  os.path.join(CSRC, "rowred_flat.hip")]
SOURCES = DEVICE_SOURCES + [os.path.join(CSRC, "rowred_api.cpp")]
HEADERS = [os.path.join(CSRC, "rowred_internal.h"), os.path.join(CSRC, "rowred_device.h"),
           os.path.join(INCLUDE, "rowred.h")]

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", f"-I{INCLUDE}", f"-I{CSRC}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode})")
    return r


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile every source into ``row_wise_reduction_amd/librowred.so``
    (or `out`, with extra ``-D`` build-time settings)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, *[f"-D{d}" for d in defines], "-fPIC", "-shared", "-fvisibility=hidden", "-o", tmp,
           *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, out)
    return out


def device_asm(path: str = ASM) -> str:
    """Write the gfx950 assembly of every kernel source, concatenated into
    one file (for resource/ISA checks)."""
    os.makedirs(os.path.dirname(path), exist_ok=True)
    parts = []
    tag = f"{os.getpid()}"  # concurrent callers (parallel test workers) write their own files
    for i, src in enumerate(DEVICE_SOURCES):
        part = f"{path}.{tag}.{i}"
        _run([HIPCC, *COMMON, "--cuda-device-only", "-S", "-o", part, src])
        parts.append(open(part).read())
        os.remove(part)
    tmp = f"{path}.{tag}"
    with open(tmp, "w") as f:
        f.write("\n".join(parts))
    os.replace(tmp, path)
    return path


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))
    if args.asm:
        print(device_asm())


if __name__ == "__main__":
    main()
