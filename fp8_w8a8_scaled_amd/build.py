"""Build libfp8mm.so (the C-ABI library) in-tree for gfx950 with hipcc.

    python fp8_w8a8_scaled_amd/build.py

Flags: -O3 for gfx950 only; -ffp-contract=off so no multiply-add pair of the
quant and epilogue arithmetic is fused; packed fp32 instructions disabled
(-packed-fp32-ops), the compiler otherwise forms v_pk_* from ordinary float code.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8mm.so")
ROOT = os.path.dirname(HERE)

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Werror=uninitialized", "-Werror=sometimes-uninitialized",
    "-I", os.path.join(ROOT, "include"),
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every source to an object in parallel (one hipcc per file), then
    link the shared library."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(objdir, os.path.basename(f) + ".o") for f in srcs]
    cmds = [[hipcc, *HIPCC_FLAGS, "-c", f, "-o", o] for f, o in zip(srcs, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for rc in ex.map(lambda c: subprocess.call(c), cmds):
            if rc != 0:
                raise subprocess.CalledProcessError(rc, "hipcc")
    tmp = LIB + ".tmp"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
