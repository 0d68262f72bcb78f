"""Build ``libbilogp.so`` in-tree with hipcc for gfx950.

    python -m invariant_linear_log_amd.build [--asm]

Compiles every source under ``csrc/`` into one shared library next to this
file.  The library is written to a temporary name and renamed into place, so
a concurrent reader never sees a half-written file.  ``--asm`` also writes the
device assembly of each kernel source to ``_build/`` for inspection.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_NAME = "libbilogp.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["bilogp_host.cpp", "proj_fwd.hip", "aux_kernels.hip", "merge.hip", "det_gemm.hip"]

# Packed fp32 VALU forms are kept out of all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-command-line-argument",
                f"--offload-arch={ARCH}", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def build(verbose: bool = False, asm: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-shared", "-x", "hip", *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB_PATH)
    if asm:
        bdir = os.path.join(ROOT, "_build")
        os.makedirs(bdir, exist_ok=True)
        for s in srcs:
            if not s.endswith(".hip"):
                continue
            dst = os.path.join(bdir, os.path.basename(s).replace(".hip", ".s"))
            acmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "--cuda-device-only", "-S", "-x",
                    "hip", s, "-o", dst]
            r = subprocess.run(acmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"asm build failed for {s}:\n{r.stderr}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True, asm="--asm" in sys.argv)
    print("built", LIB_PATH)
