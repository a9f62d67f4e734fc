"""Build libsparsemla.so in-tree with hipcc for gfx950.

``python -m sparse_mla_decode_gather_amd.build`` (or ``build()``) compiles
the HIP kernels and the host C-ABI layer into
``sparse_mla_decode_gather_amd/libsparsemla.so``.  It always recompiles.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libsparsemla.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["kernels.hip", "api.cpp"]

# Packed FP32 VALU forms are kept out of the generated code on purpose.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc",
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (expected /opt/rocm/bin/hipcc)")


def build(verbose: bool = False, extra_flags=None) -> str:
    out_tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-shared", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}",
           f"-I{CSRC}", *DEVICE_FLAGS, *(extra_flags or []),
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", out_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    if verbose and (r.stderr.strip() or r.stdout.strip()):
        print(r.stdout, r.stderr, file=sys.stderr)
    os.replace(out_tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
