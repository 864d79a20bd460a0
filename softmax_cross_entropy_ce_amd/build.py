"""Build libce_mi355x.so in-tree with hipcc for gfx950.

Run as ``python -m softmax_cross_entropy_ce_amd.build`` (or through
``__graft_entry__.build()``).  The library is written next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libce_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["ce_api.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay disabled: hipcc -O3 would otherwise pair fp32
# adds/multiplies into v_pk_*_f32.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile the library; returns its path.  Always recompiles."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}",
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
