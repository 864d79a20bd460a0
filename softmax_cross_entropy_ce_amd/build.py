"""Build libce_mi355x.so in-tree with hipcc for gfx950.

Run as ``python -m softmax_cross_entropy_ce_amd.build`` (or through
``__graft_entry__.build()``).  The library is written next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libce_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["ce_api.hip", "ce_wave.hip"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay disabled: hipcc -O3 would otherwise pair fp32
# adds/multiplies into v_pk_*_f32.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _quiet(text: str) -> str:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile the library; returns its path.  Always recompiles: every
    source to an object in a temporary folder, all at once, then one link."""
    cc = hipcc()
    tmp = LIB_PATH + ".tmp"
    with tempfile.TemporaryDirectory(prefix="ce_build_") as work:
        jobs = []
        for src in SOURCES:
            obj = os.path.join(work, os.path.splitext(src)[0] + ".o")
            cmd = [cc, *HIP_FLAGS, *(extra_flags or []), f"-I{INCLUDE}", f"-I{CSRC}", "-c",
                   os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            jobs.append((src, obj, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                    stderr=subprocess.STDOUT, text=True)))
        failed = []
        for src, obj, proc in jobs:
            out = _quiet(proc.communicate()[0])
            if proc.returncode != 0:
                failed.append(f"{src} ({proc.returncode}):\n{out}")
            elif verbose and out.strip():
                print(out)
        if failed:
            raise RuntimeError("hipcc failed: " + "\n".join(failed))
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for _, o, _ in jobs],
               "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link failed ({res.returncode}):\n{_quiet(res.stdout + res.stderr)}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
