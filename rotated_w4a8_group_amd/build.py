"""Builds the package's HIP library ``libpq.so`` in-tree for gfx950 with hipcc.

Usage: ``python -m rotated_w4a8_group_amd.build`` (also called by ``__graft_entry__.build``).
Every call recompiles. Objects go to ``_build/`` under the repository root.
"""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libpq.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

# hipcc flags for every HIP translation unit. Packed fp32 instructions are disabled.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-result", "-Wno-unused-command-line-argument"]

SOURCES = [
    # (source, extra flags)
    ("pq_host.cpp", []),
    # the prologue's results are defined by binary32 ops that each round: no contraction
    ("pq_prologue.hip", ["-ffp-contract=off"]),
    # matrix-core results land in VGPRs (the fold reads them there; no AGPR copies)
    ("pq_gemm.hip", ["-mllvm", "-amdgpu-mfma-vgpr-form"]),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False) -> str:
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    for src, extra in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmd = [cc, "-c"] + lang + HIP_FLAGS + extra + ["-I", INCLUDE, "-I", CSRC,
                                                       os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
