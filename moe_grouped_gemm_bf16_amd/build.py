"""Build libmgemm.so (and the matrix-core ceiling probe, libmgemm_probe.so)
in-tree with hipcc for gfx950.

    python moe_grouped_gemm_bf16_amd/build.py [--verbose]

(run as a script: importing the package would load the library first).

Always recompiles (it is the "does it build" check as well as the build).
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
LIB = os.path.join(PKG, "libmgemm.so")
SOURCES = ["mgemm_kernels.hip", "mgemm_combine.hip", "mgemm_api.cpp"]
PROBE_LIB = os.path.join(PKG, "libmgemm_probe.so")
PROBE_SOURCES = ["mgemm_probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep packed fp32 vector ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmgemm.so)")


def _link(sources: list[str], target: str, verbose: bool, extra: list[str] | None) -> str:
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *(extra or []),
           *[os.path.join(CSRC, s) for s in sources], "-o", target + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, flush=True)
    os.replace(target + ".tmp", target)
    return target


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    _link(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    return _link(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv or "-v" in sys.argv))
