"""Build libnmsparse.so in place with hipcc for gfx950.

Usage: ``python -m semi_structured_sparse_amd.build`` (or call ``build()``).
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libnmsparse.so"
ARCH = os.environ.get("NM_OFFLOAD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # Packed-FP32 instructions are kept out of the generated code on this platform.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libnmsparse.so)")


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    """Compile every HIP source into PKG_DIR/libnmsparse.so (always recompiles)."""
    out = os.path.join(PKG_DIR, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    # the host pass does not know the packed-fp32 target feature and says so; drop that noise
    noise = ("packed-fp32-ops", "is not a recognized feature", "--hip-link")
    msgs = [l for l in res.stderr.splitlines() if l.strip() and not any(n in l for n in noise)]
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
