"""Build the gfx950 HQQ library in-tree: bit_weight_quantization_amd/libhqq_mi355x.so.

    python -m bit_weight_quantization_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libhqq_mi355x.so")
SOURCES = [os.path.join(CSRC, "hqq_kernels.hip"), os.path.join(CSRC, "hqq_tensor_stop.hip"),
           os.path.join(CSRC, "hqq_matmul.hip"), os.path.join(CSRC, "hqq_lowrank.hip"),
           os.path.join(CSRC, "hqq_meta.hip"), os.path.join(CSRC, "hqq_api.hip")]
HEADERS = [os.path.join(CSRC, "hqq_internal.h"), os.path.join(CSRC, "hqq_solver.h"),
           os.path.join(CSRC, "hqq_tensor_stop.h"), os.path.join(CSRC, "hqq_matmul.h"),
           os.path.join(CSRC, "hqq_lowrank.h"),
           os.path.join(ROOT, "include", "hqq.h")]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # packed fp32 VALU forms stay off: every fp32 op is a plain single-lane op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
