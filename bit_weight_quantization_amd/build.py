"""Build the gfx950 HQQ library in-tree: bit_weight_quantization_amd/libhqq_mi355x.so.

    python -m bit_weight_quantization_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys
import tempfile

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

# The issue-rate probe the benchmark prices its VALU roofline with: a library of its own,
# not part of the quantizer's C ABI.
PROBE_SRC = os.path.join(CSRC, "hqq_valu_probe.hip")
PROBE_LIB = os.path.join(PKG, "libhqq_valu_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
    # packed fp32 VALU forms stay off: every fp32 op is a plain single-lane op
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
# hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
_NOISE = "is not a recognized feature for this target"


def _run(cmd: list[str]) -> list[str]:
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if _NOISE not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    return msgs


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path.  The sources are
    compiled to objects in parallel, then linked into the shared library."""
    jobs = min(len(SOURCES) + 1, int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)))
    with tempfile.TemporaryDirectory(prefix="hqq_build_") as tmp:
        objs = [os.path.join(tmp, os.path.splitext(os.path.basename(s))[0] + ".o") for s in SOURCES]
        cmds = [[HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-c", s, "-o", o]
                for s, o in zip(SOURCES, objs)]
        cmds.append([HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", PROBE_LIB + ".tmp"])
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with concurrent.futures.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
            msgs = [m for ms in ex.map(_run, cmds) for m in ms]
        link = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
        if verbose:
            print(" ".join(link), flush=True)
        msgs += _run(link)
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(LIB + ".tmp", LIB)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in SOURCES + HEADERS)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
