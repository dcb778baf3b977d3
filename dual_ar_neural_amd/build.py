"""Build libs2fast.so (the HIP library behind include/s2fast.h) for gfx950.

    python -m dual_ar_neural_amd.build

The library is built in-tree next to this file, so it travels with the
repository to the GPU machine.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libs2fast.so")
SOURCES = [os.path.join(HERE, "csrc", "s2fast.hip")]
DEPS = SOURCES + [os.path.join(HERE, "csrc", f) for f in ("device_common.h", "sampler.h", "batched.h", "slow_step.h", "prefill.h", "slow_host.h")] + \
    [os.path.join(ROOT, "include", "s2fast.h")]

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # keep the compiler away from packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for c in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libs2fast.so")


def build(verbose: bool = False) -> str:
    """Compile the library (always), atomically replacing any previous build."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-o", tmp, *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
