"""Build libmoe_matvec.so in-tree with hipcc for gfx950.

    python -m moe_matvec_amd.build          # compile (always recompiles)

The library is one shared object: the HIP kernels, the host launchers and the
extern "C" ABI of include/moe_matvec.h.  Correctly rounded fp32 division and
square root are requested explicitly (the Q8_1 scale is amax / 127), and the
packed-fp32 instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmoe_matvec.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "validate.cpp", "gemv_bf16.hip", "gemv_q4_0.hip", "moe.hip", "probe.hip", "argmax.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-fno-gpu-rdc", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "bin", "hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = SO + ".tmp"
    cmd = [hipcc(), *FLAGS, *(extra_flags or []), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libmoe_matvec.so")
    # the host pass does not know the packed-fp32 feature; drop that warning
    noise = [l for l in res.stderr.splitlines()
             if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose=True))
