"""Build libmoe_matvec.so in-tree with hipcc for gfx950.

    python -m moe_matvec_amd.build             # compile (always recompiles)
    python -m moe_matvec_amd.build --timeline  # the measurement build with MoE kernel
                                               # timestamps: libmoe_matvec_timeline.so

The library is one shared object: the HIP kernels, the host launchers and the
extern "C" ABI of include/moe_matvec.h.  Each source is compiled to an object
file in its own hipcc process (in parallel), then the objects are linked.
Correctly rounded fp32 division and square root are requested explicitly (the
Q8_1 scale is amax / 127), and the packed-fp32 instructions are disabled for
all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libmoe_matvec.so")
SO_TIMELINE = os.path.join(HERE, "libmoe_matvec_timeline.so")
ARCH = "gfx950"

SOURCES = ["api.hip", "validate.cpp", "gemv_bf16.hip", "gemv_q4_0.hip", "moe.hip", "probe.hip",
           "argmax.hip"]

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-fno-gpu-rdc", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(root, "bin", "hipcc")


def _noise_free(text: str) -> str:
    # the host pass does not know the packed-fp32 feature; drop that warning
    keep = [l for l in text.splitlines()
            if l.strip() and "packed-fp32-ops" not in l and "is not a recognized feature" not in l]
    return "\n".join(keep)


def build(verbose: bool = False, extra_flags=None, timeline: bool = False) -> str:
    """Compile every source and link the library (the timeline build adds
    -DMMV_TIMELINE and writes libmoe_matvec_timeline.so instead)."""
    out = SO_TIMELINE if timeline else SO
    if timeline:
        extra_flags = list(extra_flags or []) + ["-DMMV_TIMELINE=1"]
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="mmv_build_") as tmpdir:
        objs, running, failed = [], [], []
        pending = list(SOURCES)

        def finish(entry):
            proc, src, log = entry
            proc.wait()
            with open(log) as f:
                msg = _noise_free(f.read())
            if proc.returncode != 0:
                failed.append((src, msg))
            elif verbose and msg:
                sys.stderr.write(msg + "\n")

        while pending or running:
            while pending and len(running) < jobs:
                src = pending.pop(0)
                obj = os.path.join(tmpdir, src + ".o")
                log = os.path.join(tmpdir, src + ".log")
                objs.append(obj)
                cmd = [hipcc(), *FLAGS, *(extra_flags or []), "-c", os.path.join(CSRC, src),
                       "-o", obj]
                if verbose:
                    print(" ".join(cmd), flush=True)
                with open(log, "w") as lf:  # output to a file: no pipe to fill up
                    running.append((subprocess.Popen(cmd, stdout=lf, stderr=subprocess.STDOUT),
                                     src, log))
            finish(running.pop(0))
        if failed:
            for src, msg in failed:
                sys.stderr.write(f"--- {src}\n{msg}\n")
            raise RuntimeError("hipcc failed building libmoe_matvec.so: "
                               + ", ".join(s for s, _ in failed))
        tmp = out + ".tmp"
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError("hipcc failed linking libmoe_matvec.so")
        os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
