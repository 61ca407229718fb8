"""Builds libfp4q.so (gfx950 only) in place with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(HERE, "csrc", "fp4q.hip")]
HEADERS = [os.path.join(ROOT, "include", "fp4q.h"), os.path.join(HERE, "csrc", "fp4q_numerics.h")]
LIB = os.path.join(HERE, "libfp4q.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # the kernels reproduce an fp32 operation order: no contraction into FMA,
    # IEEE division, fp32 denormals kept
    "-ffp-contract=off",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # never emit packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(force: bool = True, verbose: bool = False) -> str:
    stale = not os.path.exists(LIB) or any(
        os.path.getmtime(s) > os.path.getmtime(LIB) for s in SOURCES + HEADERS)
    if not (force or stale):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
