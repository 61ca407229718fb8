"""Builds the test-only instruction-check library (libfp4q_instr_check.so, gfx950)
in place, with the same hipcc flags as the product library."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "fp4q_instr_check.hip")
LIB = os.path.join(HERE, "libfp4q_instr_check.so")


def build() -> str:
    sys.path.insert(0, ROOT)
    from fp4_communication_compression_amd import _build
    flags = [f for f in _build.HIPCC_FLAGS]
    flags += ["-I", os.path.join(ROOT, "fp4_communication_compression_amd", "csrc")]
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_build.HIPCC, *flags, SRC, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
