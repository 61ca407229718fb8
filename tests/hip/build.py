"""Builds the test and measurement HIP libraries in place (gfx950, the product
library's hipcc flags): libfp4q_instr_check.so (exhaustive sweeps of the
kernels' rounding primitives, for tests/test_gpu_instructions.py) and
libfp4q_twins.so (compute-free traffic twins of the kernels, for bench.py's
ceilings leg)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIBS = {"libfp4q_instr_check.so": "fp4q_instr_check.hip", "libfp4q_twins.so": "fp4q_twins.hip"}


def build() -> list:
    sys.path.insert(0, ROOT)
    from fp4_communication_compression_amd import _build
    flags = list(_build.HIPCC_FLAGS) + ["-I", os.path.join(ROOT, "fp4_communication_compression_amd", "csrc")]
    built = []
    for lib, src in LIBS.items():
        out = os.path.join(HERE, lib)
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [_build.HIPCC, *flags, os.path.join(HERE, src), "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            noise = "is not a recognized feature for this target"
            err = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
            raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + err)
        os.replace(tmp, out)
        built.append(out)
    return built


if __name__ == "__main__":
    print("\n".join(build()))
