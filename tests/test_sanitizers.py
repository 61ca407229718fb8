"""The oracle and the library's host code under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only; the GPU code is built normally and never
launched): tests/sanitize/oracle_driver.c runs every oracle routine on random,
ragged and edge-case inputs (NaN and infinities included); abi_driver.cpp calls
every C entry point with arguments its validation rejects."""
import os
import shlex
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, cwd, timeout=300):
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True, timeout=timeout)
    return r.returncode, r.stdout + r.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    rc, log = _run(["gcc", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-fno-fast-math", os.path.join(SAN, "oracle_driver.c"),
                    os.path.join(ROOT, "oracle", "fp4q_oracle.c"), "-lm", "-o", exe], ROOT)
    assert rc == 0, log
    rc, log = _run([exe], str(tmp_path))
    assert rc == 0 and "oracle driver ok" in log, log


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_library_host_code_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "abi_driver")
    cmd = shlex.split(
        "%s --offload-arch=gfx950 -O1 -g -std=c++17 -Xclang -target-feature -Xclang -packed-fp32-ops "
        "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined "
        "-Xarch_host -fno-sanitize-recover=all -I %s %s %s -o %s" % (
            HIPCC, os.path.join(ROOT, "include"), os.path.join(SAN, "abi_driver.cpp"),
            os.path.join(ROOT, "fp4_communication_compression_amd", "csrc", "fp4q.hip"), exe))
    rc, log = _run(cmd, str(tmp_path))
    assert rc == 0, log
    rc, log = _run([exe], str(tmp_path), timeout=120)
    assert rc == 0 and "abi driver ok" in log, log
