"""The oracle's pins catch plausible mistakes.

Each mutant below is a copy of oracle/fp4q_oracle.c (or of the binary64 metric
and widening in oracle/__init__.py) with one planted mistake of the kinds a
from-scratch implementation could make: a wrong sign, index or constant, a
dropped term or step, swapped operands, the wrong nibble, transform domain or
summation order, the wrong norm or precision.  Each C mutant is built with the
oracle's own gcc flags; the pin tests (tests/test_oracle_*.py, which compare
the oracle with closed forms, brute force and properties, never with itself)
run against it in a fresh process; every mutant must make at least one pin
fail.  Every mutant stays
memory-safe (no index leaves its array), so a failure is a failed pin, never a
crash.  Runs on the CPU only."""
import concurrent.futures
import os
import subprocess
import sys

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_TESTS = ["tests/test_oracle_formats.py", "tests/test_oracle_fwht.py",
             "tests/test_oracle_pipeline.py", "tests/test_oracle_requantize.py",
             "tests/test_oracle_mx.py", "tests/test_oracle_properties.py",
             "tests/test_oracle_bf16.py", "tests/test_oracle_metrics.py"]

# name -> (text in the oracle source, its replacement); the text must occur once
MUTANTS = {
    # bf16 input
    "widen: shift by 15": ("(uint32_t)h << 16", "(uint32_t)h << 15"),
    # E2M1
    "e2m1 decode: subnormal step 1": ("0.5f * (float)m : ldexpf", "1.0f * (float)m : ldexpf"),
    "e2m1 decode: exponent bias 0": ("ldexpf(1.0f + 0.5f * (float)m, e - 1)",
                                     "ldexpf(1.0f + 0.5f * (float)m, e)"),
    "e2m1 encode: ties to odd": ("(u == mid && (c & 1))", "(u == mid && !(c & 1))"),
    "e2m1 encode: ties always up": ("(u == mid && (c & 1))", "(u == mid)"),
    "e2m1 encode: sign dropped": ("return mag | (signbit(v) ? 8 : 0);", "return mag;"),
    "e2m1 encode: no saturation step": ("for (int c = 0; c < 7; ++c)", "for (int c = 0; c < 6; ++c)"),
    # E4M3
    "e4m3 decode: bias 8": ("ldexpf(1.0f + (float)m / 8.0f, e - 7)",
                            "ldexpf(1.0f + (float)m / 8.0f, e - 8)"),
    "e4m3 decode: subnormal step 2^-10": ("ldexpf((float)m, -9)", "ldexpf((float)m, -10)"),
    "e4m3 encode: subnormal range one binade short": ("if (E < -6) {", "if (E < -7) {"),
    "e4m3 encode: truncation": ("double q = nearbyint(ldexp(u, 3 - E));",
                                "double q = floor(ldexp(u, 3 - E));"),
    # transform
    "fwht: butterfly sign": ("y[i + h] = a - b;\n            }\n    for (int i = 0; i < BLOCK; ++i) y[i] *= 0.0625f;",
                             "y[i + h] = b - a;\n            }\n    for (int i = 0; i < BLOCK; ++i) y[i] *= 0.0625f;"),
    "fwht: last stage dropped": ("for (int h = 1; h < BLOCK; h <<= 1)\n        for (int i = 0; i < BLOCK; ++i)\n            if ((i & h) == 0) {\n                float",
                                 "for (int h = 1; h < BLOCK / 2; h <<= 1)\n        for (int i = 0; i < BLOCK; ++i)\n            if ((i & h) == 0) {\n                float"),
    "fwht: normalised by 1/8": ("y[i] *= 0.0625f;", "y[i] *= 0.125f;"),
    "fwht (binary64): butterfly sign": ("double a = y[i], b = y[i + h];\n                y[i] = a + b;\n                y[i + h] = a - b;",
                                        "double a = y[i], b = y[i + h];\n                y[i] = a + b;\n                y[i + h] = b - a;"),
    # dual scale and quantisation
    "coarse scale: divided by 448": ("float s = A / 2688.0f;", "float s = A / 448.0f;"),
    "micro-scale: 6 dropped": ("float d = 6.0f * s;", "float d = s;"),
    "micro-scale: block maximum for every group": ("for (int i = 0; i < GROUP; ++i) a = fmaxf(a, fabsf(yg[i]));\n        float t",
                                                   "a = A;\n        float t"),
    "quantise: scale instead of its reciprocal": ("float r = (S == 0.0f) ? 0.0f : 1.0f / S;",
                                                  "float r = S;"),
    "quantise: micro-scale left out of S": ("float S = s * fp4q_ref_e4m3_decode(m);", "float S = s;"),
    # packing
    "pack: high nibble first": ("codes[k] = (uint8_t)(code[2 * k] | (code[2 * k + 1] << 4));\n}\n\nstatic void compress_block(",
                                "codes[k] = (uint8_t)(code[2 * k + 1] | (code[2 * k] << 4));\n}\n\nstatic void compress_block("),
    # receiver
    "decompress: nibble order swapped": ("int c = (codes[e >> 1] >> (4 * (e & 1))) & 15;\n            out[e] = fp4q_ref_e2m1_decode(c) * S;",
                                         "int c = (codes[e >> 1] >> (4 * !(e & 1))) & 15;\n            out[e] = fp4q_ref_e2m1_decode(c) * S;"),
    "decompress: inverse transform dropped": ("    if (fwht) fp4q_ref_fwht256(out);\n}\n\nvoid fp4q_ref_decompress(",
                                              "}\n\nvoid fp4q_ref_decompress("),
    "decompress (binary64): micro-scale dropped": ("double S = (double)s * (double)fp4q_ref_e4m3_decode(micro[g]);",
                                                   "double S = (double)s;"),
    "reduce: only the last peer kept": ("for (int i = 0; i < BLOCK; ++i) acc[i] += d[i];",
                                        "for (int i = 0; i < BLOCK; ++i) acc[i] = d[i];"),
    "re-quantise: peers transformed back": ("block[p][b], 0, d);", "block[p][b], 1, d);"),
    "re-quantise: local slice not transformed": ("if (fwht) fp4q_ref_fwht256(acc);", ""),
    "re-quantise: first peer skipped": ("for (int p = 0; p < k; ++p) {\n            decompress_block(",
                                        "for (int p = 1; p < k; ++p) {\n            decompress_block("),
    "re-quantise: peers in reverse order": ("for (int p = 0; p < k; ++p) {\n            decompress_block(",
                                            "for (int p = k - 1; p >= 0; --p) {\n            decompress_block("),
    # bfloat16 output option
    "bf16 round: ties away from zero": ("return (lo & 1u) ? hi : lo;", "return hi;"),
    "bf16 round: truncation": ("if (x - a < b - x) return lo;", "if (x - a < b - x || 1) return lo;"),
    # MX variant
    "mx: scale exponent off by one": ("int e = (e2 - 1) - 2;", "int e = (e2 - 1) - 1;"),
    "mx: zero group exponent": ("if (!(amax > 0.0f)) return -127;", "if (!(amax > 0.0f)) return 0;"),
    "mx decode: scale bias 126": ("int ex = (int)scales[MXNGROUP * b + e / MXGROUP] - 127;",
                                  "int ex = (int)scales[MXNGROUP * b + e / MXGROUP] - 126;"),
}


# the same for oracle/__init__.py (the binary64 error metric and the widening)
PY_MUTANTS = {
    "rel_rmse: norm of the output in the denominator": (
        "nx = float(np.sqrt(np.sum(x * x)))",
        "nx = float(np.sqrt(np.sum(np.asarray(xhat, np.float64) ** 2)))"),
    "rel_rmse: no square root": ("return float(np.sqrt(np.sum(d * d))) / nx if nx > 0 else 0.0",
                                 "return float(np.sum(d * d)) / (nx * nx) if nx > 0 else 0.0"),
    "rel_rmse: binary32 difference": ("d = np.asarray(xhat, np.float64) - x",
                                      "d = (np.asarray(xhat, np.float32) - x.astype(np.float32)).astype(np.float64)"),
    "rel_rmse: mean of per-row ratios": (
        "return float(np.sqrt(np.sum(d * d))) / nx if nx > 0 else 0.0",
        "return float(np.mean(np.sqrt(np.sum(np.atleast_2d(d) ** 2, axis=-1)) / "
        "np.sqrt(np.sum(np.atleast_2d(x) ** 2, axis=-1)))) if nx > 0 else 0.0"),
    "widen: shift by 15": ("return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 16).view(np.float32)",
                           "return (np.asarray(x_bf16, np.uint16).astype(np.uint32) << 15).view(np.float32)"),
}


def _source():
    with open(os.path.join(ROOT, "oracle", "fp4q_oracle.c")) as f:
        return f.read()


def _py_source():
    with open(os.path.join(ROOT, "oracle", "__init__.py")) as f:
        return f.read()


def test_every_mutation_applies_once():
    for src, table in ((_source(), MUTANTS), (_py_source(), PY_MUTANTS)):
        for name, (old, new) in table.items():
            assert src.count(old) == 1, "mutant %r: its text occurs %d times" % (name, src.count(old))


def _run_pins(name, old, new, tmp, python=False):
    """Builds the source with `old` replaced by `new` (python: the package's
    __init__.py, loaded first in the test process so that every `import oracle`
    gets the copy; the unchanged C library) and runs the pins against it in a
    fresh process: pytest's exit status (0 all passed, 1 a pin failed) and the
    end of its report."""
    tag = "".join(ch if ch.isalnum() else "_" for ch in name) + ("_py" if python else "")
    lib_path = os.path.join(tmp, tag + ".so")
    if python:
        pkg = os.path.join(tmp, tag, "oracle")
        os.makedirs(pkg)
        with open(os.path.join(pkg, "__init__.py"), "w") as f:
            f.write(_py_source().replace(old, new))
        lib_path = oracle.build()
        pre = ("import sys; sys.path.insert(0, %r); import oracle; sys.path.pop(0); "
               "import pytest; sys.exit(pytest.main(sys.argv[1:]))" % os.path.join(tmp, tag))
        cmd = [sys.executable, "-c", pre]
    else:
        src_path = os.path.join(tmp, tag + ".c")
        with open(src_path, "w") as f:
            f.write(_source().replace(old, new) if old else _source())
        subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-o", lib_path, src_path, "-lm"])
        cmd = [sys.executable, "-m", "pytest"]
    env = dict(os.environ, **{oracle.LIB_ENV: lib_path, "OMP_NUM_THREADS": "2"})
    r = subprocess.run([*cmd, *PIN_TESTS, "-x", "-q", "-m", "not gpu and not exhaustive",
                        "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-1500:]


def test_pins_catch_every_mutant(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as pool:
        control = pool.submit(_run_pins, "unchanged", "", "", str(tmp_path))
        futs = {name: pool.submit(_run_pins, name, old, new, str(tmp_path))
                for name, (old, new) in MUTANTS.items()}
        futs.update({name: pool.submit(_run_pins, name, old, new, str(tmp_path), True)
                     for name, (old, new) in PY_MUTANTS.items()})
        # the unchanged source, built and loaded the same way, passes every pin
        rc, report = control.result()
        assert rc == 0, "the unchanged oracle fails its pins in this harness:\n" + report
        survived = {name: f.result()[1] for name, f in futs.items() if f.result()[0] != 1}
    assert not survived, "mutants no pin catches: %s\n%s" % (
        sorted(survived), "\n".join("--- %s\n%s" % kv for kv in survived.items()))
