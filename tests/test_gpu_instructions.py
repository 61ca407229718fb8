"""Exhaustive GPU checks of the scalar operations every rounding decision of the
kernels rests on (fp4_communication_compression_amd/csrc/fp4q_numerics.h), run
through a test-only HIP library (tests/hip/fp4q_instr_check.hip) that calls the
same functions the kernels call.

* E2M1 conversion (element codes): every finite fp32, at scale 1 and at the
  power-of-two scales of the microscaling variant, against the oracle's E2M1
  encoder, described by its rounding thresholds (the smallest magnitude of each
  code, found by bisection on the oracle) and its sign rule.
* E4M3 conversion after the clamp to 448 (micro-scales): every non-negative
  finite fp32, against the oracle's E4M3 encoder's 126 thresholds.
* rcp_rn: every fp32 with 2^-125 <= |x| < 2^125, against IEEE 1/x.
* coarse_scale: every A in [2^-100, 2^125), against IEEE A / 2688.
* The micro-scale division t = a / (6 s): 2^32 random blocks, bit-exact against
  IEEE division for a >= 2^-99, the same E4M3 code below.
* bfloat16 rounding of the bf16-output receivers: every finite fp32, against
  round-to-nearest-even on the bit pattern.
Each sweep compares on the GPU, in chunks of 2^30 patterns, and stops at the
first chunk with a mismatch.  Samples of every function are also compared with
the oracle (and numpy's IEEE division) directly on the host, and the decode
tables (E4M3 bytes, E2M1 codes at every power-of-two scale the kernels use) are
compared with the oracle's decoders."""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hip", "libfp4q_instr_check.so")
CHUNK = 1 << 30


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ------------------------------------------------- thresholds from the oracle

def _f32(u):
    return np.array([u], np.uint32).view(np.float32)


def _first_at_least(code_of, target: int, lo: int = 0, hi: int = 0x7F7FFFFF) -> int:
    """Smallest non-negative fp32 bit pattern u in [lo, hi] whose code is >= target
    (the oracle's encoders are monotone in the magnitude), by bisection."""
    while lo < hi:
        mid = (lo + hi) // 2
        if code_of(_f32(mid))[0] >= target:
            hi = mid
        else:
            lo = mid + 1
    return lo


def e2m1_thresholds():
    """For magnitude codes m = 1..7: the smallest fp32 that the oracle rounds to m."""
    enc = lambda v: oracle.e2m1_encode(v) & 7
    return [float(_f32(_first_at_least(enc, m))[0]) for m in range(1, 8)]


def e4m3_thresholds():
    """For codes 1..126: the smallest fp32 that the oracle rounds to that code."""
    return [float(_f32(_first_at_least(oracle.e4m3_encode, m))[0]) for m in range(1, 127)]


def test_e2m1_thresholds_are_the_grid_midpoints():
    """The bisection finds the E2M1 grid's midpoints: a midpoint whose upper
    neighbour has an even mantissa (0.75, 1.75, 3.5) belongs to it; the others
    (0.25, 1.25, 2.5, 5) round down, so the threshold is the next fp32 up."""
    up = lambda x: float(np.nextafter(np.float32(x), np.float32(np.inf)))
    assert e2m1_thresholds() == [up(0.25), 0.75, up(1.25), 1.75, up(2.5), 3.5, up(5.0)]
    assert int(oracle.e2m1_encode(np.array([-0.0], np.float32))[0]) == 8


def test_e4m3_thresholds_are_the_grid_midpoints():
    """Each E4M3 threshold is the midpoint between neighbouring codes (ties to the
    even mantissa); the last one, 432, lies between 416 and 448."""
    thr = e4m3_thresholds()
    vals = [oracle.e4m3_decode(c) for c in range(0, 127)]
    for m in range(1, 127):
        mid = 0.5 * (vals[m - 1] + vals[m])
        want = mid if (m & 1) == 0 else float(np.nextafter(np.float32(mid), np.float32(np.inf)))
        assert thr[m - 1] == want, m
    assert thr[-1] == 432.0


# --------------------------------------------------------------- GPU checks

@pytest.fixture(scope="module")
def ic():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    if not os.path.exists(LIB):   # built by __graft_entry__.build(); else build it now
        import importlib.util
        spec = importlib.util.spec_from_file_location("hip_build", os.path.join(HERE, "hip", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    L = ctypes.CDLL(LIB)
    U64, P, I = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_int
    L.ic_e2m1_sweep.argtypes = [U64, U64, ctypes.c_float, P, I, P, P]
    L.ic_e4m3_sweep.argtypes = [U64, U64, P, P, P]
    L.ic_rcp_sweep.argtypes = [U64, U64, P, P]
    L.ic_scale_sweep.argtypes = [U64, U64, P, P]
    L.ic_micro_div_random.argtypes = [U64, U64, U64, P, P]
    L.ic_bf16_sweep.argtypes = [U64, U64, P, P]
    L.ic_half_fma_random.argtypes = [U64, U64, U64, P, P]
    L.ic_eval.argtypes = [I, P, ctypes.c_int64, P, P]
    L.ic_decode_tables.argtypes = [P, I, P, P]
    return L, torch


def _sweep(ic, name, ranges, launch):
    """Runs launch(begin, count, res_ptr, stream) over the ranges in chunks;
    returns (mismatches, first mismatching pattern or index)."""
    L, torch = ic
    res = torch.zeros(2, dtype=torch.int64, device="cuda")
    res[1] = -1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    total = 0
    for lo, hi in ranges:
        for begin in range(lo, hi, CHUNK):
            count = min(CHUNK, hi - begin)
            rc = launch(begin, count, ctypes.c_void_p(res.data_ptr()), stream)
            assert rc == 0, "%s: launch failed (%d)" % (name, rc)
            torch.cuda.synchronize()
            total += count
            bad, first = (int(v) for v in res.cpu().numpy().view(np.uint64))
            if bad:
                _say("%s: %d mismatches in chunk at %#x, first %#x" % (name, bad, begin, first))
                return bad, first
    _say("%s: %d patterns, 0 mismatches" % (name, total))
    return 0, None


FINITE = [(0x00000000, 0x7F800000), (0x80000000, 0xFF800000)]


@pytest.mark.gpu
def test_e2m1_conversion_every_finite_float(ic):
    L, _ = ic
    thr = (ctypes.c_double * 7)(*e2m1_thresholds())
    bad, first = _sweep(ic, "e2m1 scale 1", FINITE,
                        lambda b, c, r, s: L.ic_e2m1_sweep(b, c, 1.0, thr, 8, r, s))
    assert bad == 0, "E2M1 conversion differs from the oracle at pattern %#x" % first


@pytest.mark.gpu
def test_sweep_detects_a_planted_difference(ic):
    """The comparison really runs: with the expectation moved (the threshold of
    code 1 raised by 2^20 ulps, a mistake planted in the host's expectation, not
    in the GPU code) the sweep over [0, 1) reports exactly the patterns in between."""
    L, torch = ic
    thr = e2m1_thresholds()
    u1 = int(np.float32(thr[0]).view(np.uint32))
    moved = (ctypes.c_double * 7)(float(_f32(u1 + (1 << 20))[0]), *thr[1:])
    res = torch.zeros(2, dtype=torch.int64, device="cuda")
    res[1] = -1
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ic_e2m1_sweep(0, 0x3F800000, 1.0, moved, 8, ctypes.c_void_p(res.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    bad, first = (int(v) for v in res.cpu().numpy().view(np.uint64))
    assert bad == 1 << 20 and first == u1


@pytest.mark.gpu
@pytest.mark.parametrize("k", [-126, -123, -4, 4, 60, 125])
def test_e2m1_conversion_power_of_two_scales(ic, k):
    """The microscaling variant converts y / 2^e with the power of two as the
    conversion's scale operand (exponents -126 .. 125 reach it)."""
    L, _ = ic
    thr = (ctypes.c_double * 7)(*[t * 2.0 ** k for t in e2m1_thresholds()])
    bad, first = _sweep(ic, "e2m1 scale 2^%d" % k, FINITE,
                        lambda b, c, r, s: L.ic_e2m1_sweep(b, c, float(2.0 ** k), thr, 8, r, s))
    assert bad == 0, "E2M1 conversion at scale 2^%d differs at pattern %#x" % (k, first)


@pytest.mark.gpu
def test_e4m3_conversion_every_nonnegative_float(ic):
    L, torch = ic
    thr = torch.tensor(e4m3_thresholds(), dtype=torch.float32, device="cuda")
    bad, first = _sweep(ic, "e4m3 (clamped to 448)", [(0x00000000, 0x7F800000)],
                        lambda b, c, r, s: L.ic_e4m3_sweep(b, c, ctypes.c_void_p(thr.data_ptr()), r, s))
    assert bad == 0, "E4M3 conversion differs from the oracle at t = %r" % float(_f32(first)[0])


@pytest.mark.gpu
def test_reciprocal_every_float_in_range(ic):
    L, _ = ic
    lo, hi = 0x01000000, 0x7E000000          # 2^-125 .. 2^125
    bad, first = _sweep(ic, "rcp_rn", [(lo, hi), (lo | 0x80000000, hi | 0x80000000)],
                        lambda b, c, r, s: L.ic_rcp_sweep(b, c, r, s))
    assert bad == 0, "rcp_rn(%r) is not the IEEE reciprocal" % float(_f32(first)[0])


@pytest.mark.gpu
def test_coarse_scale_every_float_in_range(ic):
    L, _ = ic
    bad, first = _sweep(ic, "A / 2688", [(0x0D800000, 0x7E000000)],   # 2^-100 .. 2^125
                        lambda b, c, r, s: L.ic_scale_sweep(b, c, r, s))
    assert bad == 0, "coarse_scale(%r) is not IEEE A / 2688" % float(_f32(first)[0])


@pytest.mark.gpu
def test_micro_scale_division_random_blocks(ic):
    L, _ = ic
    bad, first = _sweep(ic, "a / (6 s), random", [(0, 1 << 32)],
                        lambda b, c, r, s: L.ic_micro_div_random(0x5EED, b, c, r, s))
    assert bad == 0, "micro-scale division differs from IEEE at random index %d" % first


@pytest.mark.gpu
def test_binary16_decode_and_mixed_fma_random(ic):
    """The receivers may decode E2M1 to binary16 and use a mixed-precision fused
    multiply-add: on 2^32 random (code, b, c) draws (scale 1 or 1/16, b and c any
    finite fp32 or typical magnitudes, c also +-0) it equals the binary32 decode
    and fmaf bit for bit, and fma(h, b, -0) equals the rounded product."""
    L, _ = ic
    bad, first = _sweep(ic, "binary16 decode + mixed fma, random", [(0, 1 << 32)],
                        lambda b, c, r, s: L.ic_half_fma_random(0xF16, b, c, r, s))
    assert bad == 0, "binary16 decode / mixed fma differs at random index %d" % first


@pytest.mark.gpu
def test_bf16_rounding_every_finite_float(ic):
    L, _ = ic
    bad, first = _sweep(ic, "bf16 rounding", FINITE, lambda b, c, r, s: L.ic_bf16_sweep(b, c, r, s))
    assert bad == 0, "bfloat16 rounding differs at pattern %#x" % first


def _eval(ic, what, x):
    L, torch = ic
    xd = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    out = torch.empty(x.size, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ic_eval(what, ctypes.c_void_p(xd.data_ptr()), x.size, ctypes.c_void_p(out.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint32)


def _sample_patterns(n, seed, lo=0, hi=1 << 32):
    rng = np.random.default_rng(seed)
    u = rng.integers(lo, hi, size=n, dtype=np.uint64).astype(np.uint32)
    return u[(u & 0x7F800000) != 0x7F800000].view(np.float32)


@pytest.mark.gpu
def test_samples_against_the_oracle_directly(ic):
    """The device functions on random patterns (and on every fp32 within 2^12 ulps
    of each threshold), compared on the host with the oracle's own encoders, its
    bfloat16 rounding and numpy's IEEE reciprocal."""
    near = []
    for t in e2m1_thresholds() + e4m3_thresholds():
        u = int(np.float32(t).view(np.uint32))
        near.append(np.arange(u - 4096, u + 4096, dtype=np.uint32))
    near = np.concatenate(near).view(np.float32)
    x = np.concatenate([_sample_patterns(1 << 20, 11), near, -near])
    np.testing.assert_array_equal(_eval(ic, 0, x), oracle.e2m1_encode(x))
    t = np.abs(x)
    np.testing.assert_array_equal(_eval(ic, 1, t), oracle.e4m3_encode(t))
    np.testing.assert_array_equal(_eval(ic, 3, x), oracle.round_bf16(x))
    r = _sample_patterns(1 << 20, 12, 0x01000000, 0x7E000000)
    r = np.concatenate([r, -r])
    with np.errstate(over="ignore"):
        want = (np.float32(1.0) / r).view(np.uint32)
    np.testing.assert_array_equal(_eval(ic, 2, r), want)


@pytest.mark.gpu
def test_decode_tables(ic):
    """E4M3: the value of every byte; E2M1: every code at every power-of-two
    scale 2^-126 .. 2^127 (the receivers decode with scale 1 or 1/16, the
    microscaling variant with 2^e)."""
    L, torch = ic
    ks = np.arange(-126, 128)
    scales = torch.tensor(np.ldexp(1.0, ks).astype(np.float32), device="cuda")
    out = torch.empty(256 + 32 * ks.size, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ic_decode_tables(ctypes.c_void_p(scales.data_ptr()), ks.size,
                              ctypes.c_void_p(out.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    e4 = np.array([oracle.e4m3_decode(c) for c in range(256)], np.float32)
    nan = np.isnan(e4)
    assert np.array_equal(np.isnan(o[:256]), nan)
    np.testing.assert_array_equal(o[:256][~nan].view(np.uint32), e4[~nan].view(np.uint32))
    e2 = np.array([oracle.e2m1_decode(c) for c in range(16)], np.float64)
    with np.errstate(over="ignore"):   # 3 x 2^127 and 6 x 2^127 round to infinity
        want = (e2[None, :] * np.ldexp(1.0, ks)[:, None]).astype(np.float32).reshape(-1)
    np.testing.assert_array_equal(o[256:256 + 16 * ks.size].view(np.uint32), want.view(np.uint32))
    # binary16 decode, at the scales where every value is a binary16 normal (2^-14 .. 2^4 x 0.5..6)
    half = o[256 + 16 * ks.size:].reshape(ks.size, 16)
    normal = (ks >= -13) & (ks <= 3)
    np.testing.assert_array_equal(half[normal].view(np.uint32), want.reshape(ks.size, 16)[normal].view(np.uint32))
