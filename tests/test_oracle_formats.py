"""Pins of the oracle's scalar formats: E2M1 and E4M3 decode and encode.

The expected values come from the value sets in tests/golden/e2m1_e4m3_values.txt
and from an exhaustive nearest-value search (tests/bruteforce.py), never from the
oracle itself."""
import os

import numpy as np
import pytest

import oracle
from tests import bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e2m1_e4m3_values.txt")


@pytest.fixture
def all_threads():
    """The exhaustive sweeps run the oracle on every host core."""
    oracle.set_threads(os.cpu_count() or 1)
    yield
    oracle.set_threads(1)


def _golden():
    e2m1, e4m3 = None, {}
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if not line:
            continue
        if line[0] == "e2m1":
            e2m1 = [float(v) for v in line[1:]]
        elif line[0] == "e4m3":
            e4m3[int(line[1], 16)] = float(line[2])
    return e2m1, e4m3


def _all_patterns(lo_bits: int, hi_bits: int) -> np.ndarray:
    return np.arange(lo_bits, hi_bits, dtype=np.uint32).view(np.float32)


def test_e2m1_decode_matches_value_set():
    e2m1, _ = _golden()
    for c in range(16):
        got = oracle.e2m1_decode(c)
        want = e2m1[c & 7] * (-1.0 if c & 8 else 1.0)
        assert got == want
        assert np.signbit(got) == bool(c & 8)


def test_e2m1_encode_midpoints_and_neighbours():
    mids = bf.e2m1_boundaries().astype(np.float32)
    vals = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(9)),
                           bf.E2M1_GRID.astype(np.float32), np.float32([6.5, 7.0, 8.0, 1e30, 3.4e38])])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    np.testing.assert_array_equal(oracle.e2m1_encode(vals), bf.nearest_e2m1(vals))
    # the seven midpoints go to the code with mantissa 0: 0.25->0, 0.75->1.0, 1.25->1.0,
    # 1.75->2.0, 2.5->2.0, 3.5->4.0, 5->4.0
    assert list(oracle.e2m1_encode(mids)) == [0, 2, 2, 4, 4, 6, 6]


def test_e2m1_sign_of_zero_kept():
    v = np.float32([0.0, -0.0, 0.1, -0.1, 0.25, -0.25, -1e-40])
    assert list(oracle.e2m1_encode(v)) == [0, 8, 0, 8, 0, 8, 8]


def _windows(points: np.ndarray, half: int) -> np.ndarray:
    """Every fp32 pattern within ``half`` ulps of each (positive, fp32-exact) point."""
    bits = np.asarray(points, np.float32).view(np.uint32).astype(np.int64)
    off = np.arange(-half, half + 1, dtype=np.int64)
    w = (bits[:, None] + off[None, :]).reshape(-1)
    return w[w >= 0].astype(np.uint32).view(np.float32)


def _exhaustive_runs(encode, brute, lo: int, hi: int, chunk: int = 1 << 24):
    """Every fp32 bit pattern in [lo, hi) (all of one sign, so the magnitude grows
    with the pattern): the oracle's code equals the brute-force code at each one.
    The brute force (nearest value on an ordered grid, ties to the even code, the
    sign copied) is monotone in the magnitude, so it is evaluated at both ends of
    every run of equal oracle codes: equal there means equal on the whole run.
    The oracle itself runs on every pattern."""
    for b in range(lo, hi, chunk):
        u = np.arange(b, min(hi, b + chunk), dtype=np.uint32)
        c = encode(u.view(np.float32))
        cut = np.flatnonzero(c[1:] != c[:-1])
        ends = np.concatenate([[0], cut, cut + 1, [c.size - 1]])
        np.testing.assert_array_equal(brute(u[ends].view(np.float32)), c[ends])


def test_e2m1_encode_exhaustive_near_every_decision_point():
    """All fp32 patterns within 2^16 ulps of every midpoint and grid value, both signs."""
    pts = np.concatenate([bf.e2m1_boundaries(), bf.E2M1_GRID[1:]]).astype(np.float32)
    v = _windows(pts, 1 << 16)
    for s_ in (v, -v):
        np.testing.assert_array_equal(oracle.e2m1_encode(s_), bf.nearest_e2m1(s_))


@pytest.mark.exhaustive
@pytest.mark.parametrize("lo,hi", [(0x3E000000, 0x3F800000), (0x3F800000, 0x40800000),
                                   (0x40800000, 0x41800000)])
def test_e2m1_encode_exhaustive_binades(lo, hi, all_threads):
    """Every fp32 pattern with magnitude in [1/8, 16), both signs, against the full
    nearest-code search at every pattern (no shortcut)."""
    step = 1 << 22
    for b in range(lo, hi, step):
        v = _all_patterns(b, min(hi, b + step))
        np.testing.assert_array_equal(oracle.e2m1_encode(v), bf.nearest_e2m1(v))
        nv = -v
        np.testing.assert_array_equal(oracle.e2m1_encode(nv), bf.nearest_e2m1(nv))


def test_e2m1_encode_random_patterns():
    rng = np.random.default_rng(11)
    u = rng.integers(0, 1 << 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[np.isfinite(v)]
    np.testing.assert_array_equal(oracle.e2m1_encode(v), bf.nearest_e2m1(v))


@pytest.mark.exhaustive
def test_e2m1_encode_exhaustive_all_finite(all_threads):
    """Every finite fp32 bit pattern, both signs (2^32 - 2^25 patterns)."""
    _exhaustive_runs(oracle.e2m1_encode, bf.nearest_e2m1, 0x00000000, 0x7F800000)
    _exhaustive_runs(oracle.e2m1_encode, bf.nearest_e2m1, 0x80000000, 0xFF800000)


def test_e4m3_decode_spot_values_and_structure():
    _, spots = _golden()
    for code, val in spots.items():
        got = oracle.e4m3_decode(code)
        assert got == val and np.signbit(got) == np.signbit(val), hex(code)
    assert np.isnan(oracle.e4m3_decode(0x7F)) and np.isnan(oracle.e4m3_decode(0xFF))
    vals = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    assert np.all(np.diff(vals) > 0)                 # strictly increasing 0x00..0x7E
    assert np.count_nonzero(vals > 0) == 126
    # spacing doubles every 8 codes above the subnormals (3 mantissa bits)
    sp = np.diff(vals)
    assert np.all(sp[:8] == 2.0 ** -9)
    for e in range(1, 15):
        assert np.all(sp[8 * e:8 * e + 8][:7 if e == 14 else 8] == 2.0 ** (e - 10))
    np.testing.assert_array_equal(vals, bf.E4M3_VALUES)
    for c in range(0x80):
        assert oracle.e4m3_decode(c | 0x80) == -oracle.e4m3_decode(c) or c == 0x7F


def test_e4m3_encode_midpoints_and_neighbours():
    mids = bf.e4m3_midpoints()
    m32 = mids.astype(np.float32)
    assert np.all(m32.astype(np.float64) == mids)    # midpoints are exact in fp32
    vals = np.concatenate([m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9)),
                           bf.E4M3_VALUES.astype(np.float32),
                           np.float32([0, 2.0 ** -10, 2.0 ** -11, 1e-30, 1e-45, 448, 449, 463.9,
                                       464, 470, 1e6, 3.4e38])])
    np.testing.assert_array_equal(oracle.e4m3_encode(vals), bf.nearest_e4m3(vals))
    got = oracle.e4m3_encode(m32)
    assert np.all(got % 2 == 0)                      # every tie lands on an even mantissa


def test_e4m3_encode_random_bruteforce():
    rng = np.random.default_rng(12)
    t = np.exp2(rng.uniform(-12, 10, size=400_000)).astype(np.float32)
    np.testing.assert_array_equal(oracle.e4m3_encode(t), bf.nearest_e4m3(t))


def test_e4m3_encode_exhaustive_near_every_midpoint():
    """All fp32 patterns within 2^12 ulps of each of the 126 rounding midpoints."""
    v = _windows(bf.e4m3_midpoints().astype(np.float32), 1 << 12)
    np.testing.assert_array_equal(oracle.e4m3_encode(v), bf.nearest_e4m3_sorted(v))


@pytest.mark.exhaustive
def test_e4m3_encode_exhaustive_range(all_threads):
    """Every non-negative finite fp32 pattern (every t the micro-scale step can
    produce), against a nearest-value rounding by binary search in the value
    table, evaluated at both ends of every run of equal codes."""
    _exhaustive_runs(oracle.e4m3_encode, bf.nearest_e4m3_sorted, 0x00000000, 0x7F800000)