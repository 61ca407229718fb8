"""The oracle's bfloat16 output rounding against a nearest search over every
bfloat16 value (tests/bruteforce.py), on random float32 patterns, exact ties,
subnormals and the overflow edge."""
import numpy as np

import oracle
from tests import bruteforce as bf


def _finite(u32):
    x = u32.view(np.float32)
    return x[np.isfinite(x)]


def test_random_patterns():
    rng = np.random.default_rng(11)
    x = _finite(rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32))
    np.testing.assert_array_equal(oracle.round_bf16(x), bf.nearest_bf16(x))


def test_ties_go_to_the_even_code():
    rng = np.random.default_rng(12)
    hi = rng.integers(0, 0x7F7F, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    u = (hi << 16) | 0x8000                     # exactly halfway between hi and hi + 1
    x = np.concatenate([u.view(np.float32), (u | 0x80000000).view(np.float32)])
    got = oracle.round_bf16(x)
    np.testing.assert_array_equal(got, bf.nearest_bf16(x))
    assert np.all(got & 1 == 0)                 # the even neighbour, always
    # spot values: 1 + 2^-8 lies halfway between 1 (0x3F80) and 1 + 2^-7 (0x3F81)
    assert oracle.round_bf16(np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)])).tolist() == \
        [0x3F80, 0x3F82, 0xBF80]


def test_subnormals_zeros_and_overflow_edge():
    rng = np.random.default_rng(13)
    sub = rng.integers(1, 0x800000, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([sub.view(np.float32), (sub | 0x80000000).view(np.float32)])
    np.testing.assert_array_equal(oracle.round_bf16(x), bf.nearest_bf16(x))
    edge = np.array([0x00000000, 0x80000000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7FFFFF, 0x7F7F0000,
                     0xFF7F8000], np.uint32).view(np.float32)
    # +0, -0, just below the overflow midpoint, the midpoint (odd code: up to infinity),
    # the largest float32, the largest bfloat16, the negative midpoint
    assert oracle.round_bf16(edge).tolist() == [0x0000, 0x8000, 0x7F7F, 0x7F80, 0x7F80, 0x7F7F, 0xFF80]
    np.testing.assert_array_equal(oracle.round_bf16(edge), bf.nearest_bf16(edge))
