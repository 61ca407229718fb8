"""Independent NumPy brute-force checker for the oracle (tests only).

It shares nothing with ``oracle/``: the element grid is the literal E2M1 value set,
the E4M3 value set is enumerated from the bit layout, rounding is a nearest-value
search over every code, and the transform is a dense Hadamard matrix in binary64.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes in code order 0..7 (OCP microscaling E2M1; the FP4 element
# type named on the gist.science page, "Problemstellung" item 2).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_values() -> np.ndarray:
    """Value of every non-negative E4M3FN code 0x00..0x7E (index = code)."""
    vals = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10))
    return np.array(vals)


E4M3_VALUES = e4m3_values()


def nearest_e2m1(v: np.ndarray) -> np.ndarray:
    """Nearest E2M1 code by exhaustive search; ties to the even code; sign kept."""
    v = np.asarray(v, np.float64)
    # beyond 8 the nearest magnitude is 6 whatever u is; clamping keeps the
    # distances below exact in binary64
    u = np.minimum(np.abs(v), 8.0)
    d = np.abs(u[..., None] - E2M1_GRID)            # distance to each magnitude
    best = np.argmin(d, axis=-1)                     # first minimum = lower code
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    dn = np.take_along_axis(d, nxt[..., None], -1)[..., 0]
    tie_up = (dn == dmin) & (nxt != best) & (best % 2 == 1)
    mag = np.where(tie_up, nxt, best)
    return (mag | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def nearest_e4m3(t: np.ndarray) -> np.ndarray:
    """Nearest non-negative E4M3 code by exhaustive search (ties to even code)."""
    t = np.minimum(np.asarray(t, np.float64), 1024.0)  # beyond 1024 the nearest is 448
    d = np.abs(t[..., None] - E4M3_VALUES)
    best = np.argmin(d, axis=-1)
    dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 0x7E)
    dn = np.take_along_axis(d, nxt[..., None], -1)[..., 0]
    tie_up = (dn == dmin) & (nxt != best) & (best % 2 == 1)
    return np.where(tie_up, nxt, best).astype(np.uint8)


def nearest_e4m3_sorted(t: np.ndarray) -> np.ndarray:
    """Same rounding as ``nearest_e4m3`` via binary search in the sorted value
    table (used for exhaustive sweeps, where the full search is too slow)."""
    t = np.asarray(t, np.float64)
    V = E4M3_VALUES
    hi = np.clip(np.searchsorted(V, t, side="left"), 1, len(V) - 1)
    lo = hi - 1
    dl = t - V[lo]
    dh = V[hi] - t
    pick_hi = (dh < dl) | ((dh == dl) & (lo % 2 == 1))
    c = np.where(pick_hi, hi, lo)
    c = np.where(t <= 0, 0, c)
    c = np.where(t >= V[-1], len(V) - 1, c)
    return c.astype(np.uint8)


def hadamard(n: int) -> np.ndarray:
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1, -1).astype(np.int64)


H256 = hadamard(256)


def e2m1_boundaries() -> np.ndarray:
    return 0.5 * (E2M1_GRID[:-1] + E2M1_GRID[1:])


def e4m3_midpoints() -> np.ndarray:
    V = E4M3_VALUES
    return 0.5 * (V[:-1] + V[1:])


def near(values: np.ndarray, points: np.ndarray, rel: float) -> np.ndarray:
    """|values| within ``rel`` (relative) of any of ``points``."""
    a = np.abs(np.asarray(values, np.float64))
    idx = np.clip(np.searchsorted(points, a), 1, len(points) - 1)
    d = np.minimum(np.abs(a - points[idx - 1]), np.abs(a - points[idx]))
    return d <= rel * np.maximum(a, 1e-300)


def bf16_magnitudes() -> np.ndarray:
    """Every non-negative finite bfloat16 value in code order (codes 0 .. 0x7F7F),
    then 2^128 standing in for the infinity past the largest one."""
    codes = np.arange(0x7F80, dtype=np.uint32)
    vals = (codes << 16).view(np.float32).astype(np.float64)
    return np.append(vals, 2.0 ** 128)


def nearest_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 by searching the whole grid of bfloat16
    values: the nearer neighbour of |x|, ties to the even code; the sign is
    copied.  uint16 bit patterns."""
    x = np.asarray(x, np.float32).reshape(-1)
    table = bf16_magnitudes()
    m = np.abs(x.astype(np.float64))
    i = np.searchsorted(table, m, side="right") - 1          # table[i] <= m < table[i + 1]
    i = np.minimum(i, table.size - 2)
    d_lo, d_hi = m - table[i], table[i + 1] - m
    code = np.where(d_lo < d_hi, i, np.where(d_hi < d_lo, i + 1, np.where(i % 2 == 0, i, i + 1)))
    code = np.where(d_lo == 0, i, code)
    return (code.astype(np.uint16) | np.where(np.signbit(x), 0x8000, 0).astype(np.uint16))
