"""Parity rule between the HIP path and the oracle (tests only).

Block scales must be bit-exact.  Micro-scales and codes must be bit-exact except
where the oracle's pre-rounding value (t_g, v_i) lies within 1e-6 (relative) of a
rounding boundary; a group whose micro-scale legitimately differs counts as
near-boundary for all its codes.  Tolerated code mismatches must be at most one
step on the signed grid and fewer than 1e-5 of the elements."""
from __future__ import annotations

import numpy as np

from tests import bruteforce as bf


def unpack(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, np.uint8).reshape(-1)
    out = np.empty(2 * c.size, np.uint8)
    out[0::2] = c & 15
    out[1::2] = c >> 4
    return out


def signed_index(c: np.ndarray) -> np.ndarray:
    c = c.astype(np.int64)
    return np.where(c & 8, -(c & 7), c & 7)


def check_compress(gpu, ref, rel: float = 1e-6) -> dict:
    """gpu: (codes, micro, block) numpy; ref: oracle.compress(..., debug=True)."""
    g_codes, g_micro, g_block = (np.asarray(a) for a in gpu)
    assert np.array_equal(g_block.reshape(-1).view(np.uint32),
                          ref["block"].reshape(-1).view(np.uint32)), "block scales differ"
    m_ok = g_micro.reshape(-1) == ref["micro"].reshape(-1)
    near_m = bf.near(ref["t"].reshape(-1), bf.e4m3_midpoints(), rel)
    assert np.all(m_ok | near_m), "micro-scale mismatch away from a rounding midpoint"
    gc, rc = unpack(g_codes), unpack(ref["codes"])
    c_ok = gc == rc
    near_c = bf.near(ref["v"].reshape(-1), bf.e2m1_boundaries(), rel) | np.repeat(~m_ok, 16)
    assert np.all(c_ok | near_c), "code mismatch away from a rounding boundary"
    bad = ~c_ok
    steps = np.abs(signed_index(gc[bad]) - signed_index(rc[bad]))
    assert np.all(steps <= 1), "tolerated code mismatch larger than one step"
    assert bad.sum() < 1e-5 * gc.size or bad.sum() == 0, "too many tolerated mismatches"
    return {"micro_mismatch": int((~m_ok).sum()), "code_mismatch": int(bad.sum()),
            "elements": int(gc.size)}


def check_rowwise(gpu: np.ndarray, ref: np.ndarray, rel: float = 1e-6, magnitude=None) -> float:
    """Per row: max |gpu - ref| <= rel * max |ref|; a zero row must be exactly zero.
    With ``magnitude`` (per element, e.g. the sum of the peers' |terms| of a
    reduce), the row scale is max magnitude instead: the accuracy any fp32
    summation can reach when the terms cancel.  Returns the largest row ratio."""
    g = np.asarray(gpu, np.float64).reshape(ref.shape[0], -1)
    r = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    err = np.abs(g - r).max(axis=1)
    scale = np.abs(r if magnitude is None else np.asarray(magnitude, np.float64).reshape(r.shape)).max(axis=1)
    assert np.all(err <= rel * scale), "row error above %g of the row maximum" % rel
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(scale > 0, err / scale, 0.0)
    return float(ratio.max()) if ratio.size else 0.0


def check_compress_exact(gpu, ref) -> dict:
    """check_compress, and no tolerated mismatch either: every code and every
    micro-scale equal to the oracle's (the kernels follow the oracle's fp32
    operation order, so no value sits on the other side of a boundary)."""
    st = check_compress(gpu, ref)
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0, \
        "near-boundary mismatches where every byte should be exact: %s" % st
    return st
