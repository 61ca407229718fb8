"""Pins of the oracle's receiver-side re-quantisation (sum of k payloads in the
transform domain, quantised again), checked without calling the oracle's own
arithmetic for the expected values."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from tests.parity import unpack
from fp4_communication_compression_amd import inputs


def _payloads(k, rows=6, L=1024, seed=40, scale=1e-3):
    out = []
    for p in range(k):
        xb = inputs.make_normal(rows, L, seed=seed + p, scale=scale)
        r = oracle.compress(xb)
        out.append((r["codes"], r["micro"], r["block"]))
    return out


def _dequant_f32(codes, micro, block):
    """Independent decode: E2M1 literal grid times fp32(block * E4M3 value)."""
    c = unpack(codes).reshape(-1, 16, 16)
    mag = bf.E2M1_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    m = np.asarray(micro).reshape(-1, 16)
    S = (np.asarray(block, np.float32).reshape(-1, 1) * bf.E4M3_VALUES[m].astype(np.float32)).astype(np.float32)
    return (mag.astype(np.float32) * S[:, :, None]).astype(np.float32).reshape(-1, 256)


def _transform_domain_sum(payloads):
    acc = np.zeros_like(_dequant_f32(*payloads[0]))
    for p in payloads:
        acc = (acc + _dequant_f32(*p)).astype(np.float32)   # fp32, peer order, from +0
    return acc


def _check_quantised(got, y):
    """Brute-force re-quantisation of the fp32 sum y [blocks, 256] (as float64):
    block scales to 1e-6, micro-scales and codes by nearest-code search, exempt
    within 1e-6 of a rounding boundary."""
    A = np.abs(y).max(axis=1)
    s = A / 2688.0
    np.testing.assert_allclose(got["block"].reshape(-1), s, rtol=1e-6)
    a = np.abs(y).reshape(-1, 16, 16).max(axis=2)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s[:, None] > 0, a / (6.0 * s[:, None]), 0.0)
    m = bf.nearest_e4m3(t)
    near_m = bf.near(t, bf.e4m3_midpoints(), 1e-6)
    assert np.all((got["micro"].reshape(-1, 16) == m) | near_m)
    S = s[:, None] * bf.E4M3_VALUES[m]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(S[:, :, None] > 0, y.reshape(-1, 16, 16) / S[:, :, None], 0.0 * y.reshape(-1, 16, 16))
    codes = bf.nearest_e2m1(v).reshape(-1, 256)
    near_c = bf.near(v.reshape(-1, 256), bf.e2m1_boundaries(), 1e-6) | np.repeat(near_m, 16, axis=1)
    gc = unpack(got["codes"]).reshape(-1, 256)
    assert np.all((gc == codes) | near_c)


@pytest.mark.parametrize("k", [1, 3, 8])
def test_requantize_against_brute_force(k):
    pay = _payloads(k)
    got = oracle.requantize(pay, debug=True)
    _check_quantised(got, _transform_domain_sum(pay).astype(np.float64))


def _local_slice(rows=6, L=1024, seed=60):
    """bf16 local slice of small multiples of 2^-10 (|x| <= 8 * 2^-10): every sum
    of the transform is exact in fp32, so the dense binary64 Hadamard product
    equals the radix-2 result exactly."""
    rng = np.random.default_rng(seed)
    x = (rng.integers(-8, 9, (rows, L)) * 2.0 ** -10).astype(np.float32)
    return inputs.f32_to_bf16_bits(x), x


@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("k", [0, 1, 3])
def test_requantize_with_local_against_brute_force(k, fwht):
    """The accumulator starts at the local slice, transformed (dense H/16) or as
    is, then each peer's decoded payload is added in fp32, in peer order."""
    xb, x = _local_slice()
    pay = []
    for p in range(k):
        r = oracle.compress(inputs.make_normal(6, 1024, seed=70 + p, scale=1e-3), fwht=fwht)
        pay.append((r["codes"], r["micro"], r["block"]))
    got = oracle.requantize(pay, debug=True, local=xb, fwht=fwht)
    blocks = x.astype(np.float64).reshape(-1, 256)
    acc = ((blocks @ bf.H256.T) / 16.0 if fwht else blocks).astype(np.float32)
    for p in pay:
        acc = (acc + _dequant_f32(*p)).astype(np.float32)
    _check_quantised(got, acc.astype(np.float64))


@pytest.mark.parametrize("fwht", [True, False])
def test_requantize_local_special_cases(fwht):
    """No peers: the result is the local slice compressed.  An all-zero local
    slice: the result equals the sum without one."""
    xb = inputs.make_normal(5, 2048, seed=81)
    alone = oracle.requantize([], local=xb, fwht=fwht)
    comp = oracle.compress(xb, fwht=fwht)
    for key in ("codes", "micro", "block"):
        np.testing.assert_array_equal(alone[key], comp[key])
    pay = _payloads(3, rows=5, L=2048, seed=83)
    zero = np.zeros((5, 2048), np.uint16)
    a = oracle.requantize(pay, local=zero, fwht=fwht)
    b = oracle.requantize(pay)
    for key in ("codes", "micro", "block"):
        np.testing.assert_array_equal(a[key], b[key])


def test_requantize_doubling_is_exact():
    """Two equal payloads sum to exactly twice one: same codes and micro-scales,
    twice the block scale."""
    pay = _payloads(1, seed=77)
    one = oracle.requantize(pay)
    two = oracle.requantize(pay + pay)
    np.testing.assert_array_equal(two["codes"], one["codes"])
    np.testing.assert_array_equal(two["micro"], one["micro"])
    np.testing.assert_array_equal(two["block"], 2 * one["block"])


def test_requantize_cancellation_gives_zero():
    """A payload plus its negation (sign bit of every code flipped) sums to +0."""
    (c, m, b), = _payloads(1, seed=91)
    neg = ((c ^ 0x88).astype(np.uint8), m, b)
    got = oracle.requantize([(c, m, b), neg])
    assert not got["codes"].any() and not got["micro"].any() and not got["block"].any()


def test_requantize_error_bound_and_meaning():
    """The re-quantised payload decodes (through the inverse transform) to the sum
    of the k decoded tensors, up to FP4 rounding of the transform-domain sum:
    per element at most half a grid step times S_g unless saturated."""
    pay = _payloads(8, rows=4, L=2048)
    got = oracle.requantize(pay, debug=True)
    y = _transform_domain_sum(pay).astype(np.float64).reshape(-1, 16, 16)
    yq = _dequant_f32(got["codes"], got["micro"], got["block"]).astype(np.float64).reshape(-1, 16, 16)
    S = (got["block"].reshape(-1, 1) * bf.E4M3_VALUES[got["micro"].reshape(-1, 16)]).astype(np.float64)
    v = got["v"].reshape(-1, 16, 16)
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0)) * S[:, :, None]
    unsat = np.abs(v) <= 6
    assert np.all(np.abs(yq - y)[unsat] <= 0.5 * step[unsat] * (1 + 1e-5) + 1e-30)
    # meaning: decompress(requantized) ~ sum of the peers' decompressed tensors
    ref = oracle.accumulate_f64(pay)
    dec = oracle.decompress_f64(got["codes"], got["micro"], got["block"])
    rel = np.linalg.norm(dec - ref) / np.linalg.norm(ref)
    assert rel < 0.2


U = 2.0 ** -24   # unit roundoff of binary32


def _exact_value(codes, micro, block):
    """A payload's exact value in binary64, by the format definition: E2M1 grid
    value x block scale x E4M3 value (2 + 24 + 4 significant bits: exact)."""
    c = unpack(codes).reshape(-1, 16, 16)
    mag = bf.E2M1_GRID[c & 7] * np.where(c & 8, -1.0, 1.0)
    S = np.asarray(block, np.float64).reshape(-1, 1) * bf.E4M3_VALUES[np.asarray(micro).reshape(-1, 16)]
    return (mag * S[:, :, None]).reshape(-1, 256)


@pytest.mark.parametrize("local", [False, True])
@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("k", [1, 3, 8])
def test_requantize_is_compress_of_the_exact_sum(k, fwht, local):
    """The plain definition of the reduce-scatter receiver: decompress every
    peer's payload exactly (binary64, its inverse transform a dense H/16), add
    the rank's own slice, and compress the sum -- transform (dense H/16 in
    binary64), block and micro-scales, E2M1 codes by nearest-code search.  The
    oracle computes the same in binary32 in the transform domain; its result
    must match wherever the exact value lies outside the band that binary32
    rounding can move it by.  Per element that band is at most
    (k + 3) u (sum over peers of |term| + |local term|) + 9 u sum_j |x_j| / 16
    (two roundings per decoded term, k + 1 additions, eight radix-2 stages of the
    local slice's transform), u = 2^-24, widened by 1 %; block scales, group
    maxima and quotients carry it into the micro-scale and code comparisons."""
    rows, L = 6, 1024
    pay, exact_terms = [], []
    for p in range(k):
        r = oracle.compress(inputs.make_normal(rows, L, seed=300 + p, scale=1e-3), fwht=fwht)
        pay.append((r["codes"], r["micro"], r["block"]))
        exact_terms.append(_exact_value(r["codes"], r["micro"], r["block"]))   # transform domain
    H = bf.H256.astype(np.float64) / 16.0
    T = (lambda z: z @ H.T) if fwht else (lambda z: z)
    signal = sum(T(t) for t in exact_terms)          # sum of the decompressed peers (H/16 self-inverse)
    xb = inputs.make_normal(rows, L, seed=399, scale=1e-3) if local else None
    if local:
        signal = signal + oracle.widen(xb).astype(np.float64).reshape(-1, 256)
    y = T(signal)                                    # compress: the transform of the exact sum
    got = oracle.requantize(pay, local=xb, fwht=fwht, debug=True)

    # the binary32 band
    mag = sum(np.abs(t) for t in exact_terms)
    E = (k + 3) * U * mag
    if local:
        xl = np.abs(oracle.widen(xb).astype(np.float64).reshape(-1, 256))
        E = E + (k + 3) * U * np.abs(T(oracle.widen(xb).astype(np.float64).reshape(-1, 256)))
        E = E + (9 * U * xl.sum(axis=1, keepdims=True) / 16.0 if fwht else 0.0)
    E = 1.01 * E

    A = np.abs(y).max(axis=1)
    EA = E.max(axis=1)
    s = A / 2688.0
    np.testing.assert_array_less(np.abs(got["block"].reshape(-1) - s), EA / 2688.0 + 2 * U * s + 1e-300)
    yg, Eg = np.abs(y).reshape(-1, 16, 16), E.reshape(-1, 16, 16)
    a = yg.max(axis=2)
    t = a / (6.0 * s[:, None])
    rel_t = Eg.max(axis=2) / np.maximum(a, 1e-300) + EA[:, None] / A[:, None] + 4 * U
    m = bf.nearest_e4m3(t)
    mids = bf.e4m3_midpoints()
    idx = np.clip(np.searchsorted(mids, t), 1, len(mids) - 1)
    dmid = np.minimum(np.abs(t - mids[idx - 1]), np.abs(t - mids[idx]))
    near_m = dmid <= rel_t * t + 1e-6 * t
    gm = got["micro"].reshape(-1, 16)
    assert np.all((gm == m) | near_m), "micro-scales differ away from a midpoint"
    S = s[:, None] * bf.E4M3_VALUES[m]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(S[:, :, None] > 0, y.reshape(-1, 16, 16) / S[:, :, None], 0.0)
        dv = np.where(S[:, :, None] > 0, np.abs(v) * (EA[:, None, None] / A[:, None, None] + 4 * U)
                      + Eg / S[:, :, None], 0.0)
    want = bf.nearest_e2m1(v).reshape(-1, 256)
    bnd = bf.e2m1_boundaries()
    av = np.abs(v).reshape(-1, 256)
    idx = np.clip(np.searchsorted(bnd, av), 1, len(bnd) - 1)
    dist = np.minimum(np.abs(av - bnd[idx - 1]), np.abs(av - bnd[idx]))
    near_c = (dist <= dv.reshape(-1, 256) + 1e-6 * av) | np.repeat(near_m | (gm != m), 16, axis=1)
    gc = unpack(got["codes"]).reshape(-1, 256)
    # a zero exact value may come out as a rounded residue of either sign
    ok = (gc == want) | near_c | (((gc & 7) == 0) & ((want & 7) == 0))
    assert np.all(ok), "codes differ away from a rounding boundary"
    assert near_c.mean() < 0.01, "the binary32 band exempts too much to pin anything"


def test_requantize_sums_in_peer_order_from_zero():
    """Peers are added to a +0 accumulator in order p = 0 .. k-1: a payload
    followed by its negation cancels exactly (x + (-x) = +0), so [P, -P, Q]
    re-quantises bit for bit as [Q] alone -- in any other order the large terms
    of P would round away part of Q's small ones."""
    big = oracle.compress(inputs.make_normal(6, 1024, seed=501))
    small = oracle.compress(inputs.make_normal(6, 1024, seed=502, scale=1e-5))
    P = (big["codes"], big["micro"], big["block"])
    negP = ((big["codes"] ^ 0x88).astype(np.uint8), big["micro"], big["block"])
    Q = (small["codes"], small["micro"], small["block"])
    a = oracle.requantize([P, negP, Q])
    b = oracle.requantize([Q])
    for key in ("codes", "micro", "block"):
        np.testing.assert_array_equal(a[key], b[key])
    # the same three peers in reverse order do not cancel exactly
    c = oracle.requantize([Q, negP, P])
    assert any(not np.array_equal(c[key], b[key]) for key in ("codes", "micro", "block"))
