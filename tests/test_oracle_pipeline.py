"""Pins of the oracle's whole compress / decompress / accumulate pipeline."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from fp4_communication_compression_amd import inputs

f32 = np.float32


def _block(x_f32):
    return inputs.f32_to_bf16_bits(np.asarray(x_f32, np.float32)).reshape(1, 256)


def _unpack(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def test_zero_block():
    p = oracle.compress(_block(np.zeros(256)))
    assert not p["codes"].any() and not p["micro"].any() and p["block"][0, 0] == 0
    out = oracle.decompress(p["codes"], p["micro"], p["block"])
    assert not out.any()


def test_spike_block_closed_form():
    """x = 16 e_0: y = H x / 16 is all ones, so every group is the block maximum."""
    x = np.zeros(256)
    x[0] = 16
    p = oracle.compress(_block(x), debug=True)
    s = f32(1) / f32(2688)
    assert p["block"][0, 0].view(np.uint32) == s.view(np.uint32) == 0x39C30C31
    assert np.all(p["micro"] == 0x7E)                # t = 1 / fl(6 s) = 447.99997 -> 448
    assert np.all(p["t"] == f32(1) / (f32(6) * s))
    assert np.all(p["codes"] == 0x77)                # v = 1 / fl(448 s) = 6.0 -> code 7
    out = oracle.decompress(p["codes"], p["micro"], p["block"])
    want = np.zeros(256, np.float32)
    want[0] = 16.0                                   # 6 * fl(448 s) = 1.0 exactly, summed
    np.testing.assert_array_equal(out[0], want)


def test_constant_block_closed_form():
    """x = 1: y = 16 e_0, one nonzero group; the other 15 groups get scale 0."""
    p = oracle.compress(_block(np.ones(256)))
    assert p["block"][0, 0].view(np.uint32) == 0x3BC30C31   # 16 / 2688
    assert p["micro"][0, 0] == 0x7E and not p["micro"][0, 1:].any()
    assert p["codes"][0, 0] == 0x07 and not p["codes"][0, 1:].any()
    out = oracle.decompress(p["codes"], p["micro"], p["block"])
    np.testing.assert_array_equal(out[0], np.ones(256, np.float32))


@pytest.mark.parametrize("j", [3, 16, 100, 255])
def test_walsh_row_block(j):
    """x = Walsh row j: y = 16 e_j; the spike lands in group j // 16."""
    p = oracle.compress(_block(bf.H256[j]))
    g = j // 16
    assert p["micro"][0, g] == 0x7E and np.count_nonzero(p["micro"]) == 1
    codes = _unpack(p["codes"])[0]
    assert codes[j] == 7 and np.count_nonzero(codes) == 1
    out = oracle.decompress(p["codes"], p["micro"], p["block"])
    np.testing.assert_array_equal(out[0], bf.H256[j].astype(np.float32))


def _brute_force_payload(xb, fwht=True):
    """Whole-pipeline brute force: dense Hadamard in binary64, exhaustive nearest
    E4M3 and E2M1 search.  Returns (codes per element, micro, block, t, v)."""
    x = inputs.bf16_bits_to_f32(xb).astype(np.float64).reshape(-1, 256)
    y = (x @ bf.H256.T) / 16.0 if fwht else x
    A = np.abs(y).max(axis=1)
    s = A / 2688.0
    a = np.abs(y).reshape(-1, 16, 16).max(axis=2)
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(s[:, None] > 0, a / (6.0 * s[:, None]), 0.0)
    m = bf.nearest_e4m3(t)
    S = s[:, None] * bf.E4M3_VALUES[m]
    with np.errstate(invalid="ignore", divide="ignore"):
        v = np.where(S[:, :, None] > 0, y.reshape(-1, 16, 16) / S[:, :, None], 0.0 * y.reshape(-1, 16, 16))
    codes = bf.nearest_e2m1(v).reshape(-1, 256)
    return codes, m, s, t, v.reshape(-1, 256)


@pytest.mark.parametrize("fwht", [True, False])
def test_tiny_config_against_brute_force(fwht):
    """The Tiny workload (4 x 256, N(0,1), seed 0) recomputed by brute force.

    The brute force works in binary64 and divides, so it may legitimately differ
    where a pre-rounding value sits within 1e-6 of a rounding boundary; anywhere
    else every byte must agree."""
    xb = inputs.make_config("tiny")
    p = oracle.compress(xb, fwht=fwht, debug=True)
    codes, m, s, t, v = _brute_force_payload(xb, fwht)
    np.testing.assert_allclose(p["block"].reshape(-1), s, rtol=1e-6)
    near_m = bf.near(t, bf.e4m3_midpoints(), 1e-6)
    assert np.all((p["micro"].reshape(-1, 16) == m) | near_m)
    got = _unpack(p["codes"]).reshape(-1, 256)
    near_c = bf.near(v, bf.e2m1_boundaries(), 1e-6) | np.repeat(near_m, 16, axis=1)
    assert np.all((got == codes) | near_c)
    assert np.count_nonzero(got != codes) <= 2


def test_larger_random_against_brute_force():
    xb = inputs.make_normal(64, 512, seed=5, scale=3.0)
    p = oracle.compress(xb, debug=True)
    codes, m, s, t, v = _brute_force_payload(xb)
    near_m = bf.near(t, bf.e4m3_midpoints(), 1e-6)
    assert np.all((p["micro"].reshape(-1, 16) == m) | near_m)
    got = _unpack(p["codes"]).reshape(-1, 256)
    near_c = bf.near(v, bf.e2m1_boundaries(), 1e-6) | np.repeat(near_m, 16, axis=1)
    assert np.all((got == codes) | near_c)


def test_invariants_on_outlier_workload():
    xb = inputs.make_config("outlier8192", rows=64)
    p = oracle.compress(xb, debug=True)
    micro = p["micro"].reshape(-1, 16)
    t = p["t"].reshape(-1, 16)
    # the group holding the block maximum gets the largest micro-scale 448
    assert np.all(micro[np.arange(len(t)), np.argmax(t, axis=1)] == 0x7E)
    # encoders are monotone: larger t never gets a smaller micro-scale in a block
    order = np.argsort(t, axis=1)
    assert np.all(np.diff(np.take_along_axis(micro.astype(int), order, 1), axis=1) >= 0)
    # with a normal micro-scale, |v| <= 6 * 16/15 (E4M3 rounds t by at most 1/16)
    v = p["v"].reshape(-1, 16, 16)
    normal = micro >= 0x08
    assert np.abs(v)[normal].max() <= 6.4 * (1 + 1e-6)
    # codes carry the sign of v
    codes = _unpack(p["codes"]).reshape(-1, 16, 16)
    assert np.all((codes >= 8) == np.signbit(v))
    # per element error after dequantisation: at most half a grid step (times S_g)
    # unless the value saturated
    y = oracle.fwht256(inputs.bf16_bits_to_f32(xb)).reshape(-1, 16, 16)
    S = (p["block"].reshape(-1, 1) * np.vectorize(oracle.e4m3_decode)(micro)).astype(np.float64)
    yq = np.vectorize(oracle.e2m1_decode)(codes) * S[:, :, None]
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0)) * S[:, :, None]
    unsat = np.abs(v) <= 6
    err = np.abs(yq - y)
    assert np.all(err[unsat] <= 0.5 * step[unsat] * (1 + 1e-5) + 1e-30)


def test_decompress_f32_agrees_with_f64():
    xb = inputs.make_config("act2048", rows=32)
    p = oracle.compress(xb)
    a = oracle.decompress(p["codes"], p["micro"], p["block"])
    b = oracle.decompress_f64(p["codes"], p["micro"], p["block"])
    rowmax = np.abs(b).max(axis=1)
    assert np.all(np.abs(a - b).max(axis=1) <= 1e-6 * rowmax)


def test_accumulate_properties():
    peers = [inputs.make_reduce_peer(p, rows=8, row_len=1024) for p in range(4)]
    pay = [oracle.compress(x) for x in peers]
    tr = [(p["codes"], p["micro"], p["block"]) for p in pay]
    one = oracle.accumulate_f64(tr[:1])
    np.testing.assert_array_equal(one, oracle.decompress_f64(*tr[0]))
    two = oracle.accumulate_f64([tr[0], tr[0]])
    np.testing.assert_array_equal(two, 2.0 * one)
    fwd = oracle.accumulate_f64(tr)
    rev = oracle.accumulate_f64(tr[::-1])
    np.testing.assert_allclose(fwd, rev, rtol=0, atol=1e-15 * np.abs(fwd).max())
    s32 = sum(oracle.decompress(*t).astype(np.float64) for t in tr)
    assert np.all(np.abs(s32 - fwd).max(axis=1) <= 1e-6 * np.abs(fwd).max(axis=1))


def test_payload_size_closed_form():
    """4 bits per element + one byte per 16 + four bytes per 256 = 4.625 bits."""
    xb = inputs.make_normal(2, 1024, seed=1)
    p = oracle.compress(xb)
    n = xb.size
    nbytes = p["codes"].nbytes + p["micro"].nbytes + p["block"].nbytes
    assert nbytes * 8 == 4.625 * n
    assert abs(2 * n / nbytes - 3.4595) < 1e-4
