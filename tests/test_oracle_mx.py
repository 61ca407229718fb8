"""Pins of the oracle's MXFP4-style variant (32-element groups, E8M0 power-of-two
scales, no coarse scale), against independent numpy computations."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from tests.parity import unpack
from fp4_communication_compression_amd import inputs


def _brute(xb, fwht=True):
    x = inputs.bf16_bits_to_f32(xb).astype(np.float64).reshape(-1, 256)
    y = (x @ bf.H256.T) / 16.0 if fwht else x
    g = y.reshape(-1, 8, 32)
    amax = np.abs(g).max(axis=2)
    # smallest power of two 2^e with amax / 2^e < 8, i.e. e = floor(log2 amax) - 2
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    e = np.clip(e, -127, 127).astype(np.int64)
    v = g / np.exp2(e)[:, :, None]
    return e, v.reshape(-1, 256)


@pytest.mark.parametrize("fwht", [True, False])
def test_mx_against_brute_force(fwht):
    xb = inputs.make_normal(32, 1024, seed=61, scale=2.0)
    got = oracle.compress_mx(xb, fwht=fwht, debug=True)
    e, v = _brute(xb, fwht)
    np.testing.assert_array_equal(got["scales"].reshape(-1, 8).astype(np.int64) - 127, e)
    codes = bf.nearest_e2m1(v)
    gc = unpack(got["codes"]).reshape(-1, 256)
    near = bf.near(v, bf.e2m1_boundaries(), 1e-6)
    assert np.all((gc == codes) | near)
    # every group's largest element lands in [4, 8) before rounding
    assert np.all(np.abs(v).reshape(-1, 8, 32).max(axis=2)[e > -127] >= 4)
    assert np.all(np.abs(v) < 8)


def test_mx_spike_block_closed_form():
    """x = 16 e_0: y = 1 everywhere -> e = -2 (scale byte 125), v = 4 -> code 6
    (bytes 0x66); decoding gives exactly 16 e_0."""
    x = np.zeros(256, np.float32)
    x[0] = 16
    xb = inputs.f32_to_bf16_bits(x).reshape(1, 256)
    got = oracle.compress_mx(xb)
    assert np.all(got["scales"] == 125) and np.all(got["codes"] == 0x66)
    out = oracle.decompress_mx(got["codes"], got["scales"])
    np.testing.assert_array_equal(out[0], x)


def test_mx_zero_and_tiny_groups():
    xb = inputs.make_edge_case("zeros", 2, 512)
    got = oracle.compress_mx(xb)
    assert np.all(got["scales"] == 0) and not got["codes"].any()
    assert not oracle.decompress_mx(got["codes"], got["scales"]).any()
    xb = inputs.make_edge_case("tiny", 4, 512, seed=5)
    got = oracle.compress_mx(xb, fwht=False, debug=True)
    e, v = _brute(xb, fwht=False)
    np.testing.assert_array_equal(got["scales"].reshape(-1, 8).astype(np.int64) - 127, e)


def test_mx_decode_error_bound():
    """Transform-domain error at most half a grid step times 2^e (unsaturated)."""
    xb = inputs.make_config("outlier8192", rows=16)
    got = oracle.compress_mx(xb, debug=True)
    codes = unpack(got["codes"]).reshape(-1, 8, 32)
    e = got["scales"].reshape(-1, 8).astype(np.int64) - 127
    dec = bf.E2M1_GRID[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    y = oracle.fwht256(inputs.bf16_bits_to_f32(xb)).astype(np.float64).reshape(-1, 8, 32)
    v = got["v"].reshape(-1, 8, 32)
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    unsat = np.abs(v) <= 6
    err = np.abs(dec * np.exp2(e)[:, :, None] - y)
    assert np.all(err[unsat] <= 0.5 * (step * np.exp2(e)[:, :, None])[unsat] * (1 + 1e-6))
    # decompress = inverse transform of the dequantised values
    out = oracle.decompress_mx(got["codes"], got["scales"])
    ref = oracle.fwht256((dec * np.exp2(e)[:, :, None]).astype(np.float32).reshape(-1, 256))
    np.testing.assert_array_equal(out.reshape(-1, 256), ref)


def test_mx_payload_size():
    xb = inputs.make_normal(2, 1024, seed=1)
    got = oracle.compress_mx(xb)
    assert (got["codes"].nbytes + got["scales"].nbytes) * 8 == 4.25 * xb.size
