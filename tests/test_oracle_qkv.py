"""Pins of the oracle's unsigned absmax QKV quantiser and its b-bit packing.

Hand-derived fixtures (tests/golden/qkv_codes.json), the range ends (the largest positive
element maps to 2^b - 1 and the most negative to 0), the reconstruction error bound
|x - xhat| <= D/2, invariance under power-of-two scaling, and packing round trips.
"""
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_qkv_fixture(orc):
    data = json.load(open(os.path.join(GOLDEN, "qkv_codes.json")))
    for case in data["cases"]:
        u, g = orc.quantize_qkv(np.array([case["x"]], np.float32), case["bits"])
        assert list(u[0]) == case["codes"], case["note"]
        assert g[0] == np.float32(case["gamma"])
        assert orc.pack_bits(u, case["bits"]).tobytes().hex() == case["packed_hex"], case["note"]


def _heads(rows, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-3, 3, (rows, 1)))
    return x.astype(np.float32)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_qkv_range_ends_and_error_bound(orc, bits):
    x = _heads(300, 128, bits)
    u, g = orc.quantize_qkv(x, bits)
    L = (1 << bits) - 1
    assert u.max() <= L
    np.testing.assert_array_equal(g, np.abs(x).max(axis=1))
    rows = np.arange(x.shape[0])
    imax, imin = x.argmax(axis=1), x.argmin(axis=1)
    pos = x[rows, imax] == g
    neg = x[rows, imin] == -g
    assert (u[rows, imax][pos] == L).all()
    assert (u[rows, imin][neg] == 0).all()
    xh = orc.dequantize_qkv(u, g, bits)
    D = 2.0 * g.astype(np.float64) / L
    err = np.abs(x.astype(np.float64) - xh)
    assert (err <= D[:, None] * (0.5 + 1e-5)).all()
    # the mean error of a uniform quantiser is about D/4; a shifted grid would double it
    assert err.mean() / D.mean() < 0.3


def test_qkv_power_of_two_invariance(orc):
    x = _heads(64, 64, 9)
    u1, g1 = orc.quantize_qkv(x, 3)
    u2, g2 = orc.quantize_qkv(x * np.float32(2.0 ** -7), 3)
    np.testing.assert_array_equal(u1, u2)
    np.testing.assert_array_equal(g2, g1 * np.float32(2.0 ** -7))


def test_qkv_bf16_input_is_exact_widening(orc):
    rng = np.random.default_rng(3)
    bits16 = (rng.integers(0, 1 << 15, (20, 64)) | (rng.integers(0, 2, (20, 64)) << 15)).astype(np.uint16)
    bits16 = np.where((bits16 & 0x7F80) == 0x7F80, 0x3F80, bits16).astype(np.uint16)  # no inf/nan
    as_f32 = (bits16.astype(np.uint32) << 16).view(np.float32)
    ub, gb = orc.quantize_qkv(bits16, 4)
    uf, gf = orc.quantize_qkv(as_f32, 4)
    np.testing.assert_array_equal(ub, uf)
    np.testing.assert_array_equal(gb, gf)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_pack_bits_round_trip(orc, bits):
    rng = np.random.default_rng(bits)
    u = rng.integers(0, 1 << bits, (7, 64)).astype(np.uint8)
    p = orc.pack_bits(u, bits)
    assert p.shape == (7, 64 * bits // 8)
    np.testing.assert_array_equal(orc.unpack_bits(p, 64, bits), u)
    # every code's bits sit where the format says
    flat = np.unpackbits(p, axis=1, bitorder="little").reshape(7, 64, bits)
    np.testing.assert_array_equal((flat * (1 << np.arange(bits))).sum(axis=2), u)


def test_qkv_scale_guard_head_below_threshold(orc):
    """A head with g < 2^-120 takes s = 0: every code is rint_ne(c) = rint_ne(3.5) = 4 at 3 bits
    (without the guard, L / 2g is still finite here and the codes would span 0 .. 7)."""
    h = np.zeros((1, 32), np.float32)
    h[0, 0], h[0, 1] = 2.0 ** -121, -(2.0 ** -121)
    u, g = orc.quantize_qkv(h, 3)
    assert (u == 4).all() and g[0] == np.float32(2.0 ** -121)
