"""Pins of the oracle's integer GEMM, dequantisation, SwiGLU and packed formats.

The integer product is checked against numpy's integer matmul (a library routine) and
against special weight matrices with known products; the packed formats against bytes
derived by hand from the documented bit positions (tests/golden/packing.json).
"""
import json
import os

import numpy as np
import pytest
import scipy.special

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 16, 5), (17, 64, 9), (64, 300, 33)])
def test_gemm_vs_numpy_integer_matmul(orc, M, K, N):
    rng = np.random.default_rng(M * 1000 + N)
    q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    want = q.astype(np.int64) @ T.astype(np.int64).T
    np.testing.assert_array_equal(orc.gemm_s32(q, T), want)


def test_gemm_special_weights(orc):
    rng = np.random.default_rng(0)
    M, K = 7, 128
    q = rng.integers(-8, 8, size=(M, K)).astype(np.int8)
    ones = np.ones((1, K), np.int8)
    np.testing.assert_array_equal(orc.gemm_s32(q, ones)[:, 0], q.astype(np.int64).sum(axis=1))
    onehot = np.zeros((K, K), np.int8)
    onehot[np.arange(K), np.arange(K)] = 1
    np.testing.assert_array_equal(orc.gemm_s32(q, onehot), q)
    np.testing.assert_array_equal(orc.gemm_s32(q, -onehot), -q.astype(np.int32))


def test_dequant_association(orc):
    acc = np.array([[3, -5, 1 << 20]], np.int32)
    deq = np.array([0.1], np.float32)
    y = orc.dequant(acc, deq, 0.3)
    # fl32(fl32(acc*deq)*alpha), exactly two float32 roundings, left to right
    for j in range(3):
        want = np.float32(np.float32(np.float32(acc[0, j]) * deq[0]) * np.float32(0.3))
        assert y[0, j] == want


def test_dequant_association_hand_case(orc):
    """A case where the order of the two roundings shows (derived by hand; ulp(3) = 2^-22).
    acc = 3, deq = alpha = 1 + 2^-23:
      left to right: fl(3 deq) = 3 + 1.5 ulp -> tie, to even -> 3 + 2 ulp;
                     fl((3 + 2 ulp) alpha) = 3 + 3.5 ulp + 2^-44 -> 3 + 4 ulp = 3 + 2^-20 (0x40400004)
      scales first:  fl(deq alpha) = 1 + 2^-22;  3 (1 + 2^-22) = 3 + 3 ulp (0x40400003)"""
    one_ulp = np.array([0x3F800001], np.uint32).view(np.float32)
    y = orc.dequant(np.array([[3]], np.int32), one_ulp, float(one_ulp[0]))
    assert y.view(np.uint32)[0, 0] == 0x40400004


def test_swiglu_vs_scipy_expit(orc):
    rng = np.random.default_rng(1)
    g = (rng.standard_normal(10000) * 4).astype(np.float32)
    u = rng.standard_normal(10000).astype(np.float32)
    want = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u.astype(np.float64)
    np.testing.assert_allclose(orc.swiglu(g, u), want, rtol=1e-6, atol=1e-30)


def test_weight_packing_fixture(orc):
    data = json.load(open(os.path.join(GOLDEN, "packing.json")))
    for case in data["weights"]:
        t = np.array([case["t"]], np.int8)
        Wq = orc.pack_weights(t)
        assert list(Wq[0]) == case["bytes"], case["note"]
        np.testing.assert_array_equal(orc.unpack_weights(Wq, 16), t)


def test_code_packing_fixture(orc):
    data = json.load(open(os.path.join(GOLDEN, "packing.json")))
    for case in data["codes4"]:
        q = np.array([case["q"]], np.int8)
        b = orc.pack_codes(q, 4)
        assert list(b[0]) == case["bytes"], case["note"]
        np.testing.assert_array_equal(orc.unpack_codes(b, 16, 4), q)


@pytest.mark.parametrize("abits", [4, 8])
def test_packing_round_trip(orc, abits):
    rng = np.random.default_rng(abits)
    Qb = 7 if abits == 4 else 127
    q = rng.integers(-Qb - 1, Qb + 1, size=(9, 256)).astype(np.int8)
    np.testing.assert_array_equal(orc.unpack_codes(orc.pack_codes(q, abits), 256, abits), q)
    T = rng.integers(-1, 2, size=(9, 256)).astype(np.int8)
    Wq = orc.pack_weights(T)
    assert Wq.shape == (9, 64)
    np.testing.assert_array_equal(orc.unpack_weights(Wq, 256), T)


def _fp6_value(code: int) -> float:
    """FP6 E2M3 value from its definition (independent of the oracle's encoder)."""
    s = -1.0 if code & 0x20 else 1.0
    e, m = (code >> 3) & 3, code & 7
    return s * (m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 8.0))


def _fp4_value(code: int) -> float:
    s = -1.0 if code & 8 else 1.0
    e, m = (code >> 1) & 3, code & 1
    return s * (m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0))


def test_fp6_fp4_fixture(orc):
    data = json.load(open(os.path.join(GOLDEN, "fp6_fp4_codes.json")))
    for q, code in data["fp6_e2m3"].items():
        assert _fp6_value(code) == int(q)
        packed = orc.pack_codes_fp6(np.full((1, 4), int(q), np.int8))
        assert packed[0, 0] & 63 == code
    row = data["fp6_row"]
    b = orc.pack_codes_fp6(np.array([row["q"]], np.int8))
    assert b.tobytes().hex() == row["bytes_hex"]
    for t, code in data["fp4_e2m1"].items():
        assert _fp4_value(code) == int(t)
    row = data["fp4_row"]
    assert orc.pack_weights_fp4(np.array([row["t"]], np.int8)).tobytes().hex() == row["bytes_hex"]


def test_fp6_round_trip_and_decoded_values(orc):
    rng = np.random.default_rng(6)
    q = rng.integers(-7, 8, size=(5, 256)).astype(np.int8)
    b = orc.pack_codes_fp6(q)
    assert b.shape == (5, 192)
    np.testing.assert_array_equal(orc.unpack_codes_fp6(b, 256), q)
    bits = np.unpackbits(b, axis=1, bitorder="little").reshape(5, 256, 6)
    codes = (bits * (1 << np.arange(6))).sum(axis=2)
    np.testing.assert_array_equal(np.vectorize(_fp6_value)(codes), q.astype(np.float64))
    T = rng.integers(-1, 2, size=(3, 128)).astype(np.int8)
    w = orc.pack_weights_fp4(T)
    nib = np.stack([w & 15, w >> 4], axis=2).reshape(3, 128)
    np.testing.assert_array_equal(np.vectorize(_fp4_value)(nib), T.astype(np.float64))
