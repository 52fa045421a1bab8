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
