"""Pins of the oracle's fast Walsh-Hadamard transform.

What the pages fix (BitNet v2 write-up, section H-BitLinear模塊): the transform is a
matrix product with a Hadamard matrix, every entry is +1 or -1, rows are mutually
orthogonal, and it is computed by the fast Hadamard transform in O(n log n).  The checks
below compare the oracle with SciPy's Sylvester-construction Hadamard matrix (a library
routine), with closed forms, and with the defining properties.
"""
import numpy as np
import pytest
import scipy.linalg

pytestmark = pytest.mark.filterwarnings("ignore")

SIZES = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("n", SIZES)
def test_matrix_entries_pm1_and_orthogonal_rows(orc, n):
    # The transform of the identity's rows is the matrix itself (it is symmetric).
    H = orc.fwht_f64(np.eye(n))
    assert set(np.unique(H)).issubset({-1.0, 1.0})
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))


@pytest.mark.parametrize("n", SIZES)
def test_fwht_equals_sylvester_matmul_exact_on_integers(orc, n):
    rng = np.random.default_rng(n)
    x = rng.integers(-1000, 1001, size=(5, n)).astype(np.float32)
    want = x.astype(np.float64) @ scipy.linalg.hadamard(n).T.astype(np.float64)
    np.testing.assert_array_equal(orc.fwht_f32(x).astype(np.float64), want)
    np.testing.assert_array_equal(orc.fwht_f64(x), want)


@pytest.mark.parametrize("n", [64, 256])
def test_fwht_f32_close_to_sylvester_on_gaussian(orc, n):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((8, n)).astype(np.float32)
    want = x.astype(np.float64) @ scipy.linalg.hadamard(n).T
    got = orc.fwht_f32(x).astype(np.float64)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 1e-6


def test_involution(orc):
    rng = np.random.default_rng(3)
    for n in [16, 1024, 16384]:
        x = rng.integers(-50, 51, size=n).astype(np.float32)
        np.testing.assert_array_equal(orc.fwht_f32(orc.fwht_f32(x)), n * x)


def test_special_vectors(orc):
    for n in [2, 128, 4096]:
        e0 = np.zeros(n, np.float32)
        e0[0] = 1
        np.testing.assert_array_equal(orc.fwht_f32(e0), np.ones(n, np.float32))
        np.testing.assert_array_equal(orc.fwht_f32(np.ones(n, np.float32)), n * e0)
        # the last basis vector maps to the last (alternating-parity) row of H
        el = np.zeros(n, np.float32)
        el[-1] = 1
        signs = np.array([(-1) ** bin(j & (n - 1)).count("1") for j in range(n)], np.float32)
        np.testing.assert_array_equal(orc.fwht_f32(el), signs)


def test_parseval(orc):
    rng = np.random.default_rng(11)
    for n in [512, 16384]:
        x = rng.standard_normal(n)
        z = orc.fwht_f64(x)
        assert abs(np.dot(z, z) - n * np.dot(x, x)) <= 1e-10 * n * np.dot(x, x)


def test_fwht_f32_deviation_from_fp64_is_small_at_16384(orc):
    # The fp32 butterfly that decides the codes stays within a few ulps of the fp64 transform.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 16384)).astype(np.float32)
    z32 = orc.fwht_f32(x).astype(np.float64)
    z64 = orc.fwht_f64(x.astype(np.float64))
    scale = np.abs(z64).max(axis=1, keepdims=True)
    assert (np.abs(z32 - z64) / scale).max() < 14 * 2.0 ** -23


def test_fwht_f32_stage_order_hand_case(orc):
    """The fp32 transform runs its stages in ascending order (h = 1, 2, ...).  A 4-point case
    where the order shows (derived by hand; 1 + 2^-24 is a tie that rounds to 1):
      x = [1, 2^-24, 2^-24, 0]
      h = 1: [fl(1 + 2^-24), 1 - 2^-24, 2^-24, 2^-24] = [1, 1 - 2^-24, 2^-24, 2^-24]
      h = 2: [fl(1 + 2^-24), fl(1 - 2^-24 + 2^-24), 1 - 2^-24, 1 - 2^-23] = [1, 1, 1 - 2^-24, 1 - 2^-23]
    (descending order gives [1, 1 - 2^-24, 1, 1 - 2^-23])."""
    x = np.array([1.0, 2.0 ** -24, 2.0 ** -24, 0.0], np.float32)
    z = orc.fwht_f32(x)
    assert list(z.view(np.uint32)) == [0x3F800000, 0x3F800000, 0x3F7FFFFF, 0x3F7FFFFE]
