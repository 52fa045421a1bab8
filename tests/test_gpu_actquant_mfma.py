"""The activation kernel whose first five transform stages run on the bf16 matrix cores (bf16
rows, unit gamma, K = 2^10 .. 2^14) against the oracle.

The stages and the sums of the matrix products run in another order than the oracle's fp32
butterfly loop, so z agrees up to fp32 rounding: the codes meet the method's code bar (at
most 1e-4 of them differ, each by one step), deq (which also takes an fp32 sum of squares)
is within a few ulp, and rows whose transform is exact (integer values, |z| < 2^24) give
identical codes and deq.  The cases cover every K, both code widths, with and without
RMSNorm, rows that fill several slabs plus a ragged last one, zero rows and rows below the
2^-120 guard."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import DEQ_ULPS_MFMA, assert_close_ulps, assert_code_bar, note, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("L", [10, 11, 12, 13, 14])
@pytest.mark.parametrize("abits", [4, 8])
@pytest.mark.parametrize("norm", [True, False])
def test_codes_and_deq(orc, L, abits, norm):
    K = 1 << L
    R = 16384 // K                        # rows per slab
    M = (1 << 21) // K + R // 2 + 1       # about 2M codes; a ragged last slab
    note("actquant mfma", K, abits, norm, M)
    x = inputs.make_activations("mixture", M, K, seed=100 + L, outlier_frac=0.01, outlier_scale=50.0)
    q, deq, _ = orc.quantize_activations(x, abits, True, norm=norm)
    codes, deq_d = B.quantize_activations(to_dev(x), abits, True, norm=norm)
    assert_code_bar(orc, to_host(codes), q, K, abits, f"K={K} a{abits} norm={norm}")
    dd = to_host(deq_d)
    ulps = np.abs(dd.astype(np.float64) - deq) / (np.abs(deq.astype(np.float64)) * 2.0 ** -23)
    note(f"deq: max {ulps.max():.1f} ulp")
    assert_close_ulps(dd, deq, DEQ_ULPS_MFMA, "deq")


@pytest.mark.parametrize("L", [10, 12, 14])
def test_zero_and_tiny_rows(orc, L):
    K = 1 << L
    M = 2 * (16384 // K) + 3
    note("actquant mfma zero rows", K, M)
    x = inputs.make_activations("normal", M, K, seed=L, outlier_frac=0.01, outlier_scale=30.0)
    x[1] = 0                                                       # zero row
    x[2] = 0
    x[2, 0] = inputs.f32_to_bf16_bits(np.array([2.0 ** -126], np.float32))[0]   # max |z| below 2^-120
    x[3] = 0
    x[3, 0] = inputs.f32_to_bf16_bits(np.array([2.0 ** -119], np.float32))[0]   # max |z| above it
    x[M - 1] = 0
    x[M - 2, :] = 0
    x[M - 2, 7] = inputs.f32_to_bf16_bits(np.array([-3.0], np.float32))[0]   # one nonzero element
    for abits in (4, 8):
        q, deq, _ = orc.quantize_activations(x, abits, True, norm=False)
        codes, deq_d = B.quantize_activations(to_dev(x), abits, True, norm=False)
        got = orc.unpack_codes(to_host(codes), K, abits)
        dd = to_host(deq_d)
        for r in (1, 2, M - 1):
            assert not got[r].any() and dd[r] == 0.0
        # a single nonzero element: |z| equal everywhere, every code +-Qb, exactly
        for r in (3, M - 2):
            np.testing.assert_array_equal(got[r], q[r])
            np.testing.assert_array_equal(dd[r], deq[r])
            assert np.all(np.abs(got[r]) == (7 if abits == 4 else 127))
        assert_code_bar(orc, to_host(codes), q, K, abits, "rows")
        assert_close_ulps(dd, deq, DEQ_ULPS_MFMA, "deq")


@pytest.mark.parametrize("L", [11, 13, 14])
def test_deterministic_and_independent_of_batch(orc, L):
    """The same rows give the same codes alone, at another offset in the batch, and twice."""
    K = 1 << L
    M = 40
    note("actquant mfma batch", K)
    x = inputs.make_activations("mixture", M, K, seed=L, outlier_frac=0.01, outlier_scale=50.0)
    c_all, d_all = B.quantize_activations(to_dev(x), 4, True, norm=True)
    c_again, d_again = B.quantize_activations(to_dev(x), 4, True, norm=True)
    c_tail, d_tail = B.quantize_activations(to_dev(np.ascontiguousarray(x[7:])), 4, True, norm=True)
    np.testing.assert_array_equal(to_host(c_all), to_host(c_again))
    np.testing.assert_array_equal(to_host(d_all), to_host(d_again))
    np.testing.assert_array_equal(to_host(c_all)[7:], to_host(c_tail))
    np.testing.assert_array_equal(to_host(d_all)[7:], to_host(d_tail))
