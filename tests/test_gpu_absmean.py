"""Parity of the absmean statistic switch (HBL_STAT_ABSMEAN, INT4) against the oracle.

The statistic b = mean|z| is an fp64 sum whose order differs between the GPU (per thread,
then across threads) and the oracle (ascending); b can therefore differ by one ulp in rare
rows, which moves codes that sit exactly at a rounding boundary.  The bar: at most 1e-4 of
the codes differ, each by one; deq within 2 ulp; outputs within the method's bar."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import DEQ_ULPS_MFMA, assert_close_ulps, mfma_transform, note, rel_fro, to_dev, to_host

pytestmark = pytest.mark.gpu


def _codes_close(orc, got_packed, q_o, K):
    got = orc.unpack_codes(got_packed, K, 4).astype(np.int32)
    d = np.abs(got - q_o.astype(np.int32))
    assert d.max() <= 1, f"codes differ by {d.max()}"
    assert (d != 0).mean() <= 1e-4, f"{int((d != 0).sum())} of {d.size} codes differ"


@pytest.mark.parametrize("L", [6, 9, 10, 12, 13, 14, 15])
def test_absmean_hadamard(orc, L):
    K = 1 << L
    M = max(3, min(300, (1 << 20) // K))
    note("absmean H", K, M)
    x = inputs.make_activations("mixture", M, K, outlier_frac=0.01, outlier_scale=50.0, seed=L)
    x[1] = 0                                              # a zero row
    codes, deq = B.quantize_activations(to_dev(x), 4, True, norm=True, stat=B.HBL_STAT_ABSMEAN)
    q_o, deq_o, _ = orc.quantize_activations(x, 4, True, norm=True, stat=1)
    _codes_close(orc, to_host(codes), q_o, K)
    assert_close_ulps(to_host(deq), deq_o, DEQ_ULPS_MFMA if mfma_transform(x, K, True) else 2, "deq")


# K = 8192 and 16384 run the persistent row kernel with rows spread over two and four waves,
# where the absmean and sum-of-squares reductions each need their own slots.
@pytest.mark.parametrize("K", [64, 576, 4096, 8192, 16384, 20480])
@pytest.mark.parametrize("fmt", ["bf16", "bf16-gamma", "fp32-gamma"])
def test_absmean_plain(orc, K, fmt):
    note("absmean plain", K, fmt)
    M = 130
    x = inputs.make_activations("normal", M, K, outlier_frac=0.02, outlier_scale=40.0, seed=K)
    gamma = None
    if fmt != "bf16":
        gamma = np.random.default_rng(K).uniform(0.5, 2.0, K).astype(np.float32)
    if fmt == "fp32-gamma":
        x = inputs.bf16_bits_to_f32(x) * np.float32(0.5)
    codes, deq = B.quantize_activations(to_dev(x), 4, False, norm=True, gamma=None if gamma is None else to_dev(gamma),
                                        stat=B.HBL_STAT_ABSMEAN)
    q_o, deq_o, _ = orc.quantize_activations(x, 4, False, norm=True, gamma=gamma, stat=1)
    _codes_close(orc, to_host(codes), q_o, K)
    assert_close_ulps(to_host(deq), deq_o, 2, "deq")


def test_absmean_forward_7b_rows(orc):
    wl = inputs.WORKLOADS["wdown_7b"]
    note("absmean forward 7b")
    x = wl.activations(200)
    W = inputs.make_weights(wl.N, wl.K)
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    y = to_host(B.forward(to_dev(x), Wq, scale, 4, True, norm=True, stat=B.HBL_STAT_ABSMEAN))
    y_o = orc.forward(x, T, alpha, 4, True, norm=True, stat=1)
    assert rel_fro(y, y_o) <= 1e-3


@pytest.mark.parametrize("M", [1, 16, 64])
def test_absmean_forward_decode_rows(orc, M):
    """Few token rows: the decode GEMM multiplies absmean codes, whose range includes -8."""
    wl = inputs.WORKLOADS["wdown_7b"]
    note("absmean forward decode", M)
    x = wl.activations(M)
    W = inputs.make_weights(wl.N, wl.K)
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    ws = B.forward_workspace(M, wl.K, 4)
    y = to_host(B.forward(to_dev(x), Wq, scale, 4, True, norm=True, ws=ws, stat=B.HBL_STAT_ABSMEAN))
    y_o, q_o, _, _ = orc.forward(x, T, alpha, 4, True, norm=True, stat=1, intermediates=True)
    _codes_close(orc, to_host(ws[:M * wl.K // 2]).reshape(M, wl.K // 2), q_o, wl.K)
    assert rel_fro(y, y_o) <= 1e-3
