"""Parity of the FP6 x FP4 a4 path (gfx950 scaled f8f6f4 matrix cores) against the oracle.

The path stores the same INT4 absmax codes as FP6 E2M3 and the ternary weights as FP4 E2M1;
every value is exact and the fp32 accumulation of integer products stays below 2^24, so the
codes, the int32 product and the outputs must equal the INT4 / 2-bit path bit for bit.  Against
the oracle the codes are bit-identical, or meet the code bar where the rows are transformed
partly on the matrix cores (bf16, unit gamma, K = 2^10 .. 2^14)."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import (DEQ_ULPS_MFMA, assert_close_ulps, assert_code_bar, assert_rows_close, check_codes,
                            mfma_transform, note, rel_fro, to_dev, to_host)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K", [(3, 64), (257, 1024), (64, 16384)])
def test_weights_to_fp4(orc, N, K):
    note("weights fp4", N, K)
    W = inputs.make_weights(N, K, seed=N)
    T, _ = orc.quantize_weights(W)
    Wq, _ = B.quantize_weights(to_dev(W))
    np.testing.assert_array_equal(to_host(B.weights_to_fp4(Wq, K)), orc.pack_weights_fp4(T))


@pytest.mark.parametrize("L", [6, 8, 9, 11, 12, 13, 14, 15])
def test_actquant_fp6_codes(orc, L):
    K = 1 << L
    M = max(1, 256 // max(K // 64, 1)) + 3 if K <= 16384 else 5
    M = min(M, 300)
    note("actquant fp6", K, M)
    x = inputs.make_activations("mixture", M, K, seed=L, outlier_frac=0.01, outlier_scale=50.0)
    q, deq, _ = orc.quantize_activations(x, 4, True, norm=True)
    codes, deq_d = B.quantize_activations_fp6(to_dev(x), True, norm=True)
    if mfma_transform(x, K, True):
        # the same codes as the INT4 call on the same rows, and the code bar against the oracle
        c4, d4 = B.quantize_activations(to_dev(x), 4, True, norm=True)
        q4 = orc.unpack_codes(to_host(c4), K, 4)
        np.testing.assert_array_equal(to_host(codes), orc.pack_codes_fp6(q4))
        np.testing.assert_array_equal(to_host(deq_d), to_host(d4))
        assert_code_bar(orc, to_host(c4), q, K, 4, "fp6 codes")
        assert_close_ulps(to_host(deq_d), deq, DEQ_ULPS_MFMA, "deq")
    else:
        np.testing.assert_array_equal(to_host(codes), orc.pack_codes_fp6(q))
        assert_close_ulps(to_host(deq_d), deq, 2, "deq")


@pytest.mark.parametrize("K", [64, 4096, 4160])
def test_actquant_fp6_plain(orc, K):
    note("actquant fp6 plain", K)
    x = inputs.make_activations("normal", 9, K, seed=K, outlier_frac=0.01, outlier_scale=30.0)
    q, deq, _ = orc.quantize_activations(x, 4, False, norm=False)
    codes, deq_d = B.quantize_activations_fp6(to_dev(x), False, norm=False)
    np.testing.assert_array_equal(to_host(codes), orc.pack_codes_fp6(q))
    np.testing.assert_array_equal(to_host(deq_d), deq)


# K = 64, 320, 576: partial last stage (masked loads); the others fill every 128-deep stage.
# An odd number of stages (K = 64, 320, 576, 1152) ends on the loop's peeled last stage.
# (3100, *, 4000/4001) runs 256 x 256 tiles, loaded straight into LDS when K fills every stage
# (1, 3 and 10 stages through the three buffers); the others 128 x 128, and (64, 16384, 64),
# (128, 16384, 1024) and (300, 8320, 520) split K (the last with a partial last stage in its
# last split).
@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (200, 320, 136), (129, 1024, 257), (64, 16384, 64),
                                   (2500, 576, 2200), (2500, 1152, 2200), (2100, 64, 2060), (2100, 256, 2060),
                                   (2100, 384, 2060), (3100, 64, 4000), (3100, 128, 4000), (3100, 384, 4000),
                                   (3100, 1280, 4001), (128, 16384, 1024), (300, 8320, 520)])
def test_gemm_fp6fp4_s32(orc, M, K, N):
    note("gemm fp6fp4", M, K, N)
    rng = np.random.default_rng(M + N)
    q = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = to_host(B.gemm_fp6fp4_s32(to_dev(orc.pack_codes_fp6(q)), to_dev(orc.pack_weights_fp4(T)), K))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


def test_gemm_fp6fp4_extremes(orc):
    M, K, N = 40, 8192, 72
    note("gemm fp6fp4 extremes")
    q = np.full((M, K), 7, np.int8)
    q[1::2] = -7
    T = np.ones((N, K), np.int8)
    T[::3] = -1
    acc = to_host(B.gemm_fp6fp4_s32(to_dev(orc.pack_codes_fp6(q)), to_dev(orc.pack_weights_fp4(T)), K))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


@pytest.mark.parametrize("name,M", [("tiny_exact", None), ("wo_1p3b", 64), ("wdown_7b", 24)])
def test_forward_fp6fp4_matches_int4_path(orc, name, M):
    wl = inputs.WORKLOADS[name]
    note("forward fp6fp4", name, M)
    x = wl.activations(M)
    W = wl.weights()
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    Wq4 = B.weights_to_fp4(Wq, wl.K)
    xd = to_dev(x)
    y6 = to_host(B.forward_fp6fp4(xd, Wq4, scale, wl.use_hadamard, norm=wl.norm))
    y4 = to_host(B.forward(xd, Wq, scale, 4, wl.use_hadamard, norm=wl.norm))
    np.testing.assert_array_equal(y6, y4)
    y_o, q_o, _, _ = orc.forward(x, T, alpha, 4, wl.use_hadamard, norm=wl.norm, intermediates=True)
    if name == "tiny_exact":
        np.testing.assert_array_equal(y6, y_o)
    else:
        codes, _ = B.quantize_activations(xd, 4, wl.use_hadamard, norm=wl.norm)
        exact = not mfma_transform(x, wl.K, wl.use_hadamard)
        rows_ok = check_codes(orc, to_host(codes), q_o, wl.K, 4, exact, name)
        assert_rows_close(y6, y_o, rows_ok, exact, name)


def test_forward_fp6fp4_full_size_sampled_rows(orc):
    wl = inputs.WORKLOADS["wdown_7b"]
    note("forward fp6fp4 full size")
    x = wl.activations()
    W = wl.weights()
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    Wq4 = B.weights_to_fp4(Wq, wl.K)
    xd = to_dev(x)
    y = to_host(B.forward_fp6fp4(xd, Wq4, scale, True, norm=True))
    # every row equals the INT4 path's (whose every row the full-size forward test holds to
    # the oracle), and sampled rows meet the oracle directly
    np.testing.assert_array_equal(y.view(np.int32), to_host(B.forward(xd, Wq, scale, 4, True, norm=True)).view(np.int32))
    rows = np.unique(np.concatenate([np.random.default_rng(7).choice(wl.M, 30, replace=False), [0, wl.M - 1]]))
    xs = np.ascontiguousarray(x[rows])
    y_o, q_o, _, _ = orc.forward(xs, T, alpha, 4, True, norm=True, intermediates=True)
    codes, _ = B.quantize_activations(to_dev(xs), 4, True, norm=True)
    rows_ok = check_codes(orc, to_host(codes), q_o, wl.K, 4, False, "wdown_7b fp6fp4 codes")
    assert_rows_close(y[rows], y_o, rows_ok, False, "wdown_7b fp6fp4")


@pytest.mark.parametrize("M", [16, 300])
def test_gemm_fp6fp4_max_k(orc, M):
    """K = HBL_MAX_K (131072) at the extreme INT4 codes: fp32 partial sums stay exact integers."""
    K, N = 131072, 40
    note("fp6fp4 max K", M)
    q = np.full((M, K), -7, np.int8)
    q[1::3, ::5] = 7
    T = np.ones((N, K), np.int8)
    T[1::2] = -1
    T[::3, ::7] = 0
    acc = to_host(B.gemm_fp6fp4_s32(to_dev(orc.pack_codes_fp6(q)), to_dev(orc.pack_weights_fp4(T)), K))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


@pytest.mark.parametrize("use_h,K", [(True, 4096), (False, 2112)])
def test_forward_fp6fp4_fp32_gamma_matches_int4_path(orc, use_h, K):
    """fp32 input with RMSNorm and a per-channel gamma, with and without the transform (the
    plain path at a K that is no power of two): bit-identical to the INT4 path, and the
    oracle's bar."""
    M, N = 300, 200
    note("forward fp6fp4 fp32 gamma", use_h, K)
    x = inputs.bf16_bits_to_f32(inputs.make_activations("mixture", M, K, seed=K, outlier_frac=0.01,
                                                        outlier_scale=40.0)) * np.float32(1.7)
    gamma = np.random.default_rng(K + 1).uniform(0.5, 1.5, K).astype(np.float32)
    W = inputs.make_weights(N, K, seed=3)
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    Wq4 = B.weights_to_fp4(Wq, K)
    xd, gd = to_dev(x), to_dev(gamma)
    y6 = to_host(B.forward_fp6fp4(xd, Wq4, scale, use_h, norm=True, gamma=gd))
    y4 = to_host(B.forward(xd, Wq, scale, 4, use_h, norm=True, gamma=gd))
    np.testing.assert_array_equal(y6, y4)
    y_o = orc.forward(x, T, alpha, 4, use_h, norm=True, gamma=gamma)
    assert rel_fro(y6, y_o) <= 1e-3
