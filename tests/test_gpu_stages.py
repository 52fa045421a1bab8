"""Stage-wise parity of the HIP kernels against the CPU oracle, through the C ABI.

Integer results (packed ternary weights, activation codes, int32 accumulators) must be
bit-identical, except the codes of rows transformed partly on the matrix cores (bf16, unit
gamma, K = 2^10 .. 2^14), which are summed in another order and meet the code bar.  Floating-point scales are bit-identical where both sides evaluate the same
operations in the same order (alpha, deq without RMSNorm, the dequant epilogue); with
RMSNorm the fp64 sum of squares is reduced in a different order on the GPU, so deq may
differ by an ulp.
"""
import math

import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import (DEQ_ULPS_MFMA, assert_close_ulps, check_codes, mfma_transform, note, to_dev, to_host,
                            torch_mod)

pytestmark = pytest.mark.gpu


# Shapes: single rows, ragged row blocks (16 rows per block of the row sums), fewer chunks than
# the row-sum ring holds (K = 64 .. 320), row sums spanning several chunks of the ordered final
# sum (N = 16400 > 4096) with a ragged last chunk, and the 7B Wdown and gate shapes.
@pytest.mark.parametrize("N,K", [(1, 64), (3, 192), (257, 1024), (300, 4160), (64, 16384), (16400, 320),
                                 (4096, 16384), (16384, 4096)])
def test_weight_quantisation_bit_exact(orc, N, K):
    note("wquant", N, K)
    W = inputs.make_weights(N, K, seed=N + K)
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    assert to_host(scale)[0] == np.float32(alpha)
    np.testing.assert_array_equal(to_host(Wq), orc.pack_weights(T))


def test_weight_quantisation_ties_and_zero(orc):
    # rows crafted so W/alpha hits +-0.5 and +-1.5 exactly (alpha = 2), plus a zero matrix
    W = np.zeros((2, 64), np.float32)
    W[0, :4] = [1.0, 1.0, 1.0, 5.0]
    W[0, 4:8] = [3.0, 1.0, -1.0, -3.0]
    W[0, 8:] = 2.0
    W[1, :] = 2.0
    # mean |W| = (8 + 8 + 56*2 + 64*2) / 128 = 2, so alpha = 2 exactly
    note("wquant ties")
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    assert to_host(scale)[0] == np.float32(alpha)
    np.testing.assert_array_equal(to_host(Wq), orc.pack_weights(T))
    Z = np.zeros((4, 128), np.float32)
    Wq, scale = B.quantize_weights(to_dev(Z))
    assert to_host(scale)[0] == np.float32(1e-5)
    assert not to_host(Wq).any()


def _act_case(orc, x, abits, use_h, norm, gamma=None, eps=1e-5):
    M, K = x.shape
    q, deq, r = orc.quantize_activations(x, abits, use_h, norm=norm, gamma=gamma, eps=eps)
    codes_d, deq_d = B.quantize_activations(to_dev(x), abits, use_h, norm=norm,
                                            gamma=None if gamma is None else to_dev(gamma), eps=eps)
    codes = to_host(codes_d)
    mfma = mfma_transform(x, K, use_h, gamma)
    check_codes(orc, codes, q, K, abits, not mfma, f"codes M={M} K={K} a{abits} h={use_h} norm={norm}")
    dq = to_host(deq_d)
    if mfma:
        assert_close_ulps(dq, deq, DEQ_ULPS_MFMA, "deq")
    elif norm:
        assert_close_ulps(dq, deq, 2, "deq")
    else:
        np.testing.assert_array_equal(dq, deq)


@pytest.mark.parametrize("L", list(range(6, 16)))
@pytest.mark.parametrize("abits", [4, 8])
def test_actquant_hadamard_all_sizes(orc, L, abits):
    K = 1 << L
    rows_per_block = max(1, 256 // max(K // 64, 1))
    M = rows_per_block + 3 if K <= 16384 else 5     # ragged last block
    M = min(M, 300)
    note("actquant H", K, abits, M)
    x = inputs.make_activations("mixture", M, K, seed=L, outlier_frac=0.01, outlier_scale=50.0)
    _act_case(orc, x, abits, True, norm=True)


@pytest.mark.parametrize("abits", [4, 8])
def test_actquant_exact_class_fp32(orc, abits):
    note("actquant exact fp32", abits)
    x = inputs.make_activations("int_uniform", 40, 256, seed=3)
    _act_case(orc, x, abits, True, norm=False)
    x = inputs.make_activations("int_uniform", 9, 16384, seed=4)
    _act_case(orc, x, abits, True, norm=False)


@pytest.mark.parametrize("L", [10, 11, 12, 13, 14])
@pytest.mark.parametrize("abits", [4, 8])
def test_actquant_exact_class_bf16_matrix_cores(orc, L, abits):
    """Integer-valued bf16 rows (|x| <= 64, so |z| <= 64 K < 2^24) on the matrix-core transform:
    every partial sum is an exact integer in any order, so codes and deq equal the oracle's."""
    K = 1 << L
    M = 3 * (16384 // K) + 1
    note("actquant exact bf16", K, abits, M)
    xf = inputs.make_activations("int_uniform", M, K, seed=L)
    x = inputs.f32_to_bf16_bits(xf)
    assert np.array_equal(inputs.bf16_bits_to_f32(x), xf)   # exact in bf16
    q, deq, _ = orc.quantize_activations(x, abits, True, norm=False)
    codes, deq_d = B.quantize_activations(to_dev(x), abits, True, norm=False)
    np.testing.assert_array_equal(to_host(codes), orc.pack_codes(q, abits))
    np.testing.assert_array_equal(to_host(deq_d), deq)


@pytest.mark.parametrize("K", [256, 2048, 16384])
def test_actquant_gamma_and_fp32_input(orc, K):
    note("actquant gamma", K)
    rng = np.random.default_rng(K)
    x = (rng.standard_normal((33, K)) * 2).astype(np.float32)
    gamma = rng.uniform(0.25, 2.0, K).astype(np.float32)
    _act_case(orc, x, 4, True, norm=True, gamma=gamma, eps=1e-6)
    _act_case(orc, x, 8, True, norm=True, gamma=gamma, eps=0.0)


def test_actquant_zero_and_tiny_rows(orc):
    note("actquant zero rows")
    x = np.zeros((6, 1024), np.float32)
    x[1, 5] = 3.0
    x[2, :] = 1e-37          # absmax below 2^-120 -> zero row
    x[3, 7] = -2.0 ** -100
    x[4, :] = np.arange(1024, dtype=np.float32) - 512
    for abits in (4, 8):
        _act_case(orc, x, abits, True, norm=False)
        _act_case(orc, x, abits, False, norm=False)


@pytest.mark.parametrize("K", [64, 192, 4096, 4160, 16384, 20480])
@pytest.mark.parametrize("abits", [4, 8])
def test_actquant_plain_bitlinear(orc, K, abits):
    note("actquant plain", K, abits)
    x = inputs.make_activations("normal", 17, K, seed=K, outlier_frac=0.01, outlier_scale=30.0)
    _act_case(orc, x, abits, False, norm=True)
    _act_case(orc, x, abits, False, norm=False)


# K = 2^11 .. 2^14 without the transform run the persistent row kernel (8 chunks of 8
# elements per thread, several rows per block for K < 2^14): ragged row groups, gamma in
# the chunked element order, bf16 and fp32 inputs.
@pytest.mark.parametrize("L", [11, 12, 13, 14])
@pytest.mark.parametrize("abits", [4, 8])
def test_actquant_plain_pow2_gamma(orc, L, abits):
    K = 1 << L
    M = 256 // (K // 64) + 3
    note("actquant plain pow2 gamma", K, abits, M)
    x = inputs.make_activations("mixture", M, K, seed=200 + L, outlier_frac=0.01, outlier_scale=50.0)
    gamma = np.random.default_rng(L).uniform(0.25, 2.0, K).astype(np.float32)
    _act_case(orc, x, abits, False, norm=True, gamma=gamma)
    xf = (np.random.default_rng(300 + L).standard_normal((M, K)) * 2).astype(np.float32)
    _act_case(orc, xf, abits, False, norm=True, gamma=gamma, eps=1e-6)
    _act_case(orc, xf, abits, False, norm=False)


# Tile configurations: 256 x 256 tiles for (3100, *, 4000) (at least 192 of them), smaller
# tiles for the other problems above 64 rows (the decode kernel below); K = 64, 320, 384 and 576
# leave a partial last stage (masked loads), the other K fill every stage.  The cases run 1 to 8
# stages (INT4: 256 deep on the large tiles, otherwise 128), odd and even counts, so the
# two-stage-ahead load pipeline is exercised at its start and end.  A K that fills every stage
# (INT4: 256, 512, 768, 1024, 2048, 2560, 8192; INT8: also 384) takes the kernel that loads its
# tiles straight into LDS: 256 x 256 tiles with one to twenty stages through its three buffers,
# or 64 x 128 tiles for the (2500, *, 2200), (2100, *, 206x), 2048^2 and (1000, 8192, 600)
# problems (unaligned rows at N = 2061; the last needs no K split on these tiles); the other K
# take the register-staged kernel (128 x 128 tiles below 192 large tiles).
@pytest.mark.parametrize("M,K,N", [(1, 64, 1), (16, 256, 256), (200, 320, 136), (129, 1024, 257), (300, 2048, 520),
                                   (64, 16384, 64), (2500, 576, 2200), (2500, 1024, 2200), (2100, 64, 2060),
                                   (2100, 256, 2060), (2100, 384, 2060), (2100, 768, 2060), (3100, 64, 4000),
                                   (3100, 256, 4000), (3100, 384, 4000), (3100, 768, 4000), (3100, 2560, 4000),
                                   (3100, 512, 4001), (3100, 512, 4002), (2100, 512, 2061), (512, 2048, 2048),
                                   (1000, 8192, 600)])
@pytest.mark.parametrize("abits", [4, 8])
def test_gemm_s32_bit_exact(orc, M, K, N, abits):
    note("gemm_s32", M, K, N, abits)
    rng = np.random.default_rng(M * 7 + N)
    Qb = 7 if abits == 4 else 127
    q = rng.integers(-Qb - 1, Qb + 1, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = to_host(B.gemm_s32(to_dev(orc.pack_codes(q, abits)), to_dev(orc.pack_weights(T)), K, abits))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


# Mid-size problems whose tiles alone leave CUs idle split K over several blocks that add
# their int32 results atomically: 8 splits of 16 stages, 4 splits of 17 stages whose last has
# 14, and 8 splits of 9 stages whose last has only 2, the second and third with a partial last
# stage (K = 8320).
@pytest.mark.parametrize("M,K,N", [(128, 16384, 1024), (1000, 8320, 600), (300, 8320, 520)])
@pytest.mark.parametrize("abits", [4, 8])
def test_gemm_s32_split_k(orc, M, K, N, abits):
    note("gemm_s32 split K", M, K, N, abits)
    rng = np.random.default_rng(M + K + N)
    Qb = 7 if abits == 4 else 127
    q = rng.integers(-Qb - 1, Qb + 1, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    acc = to_host(B.gemm_s32(to_dev(orc.pack_codes(q, abits)), to_dev(orc.pack_weights(T)), K, abits))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


@pytest.mark.parametrize("abits", [4, 8])
def test_gemm_dequant_split_k(orc, abits):
    M, K, N = 200, 16384, 520
    note("gemm_dequant split K", M, K, N, abits)
    rng = np.random.default_rng(abits + 7)
    Qb = 7 if abits == 4 else 127
    q = rng.integers(-Qb, Qb + 1, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    deq = rng.uniform(1e-4, 3.0, M).astype(np.float32)
    alpha = np.float32(0.0123)
    torch = torch_mod()
    y = B.gemm_dequant(to_dev(orc.pack_codes(q, abits)), to_dev(deq), to_dev(orc.pack_weights(T)),
                       torch.tensor([alpha], device="cuda"), K, abits)
    np.testing.assert_array_equal(to_host(y), orc.dequant(orc.gemm_s32(q, T), deq, float(alpha)))


def test_gemm_s32_extremes(orc):
    # every product at its maximum magnitude: |acc| = 128 * K
    M, K, N = 32, 4096, 48
    for abits, qv in [(4, -8), (4, 7), (8, -128), (8, 127)]:
        note("gemm extremes", abits, qv)
        q = np.full((M, K), qv, np.int8)
        T = np.ones((N, K), np.int8)
        T[1::2] = -1
        acc = to_host(B.gemm_s32(to_dev(orc.pack_codes(q, abits)), to_dev(orc.pack_weights(T)), K, abits))
        np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))


# 128 x 128 tiles, then 256 x 256 tiles loaded into LDS directly (K = 512) and through registers
# (K = 1088, a partial last stage), and 64 x 128 tiles loaded into LDS directly (2100 x 2062),
# ragged in M and N; N = 4001, 4002 and 2062 leave output rows that are not 16-byte aligned (the
# staged epilogue then stores element by element).
@pytest.mark.parametrize("M,K,N", [(150, 1088, 200), (3100, 512, 4000), (3100, 1088, 4000), (3100, 512, 4001),
                                   (3100, 512, 4002), (2100, 512, 2062)])
@pytest.mark.parametrize("abits", [4, 8])
def test_gemm_dequant_bit_exact(orc, M, K, N, abits):
    note("gemm_dequant", M, K, N, abits)
    rng = np.random.default_rng(abits)
    Qb = 7 if abits == 4 else 127
    q = rng.integers(-Qb, Qb + 1, size=(M, K)).astype(np.int8)
    T = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    deq = rng.uniform(1e-4, 3.0, M).astype(np.float32)
    alpha = np.float32(0.0123)
    torch = torch_mod()
    y = B.gemm_dequant(to_dev(orc.pack_codes(q, abits)), to_dev(deq), to_dev(orc.pack_weights(T)),
                       torch.tensor([alpha], device="cuda"), K, abits)
    np.testing.assert_array_equal(to_host(y), orc.dequant(orc.gemm_s32(q, T), deq, float(alpha)))


def test_swiglu(orc):
    note("swiglu")
    rng = np.random.default_rng(5)
    n = 100003
    g = (rng.standard_normal(n) * 4).astype(np.float32)
    u = rng.standard_normal(n).astype(np.float32)
    h = to_host(B.swiglu(to_dev(g), to_dev(u)))
    assert_close_ulps(h, orc.swiglu(g, u), 4, "swiglu")


def test_swiglu_range(orc):
    """silu(g) * u over the whole range where fp32 e^-g is finite and 1 / (1 + e^-g) is normal:
    g in [-87, 88] densely, with u = 1 (the gate alone) and random u.  Below g = -87.3 the true
    |h| is under 1e-35 and the fp32 gate gives a value that small or zero."""
    note("swiglu range")
    g = np.concatenate([np.linspace(-87.0, 88.0, 400001), [0.0, 1e-30, -1e-30, 1e-6, -1e-6]]).astype(np.float32)
    for u in (np.ones_like(g), np.random.default_rng(9).standard_normal(g.size).astype(np.float32)):
        h = to_host(B.swiglu(to_dev(g), to_dev(u)))
        want = orc.swiglu(g, u)
        err = np.abs(h.astype(np.float64) - want) / np.maximum(np.abs(want.astype(np.float64)), 1e-30)
        note("swiglu range: max relative error", float(err.max()), "= ulp", float(err.max() / 2.0 ** -23))
        assert_close_ulps(h, want, 4, "swiglu range")
    gn = np.linspace(-100.0, -87.5, 1001).astype(np.float32)
    h = to_host(B.swiglu(to_dev(gn), to_dev(np.ones_like(gn))))
    assert np.all(np.abs(h) <= 1e-35) and np.all(np.abs(orc.swiglu(gn, np.ones_like(gn))) <= 1e-35)


@pytest.mark.parametrize("M", [16, 65])
@pytest.mark.parametrize("abits", [4, 8])
def test_gemm_s32_max_k(orc, M, abits):
    """K = HBL_MAX_K (131072) at the extreme codes: |acc| = 128 * K (int8) fits the int32
    accumulator of both the decode (M = 16) and the tiled (M = 65) kernels exactly."""
    K, N = 131072, 40
    note("gemm max K", M, abits)
    qv = -8 if abits == 4 else -128
    q = np.full((M, K), qv, np.int8)
    q[1::3, ::5] = 7 if abits == 4 else 127
    T = np.ones((N, K), np.int8)
    T[1::2] = -1
    T[::3, ::7] = 0
    acc = to_host(B.gemm_s32(to_dev(orc.pack_codes(q, abits)), to_dev(orc.pack_weights(T)), K, abits))
    np.testing.assert_array_equal(acc, orc.gemm_s32(q, T))
