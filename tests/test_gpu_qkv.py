"""Parity of the unsigned absmax QKV quantiser and its inverse against the oracle.

Codes are integers decided in fp32 by the same operations on both sides, so packed codes,
gamma and reconstructed values must be bit-identical."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def _heads(rows, d, seed, bf16):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-4, 4, (rows, 1)))
    x[rng.random(rows) < 0.05] = 0.0                      # some all-zero heads
    x[:, :3] *= 20.0                                      # outlier dimensions
    if bf16:
        return inputs.f32_to_bf16_bits(x.astype(np.float32))
    return x.astype(np.float32)


def _check(orc, x, bits):
    rows, d = x.shape
    codes, gamma = B.quantize_qkv(to_dev(x), bits)
    u_o, g_o = orc.quantize_qkv(x, bits)
    np.testing.assert_array_equal(to_host(gamma), g_o)
    np.testing.assert_array_equal(to_host(codes), orc.pack_bits(u_o, bits))
    xh = B.dequantize_qkv(codes, gamma, d, bits)
    np.testing.assert_array_equal(to_host(xh), orc.dequantize_qkv(u_o, g_o, bits))


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("d", [32, 64, 128, 256, 512])
def test_qkv_all_widths_and_head_sizes(orc, d, bits):
    note("qkv", d, bits)
    _check(orc, _heads(1000 + d // 32, d, d * 10 + bits, bf16=(bits % 2 == 1)), bits)


@pytest.mark.parametrize("rows", [1, 2, 7, 64, 4099])
def test_qkv_ragged_rows_fp32(orc, rows):
    note("qkv rows", rows)
    _check(orc, _heads(rows, 128, rows, bf16=False), 3)


def test_qkv_kv_cache_7b(orc):
    """8192 tokens x 32 heads x 128 (7B-like), bf16, 3-bit: every row."""
    note("qkv 7b kv cache")
    _check(orc, _heads(8192 * 32, 128, 11, bf16=True), 3)
