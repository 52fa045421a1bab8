"""hbl_forward_noalloc (codes and deq in the library's static scratch) against hbl_forward
(the same kernels with a caller workspace): outputs equal bit for bit, on two calls in a
row with the second one smaller, then at the largest size the scratch holds and at a
decode size (the fused kernel).  The size limit is checked before any HIP call and is
tested on the host (tests/test_abi.py)."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import note, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(name, M, abits):
    wl = inputs.WORKLOADS[name]
    x = to_dev(wl.activations(M))
    Wq, scale = B.quantize_weights(to_dev(inputs.make_weights(wl.N, wl.K)))
    return wl, x, Wq, scale


def _same(wl, x, Wq, scale, abits):
    y_ref = to_host(B.forward(x, Wq, scale, abits, wl.use_hadamard, norm=wl.norm))
    y = to_host(B.forward_noalloc(x, Wq, scale, abits, wl.use_hadamard, norm=wl.norm))
    np.testing.assert_array_equal(y.view(np.int32), y_ref.view(np.int32))


def test_noalloc_equals_forward_two_calls():
    # 7B Wdown a4 at half the batch (32 MiB of codes), then a smaller 1.3B Wo a8 call
    note("noalloc wdown_7b a4 M=4096")
    big = _case("wdown_7b", 4096, 4)
    _same(*big, 4)
    note("noalloc wo_1p3b a8 M=300")
    small = _case("wo_1p3b", 300, 8)
    _same(*small, 8)
    # the full 7B a4 batch fits the scratch exactly; then a decode-size call (fused kernel)
    note("noalloc wdown_7b a4 M=8192")
    _same(*_case("wdown_7b", 8192, 4), 4)
    note("noalloc wdown_7b a4 M=1")
    _same(*_case("wdown_7b", 1, 4), 4)
