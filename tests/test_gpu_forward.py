"""End-to-end parity of hbl_forward (and the FFN block built from the C ABI calls) against
the CPU oracle on the five synthetic workloads.

Bars: on the exact-arithmetic workload (integer activations, no norm) codes, int32
accumulators and outputs are bit-identical.  On the Gaussian/outlier workloads (bf16 rows,
whose first five transform stages run on the matrix cores and are summed in another order)
the codes meet the method's code bar (at most 1e-4 of them differ from the oracle's, each by
one step), the outputs meet its bar (relative Frobenius error <= 1e-3) and are within 4 ulp
on every row whose codes all match (plus the few ulp by which deq differs: its sum of squares
is taken in fp32 and g = max|z| is summed in another order).
Full-size cases run exactly the launch that bench.py times and compare every row with the
oracle.
"""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import (assert_close_ulps, assert_rows_close, check_codes, mfma_transform, note, rel_fro,
                            to_dev, to_host, torch_mod)

pytestmark = pytest.mark.gpu


def _layer(orc, wl, abits, M=None, sample=None, seed_w=inputs.SEED_W):
    """Run the GPU forward on the workload (M rows) and compare rows `sample` with the oracle."""
    x = wl.activations(M)
    W = inputs.make_weights(wl.N, wl.K, seed=seed_w)
    T, alpha = orc.quantize_weights(W)
    Wq, scale = B.quantize_weights(to_dev(W))
    np.testing.assert_array_equal(to_host(Wq), orc.pack_weights(T))
    assert to_host(scale)[0] == np.float32(alpha)
    xd = to_dev(x)
    ws = B.forward_workspace(x.shape[0], wl.K, abits)
    y = to_host(B.forward(xd, Wq, scale, abits, wl.use_hadamard, norm=wl.norm, ws=ws))
    rows = np.arange(x.shape[0]) if sample is None else sample
    xs = np.ascontiguousarray(x[rows])
    y_o, q_o, acc_o, deq_o = orc.forward(xs, T, alpha, abits, wl.use_hadamard, norm=wl.norm, intermediates=True)
    # the codes written to the workspace by the same call
    ab = x.shape[0] * wl.K * abits // 8
    codes = to_host(ws[:ab]).reshape(x.shape[0], wl.K * abits // 8)[rows]
    exact = not mfma_transform(x, wl.K, wl.use_hadamard)
    rows_ok = check_codes(orc, codes, q_o, wl.K, abits, exact, f"{wl.name} a{abits} codes")
    return y[rows], y_o, acc_o, deq_o, (xd, Wq, scale, ws, rows_ok, exact)


def test_tiny_exact_bit_exact(orc):
    wl = inputs.WORKLOADS["tiny_exact"]
    note("forward tiny_exact")
    y, y_o, acc_o, deq_o, (xd, Wq, scale, ws, _, _) = _layer(orc, wl, 4)
    np.testing.assert_array_equal(y, y_o)
    codes_d, deq_d = B.quantize_activations(xd, 4, True)
    np.testing.assert_array_equal(to_host(deq_d), deq_o)
    np.testing.assert_array_equal(to_host(B.gemm_s32(codes_d, Wq, wl.K, 4)), acc_o)


# Enough rows that one flipped code does not dominate the relative Frobenius error: a flip
# moves its row by about 1/sqrt(K E[q^2]) (1.2 % at K = 2048 with INT4), that is by
# 1/sqrt(K E[q^2] M) of the whole output.
@pytest.mark.parametrize("name,abits,M", [("wo_1p3b", 8, 512), ("wo_1p3b", 4, 512), ("wdown_3b", 4, 400),
                                          ("wdown_7b", 4, 256), ("wdown_7b", 8, 256)])
def test_workload_rows(orc, name, abits, M):
    wl = inputs.WORKLOADS[name]
    note("forward", name, abits, M)
    y, y_o, _, _, ctx = _layer(orc, wl, abits, M=M)
    assert_rows_close(y, y_o, ctx[-2], ctx[-1], name)


def test_forward_deterministic(orc):
    wl = inputs.WORKLOADS["wo_1p3b"]
    note("determinism")
    torch = torch_mod()
    x = to_dev(wl.activations(300))
    Wq, scale = B.quantize_weights(to_dev(inputs.make_weights(wl.N, wl.K)))
    y1 = B.forward(x, Wq, scale, 4, True, norm=True)
    y2 = B.forward(x, Wq, scale, 4, True, norm=True)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_ffn_block_rows(orc):
    """RMSNorm -> BitLinear gate/up (INT4, no transform) -> SwiGLU -> H-BitLinear down."""
    wl = inputs.WORKLOADS["ffn_7b"]
    hid, ffn = wl.extra["hidden"], wl.extra["ffn"]
    M = 16
    note("ffn block", M)
    x = wl.activations(M)
    Wg = inputs.make_weights(ffn, hid, seed=wl.extra["seed_gate"])
    Wu = inputs.make_weights(ffn, hid, seed=wl.extra["seed_up"])
    Wd = inputs.make_weights(hid, ffn, seed=wl.extra["seed_down"])
    # GPU
    xd = to_dev(x)
    qg, sg = B.quantize_weights(to_dev(Wg))
    qu, su = B.quantize_weights(to_dev(Wu))
    qd, sd = B.quantize_weights(to_dev(Wd))
    codes, deq = B.quantize_activations(xd, 4, False, norm=True)
    g = B.gemm_dequant(codes, deq, qg, sg, hid, 4)
    u = B.gemm_dequant(codes, deq, qu, su, hid, 4)
    h = B.swiglu(g, u)
    y = to_host(B.forward(h, qd, sd, 4, True, norm=True))
    # oracle
    Tg, ag = orc.quantize_weights(Wg)
    Tu, au = orc.quantize_weights(Wu)
    Td, ad = orc.quantize_weights(Wd)
    g_o = orc.forward(x, Tg, ag, 4, False, norm=True)
    u_o = orc.forward(x, Tu, au, 4, False, norm=True)
    assert_close_ulps(to_host(g), g_o, 4, "gate")
    assert_close_ulps(to_host(u), u_o, 4, "up")
    h_o = orc.swiglu(g_o, u_o)
    y_o = orc.forward(h_o, Td, ad, 4, True, norm=True)
    assert rel_fro(y, y_o) <= 1e-3


FULL = [("wo_1p3b", 8), ("wo_1p3b", 4), ("wdown_3b", 4), ("wdown_7b", 4), ("wdown_7b", 8)]


@pytest.mark.parametrize("name,abits", FULL)
def test_full_size_all_rows(orc, name, abits):
    """The full-size launch bench.py times, every row of it checked against the oracle
    (so every output tile of the GEMM and every row group of the activation kernel)."""
    wl = inputs.WORKLOADS[name]
    note("full size", name, abits, wl.M, wl.K, wl.N)
    y, y_o, _, _, ctx = _layer(orc, wl, abits)
    assert_rows_close(y, y_o, ctx[-2], ctx[-1], f"full size {name} a{abits}")
