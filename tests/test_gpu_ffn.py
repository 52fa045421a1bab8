"""Parity of the fused FFN gate/up projection and of the whole FFN block.

The fused kernel computes g and u exactly as hbl_gemm_dequant does and applies the same
device SwiGLU as hbl_swiglu, so its h must equal the unfused GPU sequence bit for bit
(fp32), and the bf16 h must equal torch's round-to-nearest-even cast of that fp32 h.

Against the oracle:
  - h is within 8 ulp of the fp64-evaluated SwiGLU of the oracle's g and u (fp32), or one
    bf16 step apart on fewer than 1e-3 of its elements (bf16);
  - the down projection run by the oracle on the GPU's own h meets the H-BitLinear bars:
    codes bit-identical or, for bf16 h (transformed partly on the matrix cores), the code
    bar; relative Frobenius error <= 1e-3 and 4 ulp on rows whose codes all match;
  - the whole block meets the method's code bar: at most 1e-4 of the down projection's
    INT4/INT8 codes differ from the oracle block's codes, each by one step.
The block output is not held to relative Frobenius 1e-3: one code of a row that moves by one
step moves that row's output by about 1/sqrt(F * E[q^2]) of its norm (about 0.4 % for INT4
at F = 16384), so a single flipped code exceeds 1e-3.  The output bar asserted is the one
the code bar implies, 2 * sqrt(f / E[q^2]) for a measured fraction f of flipped codes.
"""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import (assert_close_ulps, assert_code_bar, assert_rows_close, check_codes, mfma_transform, note,
                            rel_fro, to_dev, to_host, torch_mod)

pytestmark = pytest.mark.gpu


def _weights(orc, F, D, seeds=(21, 22)):
    Wg = inputs.make_weights(F, D, seed=seeds[0])
    Wu = inputs.make_weights(F, D, seed=seeds[1])
    qg, sg = B.quantize_weights(to_dev(Wg))
    qu, su = B.quantize_weights(to_dev(Wu))
    return Wg, Wu, qg, sg, qu, su


@pytest.mark.parametrize("F,K", [(32, 64), (352, 512), (4096, 256)])
def test_interleave_layout(orc, F, K):
    note("interleave", F, K)
    _, _, qg, _, qu, _ = _weights(orc, F, K)
    Wgu = to_host(B.interleave_gate_up(qg, qu, K))
    g, u = to_host(qg), to_host(qu)
    want = np.concatenate([g.reshape(F // 32, 32, K // 4), u.reshape(F // 32, 32, K // 4)], axis=1)
    np.testing.assert_array_equal(Wgu, want.reshape(2 * F, K // 4))


# (M, K, F, abits): ragged rows and output columns on the 128-tile launch; 128 x 256-tile
# launches with an even, an odd and a partial last stage count; single row and minimum F; INT8
# with a deep K; 128 x 256 tiles whose last column tile is a quarter full (F = 2080) and a
# ragged last row tile.
SHAPES = [(300, 512, 352, 4), (300, 512, 352, 8), (2048, 512, 2048, 4), (2048, 1024, 2048, 8),
          (2048, 768, 2048, 4), (2048, 320, 2048, 8), (1, 256, 32, 4), (77, 4096, 128, 8), (513, 4096, 1056, 4),
          (2050, 512, 2080, 4), (2050, 512, 2080, 8)]


@pytest.mark.parametrize("M,K,F,abits", SHAPES)
def test_fused_gate_up_equals_unfused(orc, M, K, F, abits):
    torch = torch_mod()
    note("gate_up fused vs unfused", M, K, F, abits)
    x = inputs.make_activations("normal", M, K, outlier_frac=0.01, outlier_scale=30.0, seed=M + K)
    _, _, qg, sg, qu, su = _weights(orc, F, K)
    codes, deq = B.quantize_activations(to_dev(x), abits, False, norm=True)
    Wgu = B.interleave_gate_up(qg, qu, K)
    g = B.gemm_dequant(codes, deq, qg, sg, K, abits)
    u = B.gemm_dequant(codes, deq, qu, su, K, abits)
    h_ref = B.swiglu(g, u)
    h32 = B.gate_up_swiglu(codes, deq, Wgu, sg, su, K, abits, h_dtype=torch.float32)
    h16 = B.gate_up_swiglu(codes, deq, Wgu, sg, su, K, abits, h_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(h32.view(torch.int32), h_ref.view(torch.int32))
    assert torch.equal(h16.view(torch.int16), h_ref.to(torch.bfloat16).view(torch.int16))


def test_fused_gate_up_vs_oracle(orc):
    torch = torch_mod()
    M, K, F = 130, 1024, 544
    note("gate_up vs oracle", M, K, F)
    x = inputs.make_activations("normal", M, K, outlier_frac=0.01, outlier_scale=30.0, seed=7)
    Wg, Wu, qg, sg, qu, su = _weights(orc, F, K)
    codes, deq = B.quantize_activations(to_dev(x), 4, False, norm=True)
    Wgu = B.interleave_gate_up(qg, qu, K)
    h32 = to_host(B.gate_up_swiglu(codes, deq, Wgu, sg, su, K, 4, h_dtype=torch.float32))
    h16 = to_host(B.gate_up_swiglu(codes, deq, Wgu, sg, su, K, 4, h_dtype=torch.bfloat16))
    Tg, ag = orc.quantize_weights(Wg)
    Tu, au = orc.quantize_weights(Wu)
    h_o = orc.swiglu(orc.forward(x, Tg, ag, 4, False, norm=True), orc.forward(x, Tu, au, 4, False, norm=True))
    assert_close_ulps(h32, h_o, 8, "h fp32")
    # bf16: the same rounding of values a few fp32 ulp apart: equal or one bf16 step apart
    d = np.abs(_ordered_bf16(h16) - _ordered_bf16(orc.round_bf16(h_o)))
    assert d.max() <= 1
    assert (d != 0).mean() < 1e-3


def _r256(n):
    return (n + 255) // 256 * 256


def _block(orc, M, D, F, abits, h_bf16, x=None, sample=None):
    """Runs hbl_ffn_forward; returns the sampled rows of y and of the h it stored in its
    workspace, the oracle's block output and h on the same rows, and the oracle's down
    projection applied to the GPU's h (which isolates the down projection)."""
    torch = torch_mod()
    wl = inputs.WORKLOADS["ffn_7b"]
    if x is None:
        x = inputs.make_activations("normal", M, D, outlier_frac=0.01, outlier_scale=30.0, seed=M)
    Wg, Wu, qg, sg, qu, su = _weights(orc, F, D, (wl.extra["seed_gate"], wl.extra["seed_up"]))
    Wd = inputs.make_weights(D, F, seed=wl.extra["seed_down"])
    qd, sd = B.quantize_weights(to_dev(Wd))
    Wgu = B.interleave_gate_up(qg, qu, D)
    ht = torch.bfloat16 if h_bf16 else torch.float32
    ws = B.ffn_workspace(M, D, F, abits, ht)
    y = to_host(B.ffn_forward(to_dev(x), Wgu, sg, su, qd, sd, abits=abits, h_dtype=ht, ws=ws))
    off = _r256(M * D * abits // 8) + _r256(4 * M)
    hb = 2 if h_bf16 else 4
    h = to_host(ws[off:off + M * F * hb].view(ht)).reshape(M, F)
    rows = np.arange(x.shape[0]) if sample is None else sample
    Tg, ag = orc.quantize_weights(Wg)
    Tu, au = orc.quantize_weights(Wu)
    Td, ad = orc.quantize_weights(Wd)
    y_o, h_o = orc.ffn_forward(np.ascontiguousarray(x[rows]), Tg, ag, Tu, au, Td, ad, abits=abits, h_bf16=h_bf16,
                               intermediates=True)
    h_s = np.ascontiguousarray(h[rows])
    y_down = orc.forward(h_s, Td, ad, abits, True, norm=True)
    # the down projection's codes, left in the workspace, and the oracle block's codes
    off2 = off + _r256(M * F * hb)
    codes2 = to_host(ws[off2:off2 + M * F * abits // 8]).reshape(M, F * abits // 8)[rows]
    q_o = orc.quantize_activations(h_o, abits, True, norm=True)[0]
    return dict(y=y[rows], h=h_s, y_o=y_o, h_o=h_o, y_down=y_down, codes2=codes2, q_o=q_o, F=F, abits=abits,
                ctx=(x, qg, sg, qu, su, qd, sd, Wgu, ht))


def _ordered_bf16(b):
    """bf16 patterns -> integers in value order (+0 and -0 both 0)."""
    b = b.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def _check_block(r, h_bf16):
    # gate/up: h equal to the oracle's up to the last place (device expf vs fp64 exp)
    if h_bf16:
        d = np.abs(_ordered_bf16(r["h"]) - _ordered_bf16(r["h_o"]))
        assert d.max() <= 1 and (d != 0).mean() < 1e-3
    else:
        assert_close_ulps(r["h"], r["h_o"], 8, "h")
    # down projection on the GPU's own h: the H-BitLinear bars (codes, then outputs)
    orc = _orc()
    q_down = orc.quantize_activations(r["h"], r["abits"], True, norm=True)[0]
    exact = not mfma_transform(r["h"], r["F"], True)
    rows_ok = check_codes(orc, r["codes2"], q_down, r["F"], r["abits"], exact, "down projection codes")
    assert_rows_close(r["y"], r["y_down"], rows_ok, exact, "down projection")
    # whole block: the code bar on the down projection's codes, then the output bar it implies
    f = assert_code_bar(_orc(), r["codes2"], r["q_o"], r["F"], r["abits"], "block codes")
    eq2 = float(np.mean(np.asarray(r["q_o"], np.float64) ** 2))
    err = rel_fro(r["y"], r["y_o"])
    bound = 2.0 * np.sqrt(f / eq2) + 1e-4
    note(f"block: relative Frobenius error {err:.3e} (bound from the code bar {bound:.3e}, E[q^2] {eq2:.2f})")
    assert err <= bound


@pytest.mark.parametrize("h_bf16", [True, False])
@pytest.mark.parametrize("abits", [4, 8])
def test_ffn_forward_vs_oracle(orc, abits, h_bf16):
    note("ffn_forward vs oracle", abits, h_bf16)
    _check_block(_block(orc, 40, 512, 1024, abits, h_bf16), h_bf16)


def test_ffn_forward_equals_separate_calls(orc):
    """The block entry point equals the sequence of single-step C-ABI calls bit for bit."""
    torch = torch_mod()
    note("ffn_forward vs calls")
    M, D, F = 200, 512, 1024
    r = _block(orc, M, D, F, 4, True)
    x, qg, sg, qu, su, qd, sd, Wgu, ht = r["ctx"]
    xd = to_dev(x)
    codes, deq = B.quantize_activations(xd, 4, False, norm=True)
    h = B.swiglu(B.gemm_dequant(codes, deq, qg, sg, D, 4), B.gemm_dequant(codes, deq, qu, su, D, 4))
    y2 = to_host(B.forward(h.to(torch.bfloat16), qd, sd, 4, True, norm=True))
    np.testing.assert_array_equal(r["y"].view(np.int32), y2.view(np.int32))


@pytest.mark.parametrize("h_bf16", [True, False])
def test_ffn_full_size_stratified_rows(orc, h_bf16):
    """The 7B-like block at its full size (M=8192, D=4096, F=16384) in the launch bench.py
    times; the oracle checks 4 seeded rows of every 128-row band (every row tile of both
    GEMMs), 258 rows with the first and the last."""
    wl = inputs.WORKLOADS["ffn_7b"]
    M, D, F = wl.M, wl.extra["hidden"], wl.extra["ffn"]
    note("ffn full size", M, D, F, "bf16 h" if h_bf16 else "fp32 h")
    rng = np.random.default_rng(99)
    bands = [b * 128 + rng.choice(128, 4, replace=False) for b in range(M // 128)]
    sample = np.unique(np.concatenate(bands + [np.array([0, M - 1])]))
    _check_block(_block(orc, M, D, F, 4, h_bf16, x=wl.activations(), sample=sample), h_bf16)


def _orc():
    import oracle

    return oracle
