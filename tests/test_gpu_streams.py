"""Calls on different streams are independent (the stream convention of include/hbl.h).

Problems that take the different launch paths of hbl_forward, and one FFN block, are enqueued
together, each on a stream of its own with its own output and workspace, for several rounds in
a row; every output must equal, bit for bit, the same call run alone on the current stream.
Paths: 256 x 256 tiles loaded straight into LDS (M = 4096, K = 2048, N = 4096); K split over
blocks whose int32 sums are added atomically into the caller's output after a fill kernel
(M = 128, K = 16384, N = 1024); the decode GEMM (M = 16, a8); the one-kernel decode forward
(M = 1, K = 16384); the FFN block (fused gate/up GEMM with SwiGLU, then the down projection).
"""
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import note, to_dev, torch_mod

pytestmark = pytest.mark.gpu

CASES = [(4096, 2048, 4096, 4), (128, 16384, 1024, 4), (16, 16384, 1024, 8), (1, 16384, 1024, 4)]
ROUNDS = 3


def test_concurrent_streams_equal_serial_calls(orc):
    torch = torch_mod()
    calls = []   # (label, function(y, ws), y_alone, y, ws)
    for i, (M, K, N, abits) in enumerate(CASES):
        note("streams: forward", M, K, N, f"a{abits}")
        x = to_dev(inputs.make_activations("mixture", M, K, seed=10 + i, outlier_frac=0.01, outlier_scale=50.0))
        Wq, sc = B.quantize_weights(to_dev(inputs.make_weights(N, K, seed=20 + i)))

        def fwd(y, ws, x=x, Wq=Wq, sc=sc, abits=abits):
            return B.forward(x, Wq, sc, abits, True, norm=True, y=y, ws=ws)

        y_alone = B.forward(x, Wq, sc, abits, True, norm=True)
        calls.append((f"forward M={M} K={K} N={N} a{abits}", fwd, y_alone, torch.empty_like(y_alone),
                      B.forward_workspace(M, K, abits)))

    M, D, F = 256, 512, 1024
    note("streams: ffn", M, D, F)
    x = to_dev(inputs.make_activations("normal", M, D, seed=30, outlier_frac=0.01, outlier_scale=30.0))
    qg, sg = B.quantize_weights(to_dev(inputs.make_weights(F, D, seed=31)))
    qu, su = B.quantize_weights(to_dev(inputs.make_weights(F, D, seed=32)))
    qd, sd = B.quantize_weights(to_dev(inputs.make_weights(D, F, seed=33)))
    Wgu = B.interleave_gate_up(qg, qu, D)

    def ffn(y, ws):
        return B.ffn_forward(x, Wgu, sg, su, qd, sd, h_dtype=torch.bfloat16, y=y, ws=ws)

    y_alone = B.ffn_forward(x, Wgu, sg, su, qd, sd, h_dtype=torch.bfloat16)
    calls.append((f"ffn M={M} D={D} F={F}", ffn, y_alone, torch.empty_like(y_alone),
                  B.ffn_workspace(M, D, F, 4, torch.bfloat16)))
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream() for _ in calls]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for r in range(ROUNDS):
        note("streams: round", r)
        for s, (_, fn, _, y, ws) in zip(streams, calls):
            with torch.cuda.stream(s):
                y.fill_(float("nan"))
                fn(y, ws)
        torch.cuda.synchronize()
        for label, _, y_alone, y, _ in calls:
            assert torch.equal(y.view(torch.int32), y_alone.view(torch.int32)), f"round {r}: {label}"
