"""The C-ABI calls can be captured in a HIP graph (torch.cuda.CUDAGraph) and replayed: they
enqueue only kernel launches (and, for the gate/up interleave, device copies) on the caller's
stream, allocate nothing and never synchronise.  Every replay, with eager work between the
replays, must reproduce the eager result bit for bit."""
import numpy as np
import pytest

from bit_quantized_gemm_bitlinear_amd import binding as B
from bit_quantized_gemm_bitlinear_amd import inputs
from tests.gpu_util import note, to_dev, torch_mod

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M", [1, 300])
def test_forward_graph_replay(orc, M):
    torch = torch_mod()
    note("graph replay", M)
    wl = inputs.WORKLOADS["wo_1p3b"]
    x = to_dev(wl.activations(M))
    Wq, scale = B.quantize_weights(to_dev(wl.weights()))
    ws = B.forward_workspace(M, wl.K, 4)
    y_graph = torch.empty((M, wl.N), dtype=torch.float32, device="cuda")
    y_eager = B.forward(x, Wq, scale, 4, True, norm=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm-up on the capture stream
        B.forward(x, Wq, scale, 4, True, norm=True, y=y_graph, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.forward(x, Wq, scale, 4, True, norm=True, y=y_graph, ws=ws)
    for i in range(4):
        y_graph.fill_(float("nan"))
        x.mul_(1.0)                      # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int32), y_eager.view(torch.int32)), f"replay {i}"


def test_ffn_graph_replay(orc):
    torch = torch_mod()
    note("graph replay ffn")
    M, D, F = 64, 512, 1024
    x = to_dev(inputs.make_activations("normal", M, D, outlier_frac=0.01, outlier_scale=30.0, seed=5))
    qg, sg = B.quantize_weights(to_dev(inputs.make_weights(F, D, seed=1)))
    qu, su = B.quantize_weights(to_dev(inputs.make_weights(F, D, seed=2)))
    qd, sd = B.quantize_weights(to_dev(inputs.make_weights(D, F, seed=3)))
    Wgu = B.interleave_gate_up(qg, qu, D)
    ws = B.ffn_workspace(M, D, F, 4, torch.bfloat16)
    y_eager = B.ffn_forward(x, Wgu, sg, su, qd, sd, h_dtype=torch.bfloat16)
    y_graph = torch.empty_like(y_eager)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        B.ffn_forward(x, Wgu, sg, su, qd, sd, h_dtype=torch.bfloat16, y=y_graph, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        B.ffn_forward(x, Wgu, sg, su, qd, sd, h_dtype=torch.bfloat16, y=y_graph, ws=ws)
    for i in range(4):
        y_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph.view(torch.int32), y_eager.view(torch.int32)), f"replay {i}"
