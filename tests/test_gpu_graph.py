"""The layer's forward and backward captured in one HIP graph
(torch.cuda.graph around the C-ABI calls) and replayed.  No kernel of the
library records a memset, so the graph holds only kernel nodes; every replay
must reproduce the eager result bit for bit, with the program's own eager
work and synchronizations between the replays (the kernels are
deterministic)."""
import numpy as np
import pytest
import torch

from bit_quantized_amd import ops, synth

from _gpu import DEV, GpuCase, require_gpu, say, up as _up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _buffers(lay, M):
    bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=DEV)
    R = max(lay.R, 1)
    return dict(Y=bt(M, lay.N), U=bt(M, R), dX=bt(M, lay.K), dA=bt(lay.r_l, lay.K),
                dB=bt(lay.r_l, lay.N), P=bt(M, R))


def _step(lay, M, X, dY, b, wsf, wsb):
    d = lay.desc(M)
    ops.fourtune_linear_fwd(d, X, b["Y"], b["U"], None, None, wsf, wsf.numel())
    ops.fourtune_linear_bwd(d, dY, X, b["U"], None, b["dX"], b["dA"], b["dB"], ops.FT_BF16, b["P"],
                            None, None, wsb, wsb.numel())


@pytest.mark.parametrize("precision", ["W4A4G4", "W4A16G16"])
def test_graph_replays_match_eager(precision):
    c = synth.flux_linear_case("graph", 300, 288, 544, 16, 8, seed=12)
    other = synth.flux_linear_case("graph_other", 200, 256, 320, 8, 8, seed=13)
    say("case graph", precision)
    g = GpuCase(c, precision)
    lay, M = g.layer, c.M
    X, dY = g.X, g.dY
    b = _buffers(lay, M)
    wsf, wsb = lay.workspace(M, False), lay.workspace(M, True)
    _step(lay, M, X, dY, b, wsf, wsb)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in b.items()}
    # warm up on a side stream, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(lay, M, X, dY, b, wsf, wsb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _step(lay, M, X, dY, b, wsf, wsb)
    torch.cuda.synchronize()
    g2 = GpuCase(other, precision)
    for r in range(4):
        for t in b.values():
            t.fill_(0.0)
        g2.run()                              # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in b.items():
            np.testing.assert_array_equal(v.view(torch.int16).cpu().numpy(),
                                          ref[k].view(torch.int16).cpu().numpy(),
                                          err_msg=f"replay {r} {k}")
    say("graph replays bit-identical", precision)


def test_graph_replays_mlp_fused():
    """The MLP block's fused forward (FC1's GEMM making FC2's quantized GELU
    input and down-projection sums) and both backwards in one graph: every
    replay reproduces the eager result bit for bit."""
    from bit_quantized_amd.layer import QuantizedLinear
    G = ops.FT_ACT_GELU_TANH
    M, K, F = 300, 256, 544
    c1 = synth.flux_linear_case("graph_fc1", M, K, F, 16, 8, seed=21)
    c2 = synth.flux_linear_case("graph_fc2", M, F, K, 16, 8, seed=22)
    mk = lambda c, **kw: QuantizedLinear.from_factors(_up(c.W_res), _up(c.L1), _up(c.L2), _up(c.A),
                                                      _up(c.B), **kw)
    fc1, fc2 = mk(c1, act_out=G), mk(c2, act_in=G)
    say("case graph mlp fused", (M, K, F))
    X, dY = _up(c1.X), _up(c2.dY)
    bt = lambda *sh: torch.empty(sh, dtype=torch.bfloat16, device=DEV)
    b = dict(h=bt(M, F), U1=bt(M, fc1.R), Y=bt(M, K), U2=bt(M, fc2.R), dX2=bt(M, F),
             dA2=bt(fc2.r_l, F), dB2=bt(fc2.r_l, K), dX1=bt(M, K), dA1=bt(fc1.r_l, K),
             dB1=bt(fc1.r_l, F))
    d1, d2 = fc1.desc(M), fc2.desc(M)
    nm = ops.fourtune_mlp_workspace_bytes(d1, d2)
    wm = torch.empty(nm, dtype=torch.uint8, device=DEV)
    w1b, w2b = fc1.workspace(M, True), fc2.workspace(M, True)

    def step():
        ops.fourtune_mlp_fwd(d1, d2, X, b["h"], b["Y"], b["U1"], b["U2"], None, None, wm, nm)
        ops.fourtune_linear_bwd(d2, dY, b["h"], b["U2"], None, b["dX2"], b["dA2"], b["dB2"],
                                ops.FT_BF16, None, None, None, w2b, w2b.numel())
        ops.fourtune_linear_bwd(d1, b["dX2"], X, b["U1"], b["h"], b["dX1"], b["dA1"], b["dB1"],
                                ops.FT_BF16, None, None, None, w1b, w1b.numel())

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in b.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    other = GpuCase(synth.flux_linear_case("graph_mlp_other", 200, 256, 320, 8, 8, seed=23))
    for r in range(4):
        for t in b.values():
            t.fill_(0.0)
        other.run()                           # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in b.items():
            np.testing.assert_array_equal(v.view(torch.int16).cpu().numpy(),
                                          ref[k].view(torch.int16).cpu().numpy(),
                                          err_msg=f"replay {r} {k}")
    say("mlp graph replays bit-identical")
