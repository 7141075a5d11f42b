"""GPU: the forward that allocates nothing (fourtune_linear_fwd_noalloc)
against the forward with a caller-given workspace, through the C ABI: the
same kernels on the same inputs, so Y, U and the activation codes must
agree bit for bit.  Two calls in a row on the library's scratch array, the
second with fewer tokens (and a different layer), each checked."""
import numpy as np
import pytest
import torch

from bit_quantized_amd import ops, synth
from bit_quantized_amd.layer import QuantizedLinear, bits_of

from _gpu import require_gpu, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _layer(c):
    opt = lambda a, r: up(a) if r else None
    return QuantizedLinear.from_factors(up(c.W_res), opt(c.L1, c.r_s), opt(c.L2, c.r_s),
                                        opt(c.A, c.r_l), opt(c.B, c.r_l))


def _both(lay, X, M):
    dev = X.device
    out = {}
    for mode in ("workspace", "noalloc"):
        Y = torch.full((M, lay.N), float("nan"), dtype=torch.bfloat16, device=dev)
        U = torch.full((M, max(lay.R, 1)), float("nan"), dtype=torch.bfloat16, device=dev)
        qc = torch.full((M, lay.K // 2), 0xAB, dtype=torch.uint8, device=dev)
        qs = torch.full((M, lay.K // 32), 0xCD, dtype=torch.uint8, device=dev)
        d = lay.desc(M)
        if mode == "workspace":
            ws = lay.workspace(M, False)
            ops.fourtune_linear_fwd(d, X, Y, U if lay.R else None, qc, qs, ws, ws.numel())
        else:
            ops.fourtune_linear_fwd_noalloc(d, X, Y, U if lay.R else None, qc, qs)
        torch.cuda.synchronize()
        out[mode] = (bits_of(Y), bits_of(U)[:, :lay.R], qc.cpu().numpy(), qs.cpu().numpy())
    return out


@pytest.mark.parametrize("big, small", [
    ((520, 1024, 768, 32, 16), (130, 1024, 768, 32, 16)),    # same layer, fewer tokens
    ((4608, 3072, 2048, 32, 16), (300, 288, 544, 16, 8)),    # then a smaller, ragged layer
])
def test_noalloc_forward_matches_workspace_forward(big, small):
    for k, (M, K, N, rs, rl) in enumerate((big, small)):
        c = synth.flux_linear_case(f"noalloc_{M}x{K}x{N}", M, K, N, rs, rl, seed=31 + M + k)
        say("case noalloc", c.name, "call", k + 1)
        lay = _layer(c)
        need = ops.fourtune_workspace_bytes(lay.desc(M), False)
        assert need <= ops.FT_NOALLOC_SCRATCH_BYTES, need
        got = _both(lay, up(c.X), M)
        for name, a, b in zip(("Y", "U", "codes", "scales"), got["workspace"], got["noalloc"]):
            np.testing.assert_array_equal(a, b, err_msg=f"{c.name} {name}")
        assert not np.isnan(_f32(got["noalloc"][0])).any()


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_noalloc_refuses_oversized_layer():
    c = synth.flux_linear_case("noalloc_big", 64, 256, 256, 8, 8, seed=3)
    lay = _layer(c)
    M = 1 << 16
    d = ops.make_linear(M, 12288, 256, 8, 8, lay.w_codes, lay.w_scales, None, None, lay.L1t,
                        lay.L2, lay.At, lay.B)
    assert ops.fourtune_workspace_bytes(d, False) > ops.FT_NOALLOC_SCRATCH_BYTES
    # refused on the host before anything is read: a small buffer stands in
    X = torch.empty((64,), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(ops.FourTuneError) as e:
        ops.fourtune_linear_fwd_noalloc(d, X, X, X, None, None)
    assert e.value.status == ops.FT_EWORKSPACE
