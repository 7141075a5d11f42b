"""C-ABI checks that need no GPU: the library loads, exports every function
include/fourtune.h declares, and rejects bad arguments on the host before
touching any device memory (fake addresses are never dereferenced)."""
import ctypes
import os
import re

import pytest

from bit_quantized_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fourtune.h")

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH),
                                reason="libfourtune.so not built")

A16 = 0x10000000  # a fake 16-byte-aligned device address


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fourtune_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(ops.EXPORTS)
    L = ops.lib()
    for n in names:
        assert getattr(L, n) is not None


def test_status_strings():
    for s in range(7):
        assert ops.status_string(s)
    assert ops.status_string(99) == "unknown status"


def _q(mode, x=A16, rows=64, cols=64, ld=64, c=A16, s=A16, ct=None, st=None):
    return ops.lib().fourtune_quantize(mode, x, rows, cols, ld, c, s, ct, st, None)


def test_quantize_argument_errors():
    assert _q(3) == ops.FT_EINVAL
    assert _q(ops.FT_Q_ROW32, x=None) == ops.FT_EINVAL
    assert _q(ops.FT_Q_ROW32, ct=A16, st=A16) == ops.FT_EINVAL
    assert _q(ops.FT_Q_ROW32_T) == ops.FT_EINVAL          # transposed outputs missing
    assert _q(ops.FT_Q_TILE32, ct=A16) == ops.FT_EINVAL   # transposed codes without scales
    assert _q(ops.FT_Q_TILE32, ct=A16 + 4, st=A16) == ops.FT_EALIGN
    assert _q(ops.FT_Q_ROW32, cols=48, ld=48) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_TILE32, rows=40) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_ROW32_T, rows=40, ct=A16, st=A16) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_ROW32, rows=-1) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_ROW32, ld=32) == ops.FT_EALIGN     # ld < cols
    assert _q(ops.FT_Q_ROW32, ld=68) == ops.FT_EALIGN     # ld not a multiple of 8
    assert _q(ops.FT_Q_ROW32, x=A16 + 2) == ops.FT_EALIGN
    assert _q(ops.FT_Q_ROW32, rows=0) == ops.FT_OK        # empty is a no-op
    # a row stride out of range is refused before any product is formed
    assert _q(ops.FT_Q_ROW32, ld=1 << 62) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_ROW32, ld=-8) == ops.FT_ESHAPE
    assert _q(ops.FT_Q_ROW32, rows=0, ld=1 << 62) == ops.FT_ESHAPE


def _layer(M=64, K=64, N=64, rs=8, rl=8, **kw):
    d = dict(w_codes=A16, w_scales=A16, wt_codes=None, wt_scales=None, L1t=A16, L2=A16, At=A16,
             B=A16)
    d.update(kw)
    return ops.make_linear(M, K, N, rs, rl, **d)


def _fwd(L, X=A16, Y=A16, U=A16, qc=None, qs=None, ws=A16, wsb=1 << 40):
    return ops.lib().fourtune_linear_fwd(ctypes.byref(L), X, Y, U, qc, qs, ws, wsb, None)


def _bwd(L, dY=A16, X=A16, U=A16, dX=A16, dA=A16, dB=A16, gdt=0, P=None, qc=None, qs=None,
         ws=A16, wsb=1 << 40, H=None):
    return ops.lib().fourtune_linear_bwd(ctypes.byref(L), dY, X, U, H, dX, dA, dB, gdt, P, qc,
                                         qs, ws, wsb, None)


def test_linear_shape_errors():
    for L in (_layer(M=0), _layer(K=48), _layer(N=40), _layer(K=0), _layer(rs=70, rl=60),
              _layer(rs=-1)):
        assert _fwd(L) == ops.FT_ESHAPE
        assert _bwd(L) == ops.FT_ESHAPE
    assert ops.lib().fourtune_linear_fwd(None, A16, A16, A16, None, None, A16, 1, None) == ops.FT_EINVAL
    # within M * K * 2 < 2^31, but not once padded by 256 rows
    M = (2 ** 31 - 1) // 64
    assert M * 32 * 2 < 2 ** 31 and (M + 256) * 32 * 2 >= 2 ** 31
    assert _fwd(_layer(M=M, K=32, N=32)) == ops.FT_ESHAPE
    assert _bwd(_layer(M=M, K=32, N=32)) == ops.FT_ESHAPE


def test_linear_pointer_errors():
    assert _fwd(_layer(w_codes=None)) == ops.FT_EINVAL
    assert _fwd(_layer(L1t=None)) == ops.FT_EINVAL
    assert _fwd(_layer(B=None)) == ops.FT_EINVAL
    assert _fwd(_layer(L2=None)) == ops.FT_EINVAL
    T, R = ops.FT_WBLOCK_TILE32_T, ops.FT_WBLOCK_ROW32
    assert _fwd(_layer(w_block=T, wt_codes=A16)) == ops.FT_EINVAL   # second codes without scales
    # the method's tiles serve the dgrad as they are: a second weight is refused
    assert _fwd(_layer(wt_codes=A16, wt_scales=A16)) == ops.FT_EINVAL
    assert _bwd(_layer(wt_codes=A16, wt_scales=A16)) == ops.FT_EINVAL
    # the stored-copy and group-wise layouts need their second weight for dX only
    assert _bwd(_layer(w_block=T)) == ops.FT_EINVAL
    assert _bwd(_layer(w_block=R)) == ops.FT_EINVAL
    assert _bwd(_layer(w_block=T), dX=None) == ops.FT_EUNSUPPORTED
    assert _bwd(_layer()) == ops.FT_EUNSUPPORTED               # only the missing GPU stops it
    assert _fwd(_layer(w_block=T, wt_codes=A16 + 4, wt_scales=A16)) == ops.FT_EALIGN
    assert _fwd(_layer(), X=None) == ops.FT_EINVAL
    assert _fwd(_layer(), U=None) == ops.FT_EINVAL
    assert _fwd(_layer(), qc=A16) == ops.FT_EINVAL              # codes without scales
    assert _fwd(_layer(), X=A16 + 8) == ops.FT_EALIGN
    assert _fwd(_layer(At=A16 + 4)) == ops.FT_EALIGN
    assert _bwd(_layer(), dY=None) == ops.FT_EINVAL
    assert _bwd(_layer(), dA=None) == ops.FT_EINVAL
    assert _bwd(_layer(), gdt=7) == ops.FT_EINVAL
    assert _bwd(_layer(), dX=A16 + 2) == ops.FT_EALIGN
    # activations: enum values checked; act_out needs H, aligned
    assert _fwd(_layer(act_in=2)) == ops.FT_EINVAL
    assert _bwd(_layer(act_out=5), H=A16) == ops.FT_EINVAL
    assert _bwd(_layer(act_out=ops.FT_ACT_GELU_TANH)) == ops.FT_EINVAL
    assert _bwd(_layer(act_out=ops.FT_ACT_GELU_TANH), H=A16 + 2) == ops.FT_EALIGN
    # ranks zero: no low-rank pointers are needed
    L0 = _layer(rs=0, rl=0, L1t=None, L2=None, At=None, B=None)
    assert _fwd(L0, U=None, wsb=0) == ops.FT_EWORKSPACE


def test_act_argument_errors():
    L = ops.lib()
    G = ops.FT_ACT_GELU_TANH
    assert L.fourtune_act_fwd(0, A16, 64, A16, None) == ops.FT_EINVAL       # no activation
    assert L.fourtune_act_fwd(G, None, 64, A16, None) == ops.FT_EINVAL
    assert L.fourtune_act_fwd(G, A16, -1, A16, None) == ops.FT_ESHAPE
    assert L.fourtune_act_fwd(G, A16 + 2, 64, A16, None) == ops.FT_EALIGN
    assert L.fourtune_act_fwd(G, A16, 0, A16, None) == ops.FT_OK           # empty is a no-op
    assert L.fourtune_act_bwd(G, A16, None, 64, A16, None) == ops.FT_EINVAL
    assert L.fourtune_act_bwd(G, A16, A16 + 8, 64, A16, None) == ops.FT_EALIGN
    assert L.fourtune_act_bwd(3, A16, A16, 64, A16, None) == ops.FT_EINVAL


def test_workspace_size_checked_before_launch():
    L = _layer(M=300, K=288, N=544)
    need_f = ops.fourtune_workspace_bytes(L, False)
    need_b = ops.fourtune_workspace_bytes(L, True)
    assert need_f >= 300 * 288 // 2 + 300 * 288 // 32
    assert need_b >= 300 * 544 // 2 + 300 * 544 // 32 + 300 * 16 * 2
    assert _fwd(L, wsb=need_f - 1) == ops.FT_EWORKSPACE
    assert _bwd(L, wsb=need_b - 1) == ops.FT_EWORKSPACE
    assert _fwd(L, ws=None, wsb=need_f) == ops.FT_EINVAL
    assert ops.fourtune_workspace_bytes(_layer(K=40), False) == 0


def test_valid_call_without_gpu_reports_unsupported():
    # With no GPU present the first HIP query fails; the call must say so
    # instead of launching anything.
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _fwd(_layer()) == ops.FT_EUNSUPPORTED


def _dq(mode=ops.FT_Q_TILE32, c=A16, s=A16, rows=64, cols=64, out=A16):
    return ops.lib().fourtune_dequantize(mode, c, s, rows, cols, out, None)


def test_dequantize_argument_errors():
    assert _dq(mode=ops.FT_Q_ROW32) == ops.FT_EINVAL
    assert _dq(c=None) == ops.FT_EINVAL
    assert _dq(out=None) == ops.FT_EINVAL
    assert _dq(rows=48) == ops.FT_ESHAPE
    assert _dq(cols=40) == ops.FT_ESHAPE
    assert _dq(rows=-32) == ops.FT_ESHAPE
    assert _dq(rows=1 << 16, cols=1 << 15) == ops.FT_ESHAPE       # 2^32 bytes of bf16
    assert _dq(s=A16 + 8) == ops.FT_EALIGN
    assert _dq(rows=0) == ops.FT_OK


def test_precision_argument_errors_and_workspace():
    assert _fwd(_layer(precision=4)) == ops.FT_EINVAL
    assert _fwd(_layer(precision=-1)) == ops.FT_EINVAL
    assert ops.fourtune_workspace_bytes(_layer(precision=7), False) == 0
    # a 16-bit side has no codes to hand out
    assert _fwd(_layer(precision=ops.FT_W4A16G4), qc=A16, qs=A16) == ops.FT_EINVAL
    assert _bwd(_layer(precision=ops.FT_W4A4G16), qc=A16, qs=A16) == ops.FT_EINVAL
    # ... while the other side still may
    M, K, N = 4096, 1024, 2048
    base = {b: ops.fourtune_workspace_bytes(_layer(M=M, K=K, N=N), b) for b in (False, True)}
    a16 = {b: ops.fourtune_workspace_bytes(_layer(M=M, K=K, N=N, precision="W4A16G4"), b)
           for b in (False, True)}
    g16 = {b: ops.fourtune_workspace_bytes(_layer(M=M, K=K, N=N, precision="W4A4G16"), b)
           for b in (False, True)}
    # A16 drops X's codes and scales and adds the bf16 weight [N, K]
    assert a16[False] == base[False] - M * K // 2 - M * K // 32 + N * K * 2
    assert a16[True] == base[True]
    # G16 drops dY's codes and scales and adds the transposed bf16 weight
    assert g16[True] == base[True] - M * N // 2 - M * N // 32 + K * N * 2
    assert g16[False] == base[False]
    # with an activation next to the layer, its bf16 output is made as well
    act = ops.fourtune_workspace_bytes(_layer(M=M, K=K, N=N, precision="W4A16G16",
                                              act_in=ops.FT_ACT_GELU_TANH), False)
    assert act == a16[False] + M * K * 2
    # the dequantized weight must fit 32-bit offsets with its padded rows
    big = _layer(M=64, K=(1 << 16), N=(1 << 14) - 32, precision="W4A16G4")
    assert _fwd(big) == ops.FT_ESHAPE
    assert _fwd(_layer(M=64, K=(1 << 16), N=(1 << 14) - 32)) != ops.FT_ESHAPE


def test_weight_block_argument_errors():
    assert _fwd(_layer(w_block=3)) == ops.FT_EINVAL
    assert _fwd(_layer(w_block=-1)) == ops.FT_EINVAL
    assert ops.fourtune_workspace_bytes(_layer(w_block=3), False) == 0
    assert ops.fourtune_workspace_bytes(_layer(w_block=ops.FT_WBLOCK_TILE32_T), False) > 0
    # group-wise weights have no tile dequantizer: 4-bit products only
    assert _fwd(_layer(w_block=ops.FT_WBLOCK_ROW32, precision="W4A16G4")) == ops.FT_EINVAL
    assert _bwd(_layer(w_block=ops.FT_WBLOCK_ROW32, precision="W4A4G16")) == ops.FT_EINVAL
    # otherwise the shape checks pass and only the missing GPU stops the call
    assert _fwd(_layer(w_block=ops.FT_WBLOCK_ROW32)) == ops.FT_EUNSUPPORTED
    # the workspace does not depend on the weight's block shape
    assert (ops.fourtune_workspace_bytes(_layer(w_block=ops.FT_WBLOCK_ROW32), True)
            == ops.fourtune_workspace_bytes(_layer(), True))


def _mlp(f1, f2, X=A16, H=A16, Y=A16, U1=A16, U2=A16, qc=None, qs=None, ws=A16, wsb=1 << 40):
    return ops.lib().fourtune_mlp_fwd(ctypes.byref(f1), ctypes.byref(f2), X, H, Y, U1, U2, qc, qs,
                                      ws, wsb, None)


def test_mlp_forward_argument_errors():
    """The fused MLP forward checks both layers, that they chain (M equal,
    fc2.K == fc1.N, fc2's input activation set), its pointers and its
    workspace before touching any device."""
    G = ops.FT_ACT_GELU_TANH
    f1 = _layer(M=300, K=256, N=544)
    f2 = _layer(M=300, K=544, N=256, act_in=G)
    need = ops.fourtune_mlp_workspace_bytes(f1, f2)
    assert need == ops.fourtune_workspace_bytes(f1, False) + ops.fourtune_workspace_bytes(f2, False)
    assert ops.fourtune_mlp_workspace_bytes(f1, _layer(K=40)) == 0
    assert _mlp(f1, _layer(M=300, K=512, N=256, act_in=G)) == ops.FT_ESHAPE     # fc2.K != fc1.N
    assert _mlp(f1, _layer(M=200, K=544, N=256, act_in=G)) == ops.FT_ESHAPE     # M differs
    assert _mlp(f1, _layer(M=300, K=544, N=256)) == ops.FT_EINVAL               # no GELU input
    assert _mlp(_layer(M=300, K=256, N=544, w_codes=None), f2) == ops.FT_EINVAL
    assert _mlp(f1, f2, H=None) == ops.FT_EINVAL
    assert _mlp(f1, f2, U2=None) == ops.FT_EINVAL
    assert _mlp(f1, f2, qc=A16) == ops.FT_EINVAL                                # codes without scales
    assert _mlp(f1, f2, Y=A16 + 4) == ops.FT_EALIGN
    assert _mlp(f1, f2, qc=A16, qs=A16 + 2) == ops.FT_EALIGN
    assert _mlp(f1, f2, wsb=need - 1) == ops.FT_EWORKSPACE
    assert _mlp(f1, f2, ws=None, wsb=need) == ops.FT_EINVAL
    # A16 on fc2: no quantized input to hand out
    assert _mlp(f1, _layer(M=300, K=544, N=256, act_in=G, precision=ops.FT_W4A16G4),
                qc=A16, qs=A16) == ops.FT_EINVAL
    assert _mlp(f1, f2) == ops.FT_EUNSUPPORTED          # only the missing GPU stops it


def _mlpb(f1, f2, dY=A16, X=A16, H=A16, U1=A16, U2=A16, dX=A16, dA1=A16, dB1=A16, dA2=A16, dB2=A16,
          gdt=0, ws=A16, wsb=1 << 40):
    return ops.lib().fourtune_mlp_bwd(ctypes.byref(f1), ctypes.byref(f2), dY, X, H, U1, U2, dX, dA1,
                                      dB1, dA2, dB2, gdt, ws, wsb, None)


def test_mlp_backward_argument_errors():
    """The mirrored MLP backward checks both layers, that they chain and carry
    the GELU between them, its pointers and its workspace before touching any
    device."""
    G = ops.FT_ACT_GELU_TANH
    f1 = _layer(M=300, K=256, N=544, act_out=G)
    f2 = _layer(M=300, K=544, N=256, act_in=G)
    need = ops.fourtune_mlp_bwd_workspace_bytes(f1, f2)
    assert need > ops.fourtune_workspace_bytes(f1, True) + ops.fourtune_workspace_bytes(f2, True)
    assert need >= ops.fourtune_workspace_bytes(f1, True) + ops.fourtune_workspace_bytes(f2, True) + 300 * 544 * 2
    assert ops.fourtune_mlp_bwd_workspace_bytes(f1, _layer(K=40)) == 0
    assert _mlpb(f1, _layer(M=300, K=512, N=256, act_in=G)) == ops.FT_ESHAPE
    assert _mlpb(_layer(M=300, K=256, N=544), f2) == ops.FT_EINVAL        # no GELU after FC1
    assert _mlpb(f1, _layer(M=300, K=544, N=256)) == ops.FT_EINVAL        # no GELU before FC2
    assert _mlpb(f1, f2, dX=None) == ops.FT_EINVAL
    assert _mlpb(f1, f2, H=None) == ops.FT_EINVAL
    assert _mlpb(f1, f2, dB2=None) == ops.FT_EINVAL
    assert _mlpb(f1, f2, gdt=5) == ops.FT_EINVAL
    assert _mlpb(f1, f2, dA1=A16 + 4) == ops.FT_EALIGN
    assert _mlpb(f1, f2, wsb=need - 1) == ops.FT_EWORKSPACE
    assert _mlpb(f1, f2, ws=None, wsb=need) == ops.FT_EINVAL
    assert _mlpb(f1, f2) == ops.FT_EUNSUPPORTED          # only the missing GPU stops it


def _fwd_noalloc(L, X=A16, Y=A16, U=A16, qc=None, qs=None):
    return ops.lib().fourtune_linear_fwd_noalloc(ctypes.byref(L), X, Y, U, qc, qs, None)


def test_noalloc_forward_argument_errors():
    """The forward without workspace argument checks like the forward, and
    refuses a layer whose workspace exceeds the library's scratch array
    before touching any device."""
    assert ops.lib().fourtune_linear_fwd_noalloc(None, A16, A16, A16, None, None, None) == ops.FT_EINVAL
    assert _fwd_noalloc(_layer(K=48)) == ops.FT_ESHAPE
    assert _fwd_noalloc(_layer(w_codes=None)) == ops.FT_EINVAL
    big = _layer(M=65536, K=4096, N=4096)
    assert ops.fourtune_workspace_bytes(big, False) > ops.FT_NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(big) == ops.FT_EWORKSPACE
    small = _layer(M=64, K=256, N=256)
    assert ops.fourtune_workspace_bytes(small, False) <= ops.FT_NOALLOC_SCRATCH_BYTES
    assert _fwd_noalloc(small) == ops.FT_EUNSUPPORTED      # only the missing GPU stops it
