"""Device-side plumbing around the C ABI: a layer object that owns its
quantized frozen weight, stabilizer and adapter tensors, allocates outputs
and workspace with PyTorch, and calls fourtune_linear_fwd / _bwd.  Also a
torch.autograd.Function for use inside a training graph.

Nothing here computes any part of the layer; it only moves memory and
calls the library.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ops


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    """Upload bf16 bit patterns (uint16 numpy) as a torch.bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Download a bf16 tensor as uint16 bit patterns."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


class QuantizedLinear:
    """One triple-branch linear on the GPU.

    W_res (bf16 [N, K]) is quantized once on the device to 32x32 MXFP4 tiles
    by fourtune_quantize; the forward reads them row-wise and the backward's
    input gradient reads the same bytes transposed.  The rank factors are kept in the library's rank-major storage:
    L1t = L1^T [r_s, K], L2 [r_s, N] (frozen), At = A^T [r_l, K], B [r_l, N]
    (trainable).  act_in / act_out (ops.FT_ACT_*) mark an activation before
    or after the layer: with act_in, X is the pre-activation h; with act_out,
    the backward's dY is the gradient of act(Y) and needs H = Y.  precision:
    ops.FT_W4A4G4 (the method) .. ops.FT_W4A16G16, or its name.  w_block:
    "tile32" (the method), "tile32_t" (the tiles plus a stored transposed
    layout copy that the input gradient reads instead; a measured
    alternative) or "row32" (group-wise 1x32 blocks: W_res and W_res^T are
    quantized separately, by one FT_Q_ROW32_T pass).
    """

    def __init__(self, W_res: torch.Tensor, L1t: torch.Tensor | None, L2: torch.Tensor | None,
                 At: torch.Tensor | None, B: torch.Tensor | None, stream=None,
                 act_in: int = ops.FT_ACT_NONE, act_out: int = ops.FT_ACT_NONE,
                 precision=ops.FT_W4A4G4, w_block: str = "tile32"):
        N, K = W_res.shape
        self.act_in, self.act_out = int(act_in), int(act_out)
        if isinstance(precision, str):
            precision = ops.PRECISION_NAMES[precision]
        self.precision = int(precision)
        dev = W_res.device
        self.N, self.K = int(N), int(K)
        self.r_s = 0 if L1t is None else int(L1t.shape[0])
        self.r_l = 0 if At is None else int(At.shape[0])
        self.L1t, self.L2, self.At, self.B = L1t, L2, At, B
        self.w_block = {"tile32": ops.FT_WBLOCK_TILE32, "row32": ops.FT_WBLOCK_ROW32,
                        "tile32_t": ops.FT_WBLOCK_TILE32_T}[w_block]
        self.w_codes = _empty((N, K // 2), torch.uint8, dev)
        if self.w_block == ops.FT_WBLOCK_TILE32:
            self.w_scales = _empty((N // 32, K // 32), torch.uint8, dev)
            self.wt_codes = self.wt_scales = None
            mode = ops.FT_Q_TILE32
        elif self.w_block == ops.FT_WBLOCK_TILE32_T:
            self.w_scales = _empty((N // 32, K // 32), torch.uint8, dev)
            self.wt_codes = _empty((K, N // 2), torch.uint8, dev)
            self.wt_scales = _empty((K // 32, N // 32), torch.uint8, dev)
            mode = ops.FT_Q_TILE32
        else:
            self.wt_codes = _empty((K, N // 2), torch.uint8, dev)
            self.w_scales = _empty((N, K // 32), torch.uint8, dev)
            self.wt_scales = _empty((K, N // 32), torch.uint8, dev)
            mode = ops.FT_Q_ROW32_T
        ops.fourtune_quantize(mode, W_res, N, K, K, self.w_codes, self.w_scales,
                              self.wt_codes, self.wt_scales, stream=stream)
        self.device = dev
        self._ws = {}

    @classmethod
    def from_factors(cls, W_res, L1, L2, A, B, stream=None, act_in: int = ops.FT_ACT_NONE,
                     act_out: int = ops.FT_ACT_NONE, precision=ops.FT_W4A4G4,
                     w_block: str = "tile32") -> "QuantizedLinear":
        """From factors in the method's orientation (L1 [K, r_s], A [K, r_l]):
        the down-projections are copied once into the rank-major storage."""
        t = lambda x: None if x is None else x.t().contiguous()
        return cls(W_res, t(L1), L2, t(A), B, stream=stream, act_in=act_in, act_out=act_out,
                   precision=precision, w_block=w_block)

    @property
    def a16(self) -> bool:
        return bool(self.precision & ops.FT_W4A16G4)

    @property
    def g16(self) -> bool:
        return bool(self.precision & ops.FT_W4A4G16)

    @property
    def R(self):
        return self.r_s + self.r_l

    def weight_bytes(self) -> int:
        """Device bytes the quantized residual weight occupies (codes and
        scales, every stored layout)."""
        ts = (self.w_codes, self.w_scales, self.wt_codes, self.wt_scales)
        return int(sum(t.numel() for t in ts if t is not None))

    def desc(self, M: int) -> ops.FtLinear:
        return ops.make_linear(M, self.K, self.N, self.r_s, self.r_l, self.w_codes,
                               self.w_scales, self.wt_codes, self.wt_scales, self.L1t, self.L2,
                               self.At, self.B, self.act_in, self.act_out, self.precision,
                               self.w_block)

    def workspace(self, M: int, is_bwd: bool):
        key = (M, bool(is_bwd))
        if key not in self._ws:
            n = ops.fourtune_workspace_bytes(self.desc(M), is_bwd)
            self._ws[key] = _empty((max(n, 256),), torch.uint8, self.device)
        return self._ws[key]

    def forward(self, X: torch.Tensor, stream=None, want_codes: bool = False):
        """Returns (Y, U) or (Y, U, xq_codes, xq_scales); the codes are None
        when the layer's precision keeps activations in bf16 (A16)."""
        M = int(X.shape[0])
        dev = self.device
        Y = _empty((M, self.N), torch.bfloat16, dev)
        U = _empty((M, max(self.R, 1)), torch.bfloat16, dev)
        codes = want_codes and not self.a16
        qc = _empty((M, self.K // 2), torch.uint8, dev) if codes else None
        qs = _empty((M, self.K // 32), torch.uint8, dev) if codes else None
        ws = self.workspace(M, False)
        ops.fourtune_linear_fwd(self.desc(M), X, Y, U if self.R else None, qc, qs, ws,
                                ws.numel(), stream)
        return (Y, U, qc, qs) if want_codes else (Y, U)

    def backward(self, dY: torch.Tensor, X: torch.Tensor, U: torch.Tensor, need_dx: bool = True,
                 grad_f32: bool = False, stream=None, want_codes: bool = False,
                 H: torch.Tensor | None = None):
        """Returns (dX, dAt, dB, P) or (dX, dAt, dB, P, gq_codes, gq_scales);
        dAt = dA^T [r_l, K] and dB [r_l, N], the layouts of At and B.  H is
        the forward's Y, needed when the layer has act_out.  The codes are
        None when the layer's precision keeps gradients in bf16 (G16)."""
        M = int(dY.shape[0])
        dev = self.device
        dX = _empty((M, self.K), torch.bfloat16, dev) if need_dx else None
        gdt = torch.float32 if grad_f32 else torch.bfloat16
        dA = _empty((self.r_l, self.K), gdt, dev) if self.r_l else None
        dB = _empty((self.r_l, self.N), gdt, dev) if self.r_l else None
        P = _empty((M, max(self.R, 1)), torch.bfloat16, dev)
        codes = want_codes and not self.g16
        qc = _empty((M, self.N // 2), torch.uint8, dev) if codes else None
        qs = _empty((M, self.N // 32), torch.uint8, dev) if codes else None
        ws = self.workspace(M, True)
        ops.fourtune_linear_bwd(self.desc(M), dY, X, U if self.R else None, H, dX, dA, dB,
                                ops.FT_F32 if grad_f32 else ops.FT_BF16,
                                P if self.R else None, qc, qs, ws, ws.numel(), stream)
        out = (dX, dA, dB, P)
        return out + (qc, qs) if want_codes else out


_mlp_ws = {}


def mlp_forward(fc1: QuantizedLinear, fc2: QuantizedLinear, X: torch.Tensor, stream=None,
                want_codes: bool = False):
    """The MLP block's two forwards with FC1's GEMM fused with FC2's
    quantization (fourtune_mlp_fwd); fc2 must have act_in = GELU.  Returns
    (h, U1, Y, U2) or (h, U1, Y, U2, aq_codes, aq_scales), aq being FC2's
    quantized input Qrow(gelu(h))."""
    M = int(X.shape[0])
    dev = fc1.device
    H = _empty((M, fc1.N), torch.bfloat16, dev)
    Y = _empty((M, fc2.N), torch.bfloat16, dev)
    U1 = _empty((M, max(fc1.R, 1)), torch.bfloat16, dev)
    U2 = _empty((M, max(fc2.R, 1)), torch.bfloat16, dev)
    codes = want_codes and not fc2.a16
    qc = _empty((M, fc2.K // 2), torch.uint8, dev) if codes else None
    qs = _empty((M, fc2.K // 32), torch.uint8, dev) if codes else None
    d1, d2 = fc1.desc(M), fc2.desc(M)
    key = (id(fc1), id(fc2), M)
    if key not in _mlp_ws:
        n = ops.fourtune_mlp_workspace_bytes(d1, d2)
        _mlp_ws[key] = _empty((max(n, 256),), torch.uint8, dev)
    ws = _mlp_ws[key]
    ops.fourtune_mlp_fwd(d1, d2, X, H, Y, U1 if fc1.R else None, U2 if fc2.R else None, qc, qs,
                         ws, ws.numel(), stream)
    return (H, U1, Y, U2, qc, qs) if want_codes else (H, U1, Y, U2)


def mlp_backward(fc1: QuantizedLinear, fc2: QuantizedLinear, dY: torch.Tensor, X: torch.Tensor,
                 H: torch.Tensor, U1: torch.Tensor, U2: torch.Tensor, grad_f32: bool = False,
                 stream=None):
    """The MLP block's backward with FC2's input-gradient GEMM making FC1's
    incoming gradient and its quantization (fourtune_mlp_bwd); fc1 must have
    act_out = GELU and fc2 act_in = GELU.  Returns (dX, dA1t, dB1, dA2t, dB2)."""
    M = int(dY.shape[0])
    dev = fc1.device
    gdt = torch.float32 if grad_f32 else torch.bfloat16
    dX = _empty((M, fc1.K), torch.bfloat16, dev)
    dA1 = _empty((fc1.r_l, fc1.K), gdt, dev) if fc1.r_l else None
    dB1 = _empty((fc1.r_l, fc1.N), gdt, dev) if fc1.r_l else None
    dA2 = _empty((fc2.r_l, fc2.K), gdt, dev) if fc2.r_l else None
    dB2 = _empty((fc2.r_l, fc2.N), gdt, dev) if fc2.r_l else None
    d1, d2 = fc1.desc(M), fc2.desc(M)
    key = (id(fc1), id(fc2), M, "bwd")
    if key not in _mlp_ws:
        n = ops.fourtune_mlp_bwd_workspace_bytes(d1, d2)
        _mlp_ws[key] = _empty((max(n, 256),), torch.uint8, dev)
    ws = _mlp_ws[key]
    ops.fourtune_mlp_bwd(d1, d2, dY, X, H, U1 if fc1.R else None, U2 if fc2.R else None, dX, dA1,
                         dB1, dA2, dB2, ops.FT_F32 if grad_f32 else ops.FT_BF16, ws, ws.numel(),
                         stream)
    return dX, dA1, dB1, dA2, dB2


class FourTuneLinearFunction(torch.autograd.Function):
    """Y = layer(X) with gradients for X, At and B (W_res, L1, L2 frozen).
    At and B must be the tensors the layer holds.  With the layer's act_in,
    X is the pre-activation and Y = layer(act(X)); with act_out the function
    returns act(Y) (computed by the library's activation entry point) and
    keeps Y for the backward."""

    @staticmethod
    def forward(ctx, X, At, B, layer: QuantizedLinear):
        Y, U = layer.forward(X.contiguous())
        ctx.layer = layer
        if layer.act_out != ops.FT_ACT_NONE:
            ctx.save_for_backward(X, U, Y)
            out = torch.empty_like(Y)
            ops.fourtune_act_fwd(layer.act_out, Y, Y.numel(), out)
            return out
        ctx.save_for_backward(X, U)
        return Y

    @staticmethod
    def backward(ctx, dY):
        layer = ctx.layer
        if layer.act_out != ops.FT_ACT_NONE:
            X, U, H = ctx.saved_tensors
        else:
            (X, U), H = ctx.saved_tensors, None
        dX, dA, dB, _ = layer.backward(dY.contiguous().to(torch.bfloat16), X, U,
                                       need_dx=ctx.needs_input_grad[0], H=H)
        if dX is not None and layer.act_in != ops.FT_ACT_NONE:
            # the library's dX is the gradient of the layer's input act(X);
            # X's gradient is that times act'(X), by the same device function
            dh = torch.empty_like(dX)
            ops.fourtune_act_bwd(layer.act_in, X, dX, dX.numel(), dh)
            dX = dh
        return dX, dA, dB, None
