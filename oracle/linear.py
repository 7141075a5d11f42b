"""Plain CPU oracle for FourTune's W4A4G4 triple-branch linear layer.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): the product path never
imports, calls or executes anything in this package.

Notation (weights stored like a PyTorch Linear, W_res is [N, K]):

* X  [M, K] bf16 input, dY [M, N] bf16 incoming gradient;
* W_res [N, K] quantized once to 32x32 MXFP4 tiles (frozen 4-bit backbone);
* L1 [K, r_s], L2 [r_s, N]: frozen low-rank stabilizer, bf16;
* A  [K, r_l], B  [r_l, N]: trainable LoRA adapter, bf16;
* D = [L1 | A] [K, R] and V = [L2 ; B] [R, N], R = r_s + r_l.

Forward, FourTune "3.1 Triple-Branch Hybrid-Precision Pipeline", Eq. (2):
    Y = GEMM4(Q(X), Q(R)) + X L_stab + X (A B)
here with the backbone term written for W_res stored [N, K]:
    Y = deq(Q_row32(X)) deq(Q_tile32(W_res))^T + U V,   U = bf16(X D).
X (A B) is evaluated as (X A) B; the two are equal in exact arithmetic.

Backward, "3.2 4-Bit Backward Pass via Block-Quantization", Eq. (3) and the
adapter-gradient equations that follow it:
    dX = deq(Q_row32(dY)) deq(Q_tile32(W_res)) + P D^T,   P = bf16(dY V^T)
    dB = (X A)^T dY = U[:, r_s:]^T dY
    dA = X^T (dY B^T) = X^T P[:, r_s:]
Q is not differentiated (the backbone term of Eq. (3) applies Q to the
incoming gradient directly).  No gradient is produced for W_res, L1 or L2,
which the page keeps frozen.

Readings where the pages are silent: U and P are rounded to bf16 (the
low-rank products run as bf16 matrix products with bf16 outputs); every sum
is accumulated exactly enough in float64 and rounded once to the output
dtype (bf16 by default).

Precision settings ("4.3 Ablation Study", "Impact of Precision
Configurations", Table 4): W4A4G4 is the method above; A16 keeps the
forward's activation in bf16 in the backbone product (Y's first term reads
X itself instead of deq(Q_row32(X))), G16 keeps the incoming gradient in
bf16 in the input-gradient product (dX's first term reads dY itself).  The
weight stays 4-bit (deq(Q_tile32(W_res))) in all four; the low-rank
branches and the adapter gradients do not change.  The pages name the four
settings only; this reading is the plain one of their labels (W, A, G the
bit widths of weight, activation and gradient in the backbone products).
"""

from __future__ import annotations

import numpy as np

from . import mxfp4 as q

PRECISIONS = ("W4A4G4", "W4A16G4", "W4A4G16", "W4A16G16")
W_BLOCKS = ("tile32", "row32")


def _check_precision(precision: str) -> None:
    if precision not in PRECISIONS:
        raise ValueError(precision)


def weight_fwd(w_codes, w_scales, w_block="tile32") -> np.ndarray:
    """deq(Q(W_res)) [N, K] as the forward's backbone product reads it.

    tile32: the method's 32x32 tiles ("3.2").  row32: the group-wise
    alternative of the block-shape ablation ("4.3", Table 5), 1x32 blocks
    along K, codes [N, K/2] and scales [N, K/32]."""
    if w_block == "tile32":
        return q.dequantize_tile32(w_codes, w_scales)
    if w_block == "row32":
        return q.dequantize_row32(w_codes, w_scales)
    raise ValueError(w_block)


def weight_dgrad(w_codes, w_scales, w_block="tile32", wt=None) -> np.ndarray:
    """The [N, K] weight the input-gradient product reads.

    tile32: the forward's own numbers (a square tile's scale does not depend
    on the orientation).  row32: 1x32 blocks along K do not survive the
    transpose, so the dgrad needs its own quantization of W_res^T with
    blocks along N: wt = (codes [K, N/2], scales [K, N/32]) = Q_row32(W_res^T),
    and the product reads deq(wt)^T."""
    if w_block == "tile32":
        return q.dequantize_tile32(w_codes, w_scales)
    if w_block == "row32":
        if wt is None:
            raise ValueError("row32 weights need the quantized transpose wt")
        return q.dequantize_row32(*wt).T
    raise ValueError(w_block)


def _round_out(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round a float64 result to the output dtype; bf16 results are bits."""
    if out_dtype == "bf16":
        return q.f64_to_bf16_bits(x)
    if out_dtype == "f32":
        return q.f64_to_f32(x)
    if out_dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(out_dtype)


def out_to_f64(x: np.ndarray) -> np.ndarray:
    """Value of an output array as float64 (bf16 outputs are uint16 bits)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return q.bf16_bits_to_f64(x)
    return x.astype(np.float64)


def stack_down(L1: np.ndarray, A: np.ndarray) -> np.ndarray:
    """D = [L1 | A] as float64 [K, R]."""
    return np.concatenate([q.bf16_bits_to_f64(L1), q.bf16_bits_to_f64(A)], axis=1)


def stack_up(L2: np.ndarray, B: np.ndarray) -> np.ndarray:
    """V = [L2 ; B] as float64 [R, N]."""
    return np.concatenate([q.bf16_bits_to_f64(L2), q.bf16_bits_to_f64(B)], axis=0)


def down_proj(x_bits: np.ndarray, D: np.ndarray) -> np.ndarray:
    """bf16(x D): the shared down-projection of all low-rank branches (bits)."""
    return q.f64_to_bf16_bits(q.bf16_bits_to_f64(x_bits) @ D)


def linear_fwd(X, w_codes, w_scales, L1, L2, A, B, out_dtype="bf16", precision="W4A4G4",
               w_block="tile32"):
    """Forward of the triple-branch linear.

    Inputs are bf16 bit arrays except w_codes / w_scales, the 32x32-tile
    MXFP4 form of W_res.  Returns dict with Y (out_dtype), U (bf16 bits
    [M, R]), and the activation codes/scales (row32 of X; None under A16,
    which does not quantize X).
    """
    _check_precision(precision)
    if "A16" in precision:
        xq_codes = xq_scales = None
        Xh = q.bf16_bits_to_f64(X)
    else:
        xq_codes, xq_scales = q.quantize_row32(X)
        Xh = q.dequantize_row32(xq_codes, xq_scales)      # [M, K]
    Wh = weight_fwd(w_codes, w_scales, w_block)           # [N, K]
    U = down_proj(X, stack_down(L1, A))                   # [M, R] bf16
    Y = Xh @ Wh.T + q.bf16_bits_to_f64(U) @ stack_up(L2, B)
    return {"Y": _round_out(Y, out_dtype), "U": U, "xq_codes": xq_codes, "xq_scales": xq_scales}


def linear_bwd(dY, X, U, w_codes, w_scales, L1, L2, A, B, out_dtype="bf16",
               grad_dtype="bf16", precision="W4A4G4", w_block="tile32", wt=None):
    """Backward of the triple-branch linear (straight-through Q).

    U is the forward's saved bf16(X D).  Returns dict with dX, dA, dB, P and
    the gradient codes/scales (row32 of dY, blocks along N; None under G16,
    which does not quantize dY).  w_block / wt: see weight_dgrad.
    """
    _check_precision(precision)
    r_s = np.asarray(L1).shape[1]
    if "G16" in precision:
        gq_codes = gq_scales = None
        Gh = q.bf16_bits_to_f64(dY)
    else:
        gq_codes, gq_scales = q.quantize_row32(dY)
        Gh = q.dequantize_row32(gq_codes, gq_scales)      # [M, N]
    Wh = weight_dgrad(w_codes, w_scales, w_block, wt)     # [N, K]
    V = stack_up(L2, B)                                    # [R, N]
    P = down_proj(dY, V.T)                                 # [M, R] bf16
    dX = Gh @ Wh + q.bf16_bits_to_f64(P) @ stack_down(L1, A).T
    Xf = q.bf16_bits_to_f64(X)
    Gf = q.bf16_bits_to_f64(dY)
    dA = Xf.T @ q.bf16_bits_to_f64(P)[:, r_s:]
    dB = q.bf16_bits_to_f64(U)[:, r_s:].T @ Gf
    return {"dX": _round_out(dX, out_dtype), "dA": _round_out(dA, grad_dtype),
            "dB": _round_out(dB, grad_dtype), "P": P,
            "gq_codes": gq_codes, "gq_scales": gq_scales}


def linear_fwd_rows(rows, X, w_codes, w_scales, L1, L2, A, B, precision="W4A4G4",
                    w_block="tile32"):
    """Float64 forward outputs (Y before rounding, U) for selected rows only.

    Each row of the layer depends only on the same row of X, so large
    layers can be checked on a sample of rows.
    """
    _check_precision(precision)
    Xs = np.asarray(X)[rows]
    if "A16" in precision:
        Xh = q.bf16_bits_to_f64(Xs)
    else:
        xq_codes, xq_scales = q.quantize_row32(Xs)
        Xh = q.dequantize_row32(xq_codes, xq_scales)
    Wh = weight_fwd(w_codes, w_scales, w_block)
    U = down_proj(Xs, stack_down(L1, A))
    Y = Xh @ Wh.T + q.bf16_bits_to_f64(U) @ stack_up(L2, B)
    return Y, U


def linear_bwd_rows(rows, dY, w_codes, w_scales, L1, L2, A, B, precision="W4A4G4",
                    w_block="tile32", wt=None):
    """Float64 dX before rounding, and P, for selected rows only."""
    _check_precision(precision)
    Gs = np.asarray(dY)[rows]
    if "G16" in precision:
        Gh = q.bf16_bits_to_f64(Gs)
    else:
        gq_codes, gq_scales = q.quantize_row32(Gs)
        Gh = q.dequantize_row32(gq_codes, gq_scales)
    Wh = weight_dgrad(w_codes, w_scales, w_block, wt)
    P = down_proj(Gs, stack_up(L2, B).T)
    dX = Gh @ Wh + q.bf16_bits_to_f64(P) @ stack_down(L1, A).T
    return dX, P


def _sigmoid(z):
    """1 / (1 + exp(-z)) without overflow for either sign of z."""
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gelu_tanh(h_bits: np.ndarray) -> np.ndarray:
    """tanh-form GELU of bf16 input, evaluated in float64, rounded to bf16.

    0.5 h (1 + tanh(u)), u = sqrt(2/pi) (h + 0.044715 h^3): the activation
    between the two MLP linears ("MLP Fusion" names GeLU on the wide
    intermediate).  0.5 (1 + tanh(u)) is evaluated as sigmoid(2u), the same
    number without the cancellation of 1 + tanh(u) for very negative u.
    """
    h = q.bf16_bits_to_f64(h_bits)
    u = np.sqrt(2.0 / np.pi) * (h + 0.044715 * h ** 3)
    return q.f64_to_bf16_bits(h * _sigmoid(2.0 * u))


def gelu_tanh_grad(h_bits: np.ndarray, g_bits: np.ndarray) -> np.ndarray:
    """bf16(g * d/dh gelu_tanh(h)) for bf16 h and incoming gradient g.

    d/dh = s + h s (1 - s) 2 c (1 + 3 * 0.044715 h^2) with s = sigmoid(2u),
    c = sqrt(2/pi); (1 - tanh^2 u) / 2 = 2 s (1 - s).
    """
    h = q.bf16_bits_to_f64(h_bits)
    c = np.sqrt(2.0 / np.pi)
    u = c * (h + 0.044715 * h ** 3)
    s = _sigmoid(2.0 * u)
    sm = _sigmoid(-2.0 * u)                      # 1 - s without cancellation
    d = s + h * s * sm * 2.0 * c * (1.0 + 3.0 * 0.044715 * h ** 2)
    return q.f64_to_bf16_bits(q.bf16_bits_to_f64(g_bits) * d)


def rel_frobenius(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_F / ||ref||_F (0 when both are zero)."""
    got = out_to_f64(got)
    ref = out_to_f64(ref)
    den = np.linalg.norm(ref)
    num = np.linalg.norm(got - ref)
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
