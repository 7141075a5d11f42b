"""Seeded synthetic inputs for the W4A4G4 triple-branch linear.

This module only draws random numbers and rounds them to bf16; it holds
none of the layer's arithmetic (no quantization, no products of the
method).  Both the HIP path and the CPU oracle receive the arrays it makes.

The workloads stand in for the layers of FLUX.1-dev that FourTune trains
(FourTune, arXiv 2607.05711, "4.2 Main Results", efficiency at 1024x1024:
4096 image + 512 text tokens per image; "MLP Fusion": model width 3072 and
FFN width 12288).  No model weights or datasets are used.

Offline weight preparation of the tiny case follows the paper's spectral
split (Eq. (1), "3.1 Triple-Branch Hybrid-Precision Pipeline"): a rank-r SVD
of W gives the frozen stabilizer L1 L2 and W_res = W - (L1 L2)^T.  That split
happens once per layer, before the hot path, and is done here with a
library SVD to build inputs; neither side of the parity tests computes it.

Arrays are numpy: bf16 tensors are uint16 bit patterns.  Rounding to bf16
uses torch's CPU cast (round to nearest, ties to even).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32/float64 values to bf16 and return the bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class LinearCase:
    """One triple-branch linear: shapes, frozen/trainable weights, X and dY."""
    name: str
    M: int
    K: int
    N: int
    r_s: int
    r_l: int
    X: np.ndarray        # bf16 [M, K]
    W_res: np.ndarray    # bf16 [N, K]
    L1: np.ndarray       # bf16 [K, r_s]
    L2: np.ndarray       # bf16 [r_s, N]
    A: np.ndarray        # bf16 [K, r_l]
    B: np.ndarray        # bf16 [r_l, N]
    dY: np.ndarray       # bf16 [M, N]
    meta: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return self.r_s + self.r_l


def _normal(rng, shape, std=1.0):
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def _orthonormal_cols(rng, n, r):
    if r == 0:
        return np.zeros((n, 0))
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q


def _outlier_channels(rng, X, n_channels, factor):
    if n_channels:
        cols = rng.choice(X.shape[1], size=n_channels, replace=False)
        X[:, cols] *= np.float32(factor)
    return X


def tiny_case(seed: int = 0, M: int = 128, K: int = 256, N: int = 256,
              r_s: int = 16, r_l: int = 8) -> LinearCase:
    """Tiny linear with a spectrally-split weight (SVD stabilizer).

    X ~ N(0,1) with 2 channels x40; W = U0 diag(5*0.7^i) V0^T + N(0, 0.02);
    the top-r_s SVD of W is the stabilizer, W_res = W - (L1 L2)^T;
    A, B ~ 0.01 N(0,1); dY ~ 1e-3 N(0,1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _outlier_channels(rng, _normal(rng, (M, K)), 2, 40.0)
    n_spec = 16
    U0 = _orthonormal_cols(rng, N, n_spec)
    V0 = _orthonormal_cols(rng, K, n_spec)
    s = 5.0 * 0.7 ** np.arange(n_spec)
    W = (U0 * s) @ V0.T + 0.02 * rng.standard_normal((N, K))       # [N, K]
    Uw, Sw, Vwt = np.linalg.svd(W, full_matrices=False)
    sq = np.sqrt(Sw[:r_s])
    L1 = to_bf16_bits(Vwt[:r_s].T * sq)                            # [K, r_s]
    L2 = to_bf16_bits(sq[:, None] * Uw[:, :r_s].T)                 # [r_s, N]
    L1f = bf16_bits_to_f32(L1).astype(np.float64)
    L2f = bf16_bits_to_f32(L2).astype(np.float64)
    W_res = to_bf16_bits(W - (L1f @ L2f).T)
    A = to_bf16_bits(_normal(rng, (K, r_l), 0.01))
    B = to_bf16_bits(_normal(rng, (r_l, N), 0.01))
    dY = to_bf16_bits(_normal(rng, (M, N), 1e-3))
    return LinearCase("tiny", M, K, N, r_s, r_l, to_bf16_bits(X), W_res, L1, L2, A, B, dY,
                      meta={"seed": seed})


def flux_linear_case(name: str, M: int, K: int, N: int, r_s: int, r_l: int,
                     seed: int, x_kind: str = "outlier", outlier_frac: float = 0.01,
                     outlier_factor: float = 50.0) -> LinearCase:
    """A FLUX-shaped linear with synthetic weights.

    X ~ N(0,1) with round(outlier_frac*K) channels scaled by outlier_factor
    ('outlier'), or a non-negative heavy-tailed gate-like activation
    ('gated': 0.5 h (1 + tanh(0.8 h)) of such an X; it stands in for the
    activation the down-projection of an MLP receives).  W_res ~ N(0, 0.02);
    L1 = Q_K diag(sqrt s), L2 = diag(sqrt s) Q_N^T with s_i = 8 * 0.8^i and
    Q_K, Q_N orthonormal; A, B ~ 0.01 N(0,1); dY ~ 1e-3 N(0,1).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = _outlier_channels(rng, _normal(rng, (M, K)), int(round(outlier_frac * K)), outlier_factor)
    if x_kind == "gated":
        X = 0.5 * X * (1.0 + np.tanh(np.float32(0.8) * X))
    elif x_kind != "outlier":
        raise ValueError(x_kind)
    W_res = to_bf16_bits(_normal(rng, (N, K), 0.02))
    s = 8.0 * 0.8 ** np.arange(r_s)
    L1 = to_bf16_bits(_orthonormal_cols(rng, K, r_s) * np.sqrt(s))
    L2 = to_bf16_bits((_orthonormal_cols(rng, N, r_s) * np.sqrt(s)).T)
    A = to_bf16_bits(_normal(rng, (K, r_l), 0.01))
    B = to_bf16_bits(_normal(rng, (r_l, N), 0.01))
    dY = to_bf16_bits(_normal(rng, (M, N), 1e-3))
    return LinearCase(name, M, K, N, r_s, r_l, to_bf16_bits(X), W_res, L1, L2, A, B, dY,
                      meta={"seed": seed, "x_kind": x_kind})


def outlier_weight_cases(seed: int = 5, M: int = 128, K: int = 256, N: int = 256,
                         r_s: int = 16, n_out: int = 4, out_scale: float = 8.0):
    """The stabilizer ablation: one weight, quantized with and without it.

    W = N(0, 0.02) + sum of n_out rank-1 terms out_scale * u e_c^T, each on
    one input channel c (u a random unit vector): a few weight columns carry
    entries ~25x the rest, as outlier channels do.  X ~ N(0,1) with 2 input
    channels x40, dY ~ 1e-3 N(0,1).  Returns (with, without): `with` keeps
    the top-r_s SVD of W as the stabilizer (L1, L2) and quantizes only the
    residual; `without` quantizes W itself (r_s = 0).  Neither has an
    adapter.  meta["W"] is W in bf16, the weight both stand for.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    X = to_bf16_bits(_outlier_channels(rng, _normal(rng, (M, K)), 2, 40.0))
    W = 0.02 * rng.standard_normal((N, K))
    for c in rng.choice(K, n_out, replace=False):
        u = rng.standard_normal(N)
        W[:, c] += out_scale * u / np.linalg.norm(u)
    dY = to_bf16_bits(_normal(rng, (M, N), 1e-3))
    Wb = to_bf16_bits(W)
    Wf = bf16_bits_to_f32(Wb).astype(np.float64)
    Uw, Sw, Vwt = np.linalg.svd(Wf, full_matrices=False)
    sq = np.sqrt(Sw[:r_s])
    L1 = to_bf16_bits(Vwt[:r_s].T * sq)                            # [K, r_s]
    L2 = to_bf16_bits(sq[:, None] * Uw[:, :r_s].T)                 # [r_s, N]
    W_res = to_bf16_bits(Wf - (bf16_bits_to_f32(L1).astype(np.float64)
                               @ bf16_bits_to_f32(L2).astype(np.float64)).T)
    noA = np.zeros((K, 0), np.uint16)
    noB = np.zeros((0, N), np.uint16)
    meta = {"seed": seed, "W": Wb}
    with_stab = LinearCase("outlier_w_stab", M, K, N, r_s, 0, X, W_res, L1, L2, noA, noB, dY,
                           meta=dict(meta))
    without = LinearCase("outlier_w_nostab", M, K, N, 0, 0, X, Wb, np.zeros((K, 0), np.uint16),
                         np.zeros((0, N), np.uint16), noA, noB, dY, meta=dict(meta))
    return with_stab, without


def qkv_case(seed: int = 1) -> LinearCase:
    """FLUX fused QKV projection: 4608 tokens, 3072 -> 9216, r_s=32, r_l=16."""
    return flux_linear_case("qkv_4608x3072x9216", 4608, 3072, 9216, 32, 16, seed)


def mlp_cases(seed: int = 2):
    """FLUX MLP pair: up 3072 -> 12288 and down 12288 -> 3072, 4608 tokens, ranks 32/32."""
    up = flux_linear_case("mlp_up_4608x3072x12288", 4608, 3072, 12288, 32, 32, seed)
    down = flux_linear_case("mlp_down_4608x12288x3072", 4608, 12288, 3072, 32, 32, seed + 1000,
                            x_kind="gated")
    return up, down


def dit_block_linears():
    """Shapes of every linear of one double-stream DiT block at batch 2.

    Per stream (image: 2 x 4096 tokens, text: 2 x 512 tokens): QKV
    3072->9216, out-projection 3072->3072, MLP 3072->12288->3072; plus one
    modulation linear 3072->18432 per stream at M=2.  r_s=32, r_l=16.
    Returns (name, M, K, N) tuples.
    """
    out = []
    for stream, M in (("img", 8192), ("txt", 1024)):
        out += [(f"{stream}_qkv", M, 3072, 9216), (f"{stream}_out", M, 3072, 3072),
                (f"{stream}_fc1", M, 3072, 12288), (f"{stream}_fc2", M, 12288, 3072),
                (f"{stream}_mod", 2, 3072, 18432)]
    return out


def dit_block_case(name: str, seed: int = 3) -> LinearCase:
    """One linear of the DiT block, drawn independently (seed offset by index)."""
    shapes = dit_block_linears()
    idx = [s[0] for s in shapes].index(name)
    _, M, K, N = shapes[idx]
    kind = "gated" if name.endswith("fc2") else "outlier"
    return flux_linear_case(f"dit_{name}_{M}x{K}x{N}", M, K, N, 32, 16, seed * 100 + idx,
                            x_kind=kind)


def stress_activation(seed: int = 4, rows: int = 16384, cols: int = 12288,
                      zero_tile_frac: float = 0.01) -> np.ndarray:
    """Quantizer stress tensor, bf16 [rows, cols].

    1e-3 * Student-t(3); 0.1% of entries x1e3; zero_tile_frac of the 32x32
    tiles set to zero, so all-zero 32-blocks occur along both axes.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    z = rng.standard_normal((rows, cols), dtype=np.float32)
    chi2 = rng.standard_gamma(1.5, size=(rows, cols), dtype=np.float32) * np.float32(2.0)
    T = z / np.sqrt(chi2 / np.float32(3.0)) * np.float32(1e-3)
    del z, chi2
    n_out = int(round(0.001 * rows * cols))
    idx = rng.choice(rows * cols, size=n_out, replace=False)
    T.reshape(-1)[idx] *= np.float32(1e3)
    tr, tc = rows // 32, cols // 32
    n_zero = int(round(zero_tile_frac * tr * tc))
    tiles = rng.choice(tr * tc, size=n_zero, replace=False)
    T4 = T.reshape(tr, 32, tc, 32)
    T4[tiles // tc, :, tiles % tc, :] = 0.0
    return to_bf16_bits(T)


def stress_weight(seed: int = 4, n: int = 12288) -> np.ndarray:
    """Weight for the 32x32-tile quantizer stress: bf16 [n, n] ~ N(0, 0.02)."""
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    return to_bf16_bits(_normal(rng, (n, n), 0.02))


def adversarial_blocks(seed: int, n_blocks: int) -> np.ndarray:
    """bf16 rows of 32 elements exercising the encoder's corner cases.

    Mixes exact rounding ties (k/4 * 2^e for odd k), values just above and
    below ties, +-0, bf16 subnormals, saturating values in (6, 8) * 2^e,
    all-zero blocks and blocks spanning many decades.  [n_blocks, 32].
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((n_blocks, 32), dtype=np.uint16)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 7.5, 0.5, 1.0, 3.0, 4.0])
    for b in range(n_blocks):
        kind = b % 6
        e = int(rng.integers(-40, 40))
        if kind == 0:      # exact ties and grid points at a shared exponent, amax forced to 6
            v = rng.choice(ties[:8], 32) * np.where(rng.random(32) < 0.5, -1.0, 1.0)
            v[0] = 6.0
            bits = to_bf16_bits(np.ldexp(v, e))
        elif kind == 1:    # neighbours of ties: +-1 bf16 ulp
            v = to_bf16_bits(np.ldexp(rng.choice(ties, 32), e)).astype(np.int32)
            v += rng.integers(-1, 2, 32)
            v[0] = to_bf16_bits(np.ldexp(np.array([7.5]), e))[0]
            bits = (v.astype(np.uint16) | (rng.integers(0, 2, 32) << 15).astype(np.uint16))
        elif kind == 2:    # bf16 subnormals and tiny normals (scale clamps at 2^-127)
            bits = rng.integers(0, 0x0200, 32).astype(np.uint16)
            bits |= (rng.integers(0, 2, 32) << 15).astype(np.uint16)
        elif kind == 3:    # all-zero block with mixed signs of zero
            bits = (rng.integers(0, 2, 32) << 15).astype(np.uint16)
        elif kind == 4:    # very large magnitudes (scale near the top of E8M0)
            mag = rng.integers(0x7E00, 0x7F80, 32).astype(np.uint16)
            bits = mag | (rng.integers(0, 2, 32) << 15).astype(np.uint16)
        else:              # many decades in one block
            v = rng.standard_normal(32) * np.exp2(rng.uniform(-30, 30, 32))
            bits = to_bf16_bits(v)
        out[b] = bits
    return out
