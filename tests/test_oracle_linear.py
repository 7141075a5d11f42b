"""Pins for the oracle's triple-branch forward and backward (CPU only).

* integer-valued inputs on which every rounding is exact, so the oracle's
  Y, dX, dA, dB must equal torch float64 autograd of the plain layer
  Y = X W^T + (X L1) L2 + (X A) B with loss <dY, Y> exactly;
* brute-force exact triple loops (Python Fractions) on tiny inputs;
* branch structure: zero ranks, zero residual;
* the adjoint identity of the backbone product;
* autograd on random inputs within bf16 rounding error;
* group-wise (1x32) weights of the block-shape ablation: both products
  against nibble-by-nibble triple loops, the dgrad reading its own
  quantization of W^T, and exact autograd on lossless inputs;
* the precision settings of Table 4: exact agreement with autograd where
  the 16-bit side reads its input unquantized, disagreement where a 4-bit
  side rounds a lossy block;
* GELU against torch's float64 tanh-GELU and its autograd.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import linear as L
from oracle import mxfp4 as q
from bit_quantized_amd import synth


def _ternary(rng, shape):
    return synth.to_bf16_bits(rng.integers(-1, 2, size=shape).astype(np.float32))


def _case_ternary(seed, M, K, N, r_s, r_l):
    rng = np.random.default_rng(seed)
    return dict(X=_ternary(rng, (M, K)), W=_ternary(rng, (N, K)), L1=_ternary(rng, (K, r_s)),
                L2=_ternary(rng, (r_s, N)), A=_ternary(rng, (K, r_l)), B=_ternary(rng, (r_l, N)),
                dY=_ternary(rng, (M, N)))


def _autograd(c):
    f = lambda b: torch.from_numpy(q.bf16_bits_to_f64(b))
    X = f(c["X"]).requires_grad_(True)
    A = f(c["A"]).requires_grad_(True)
    B = f(c["B"]).requires_grad_(True)
    W, L1, L2, dY = f(c["W"]), f(c["L1"]), f(c["L2"]), f(c["dY"])
    Y = X @ W.T + (X @ L1) @ L2 + (X @ A) @ B
    (Y * dY).sum().backward()
    return Y.detach().numpy(), X.grad.numpy(), A.grad.numpy(), B.grad.numpy()


@pytest.mark.parametrize("shape", [(8, 64, 96, 4, 3), (5, 32, 32, 0, 2), (7, 96, 64, 3, 0)])
def test_exact_against_autograd_on_ternary_inputs(shape):
    # Ternary blocks are lossless under MXFP4 (amax 1 -> scale 2^-2, codes 0/+-6
    # i.e. +-4*2^-2), and every low-rank intermediate is a small integer, so bf16
    # rounding of U and P is exact; outputs are compared unrounded (f64).
    M, K, N, r_s, r_l = shape
    c = _case_ternary(sum(shape), M, K, N, r_s, r_l)
    wc, ws = q.quantize_tile32(c["W"])
    np.testing.assert_array_equal(q.dequantize_tile32(wc, ws), q.bf16_bits_to_f64(c["W"]))
    fwd = L.linear_fwd(c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], out_dtype="f64")
    bwd = L.linear_bwd(c["dY"], c["X"], fwd["U"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                       out_dtype="f64", grad_dtype="f64")
    Y, dX, dA, dB = _autograd(c)
    np.testing.assert_array_equal(fwd["Y"], Y)
    np.testing.assert_array_equal(bwd["dX"], dX)
    np.testing.assert_array_equal(bwd["dA"], dA)
    np.testing.assert_array_equal(bwd["dB"], dB)


@pytest.mark.parametrize("precision", L.PRECISIONS)
def test_precision_settings_exact_on_lossless_inputs(precision):
    # On ternary inputs Q(X) = X and Q(dY) = dY, so every precision setting
    # gives the same exact result as the plain layer's autograd.
    c = _case_ternary(11, 8, 64, 96, 4, 3)
    wc, ws = q.quantize_tile32(c["W"])
    fwd = L.linear_fwd(c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], out_dtype="f64",
                       precision=precision)
    bwd = L.linear_bwd(c["dY"], c["X"], fwd["U"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                       out_dtype="f64", grad_dtype="f64", precision=precision)
    Y, dX, dA, dB = _autograd(c)
    np.testing.assert_array_equal(fwd["Y"], Y)
    np.testing.assert_array_equal(bwd["dX"], dX)
    np.testing.assert_array_equal(bwd["dA"], dA)
    np.testing.assert_array_equal(bwd["dB"], dB)
    assert (fwd["xq_codes"] is None) == ("A16" in precision)
    assert (bwd["gq_codes"] is None) == ("G16" in precision)


@pytest.mark.parametrize("precision", L.PRECISIONS)
def test_precision_settings_on_lossy_integer_inputs(precision):
    # X and dY are integers in [-7, 7]: a block holding a 7 is lossy under
    # MXFP4 (scale 1, 7 rounds to 6), while the ternary weight stays exact.
    # With K = N = 32 every sum is an integer below 2^8, so U and P are exact
    # in bf16 and the plain layer's autograd is exact: a 16-bit side must
    # equal it, a 4-bit side must not.
    rng = np.random.default_rng(5)
    M, K, N, r_s, r_l = 8, 32, 32, 2, 3
    ints = lambda shape: synth.to_bf16_bits(rng.integers(-7, 8, size=shape).astype(np.float32))
    c = dict(X=ints((M, K)), W=_ternary(rng, (N, K)), L1=_ternary(rng, (K, r_s)),
             L2=_ternary(rng, (r_s, N)), A=_ternary(rng, (K, r_l)), B=_ternary(rng, (r_l, N)),
             dY=ints((M, N)))
    c["X"][:, 0] = synth.to_bf16_bits(np.float32(7.0))     # every block lossy
    c["dY"][:, 0] = synth.to_bf16_bits(np.float32(-7.0))
    wc, ws = q.quantize_tile32(c["W"])
    fwd = L.linear_fwd(c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], out_dtype="f64",
                       precision=precision)
    bwd = L.linear_bwd(c["dY"], c["X"], fwd["U"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                       out_dtype="f64", grad_dtype="f64", precision=precision)
    Y, dX, dA, dB = _autograd(c)
    assert np.array_equal(fwd["Y"], Y) == ("A16" in precision)
    assert np.array_equal(bwd["dX"], dX) == ("G16" in precision)
    # the adapter gradients and the low-rank branches do not depend on it
    np.testing.assert_array_equal(bwd["dA"], dA)
    np.testing.assert_array_equal(bwd["dB"], dB)
    base_f = L.linear_fwd(c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], out_dtype="f64")
    base_b = L.linear_bwd(c["dY"], c["X"], base_f["U"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                          out_dtype="f64", grad_dtype="f64")
    assert np.array_equal(fwd["Y"], base_f["Y"]) == ("A16" not in precision)
    assert np.array_equal(bwd["dX"], base_b["dX"]) == ("G16" not in precision)
    # row-sampled forms agree with the full ones
    rows = np.array([0, 5, 7])
    Yr, _ = L.linear_fwd_rows(rows, c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                              precision=precision)
    dXr, _ = L.linear_bwd_rows(rows, c["dY"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                               precision=precision)
    np.testing.assert_array_equal(Yr, fwd["Y"][rows])
    np.testing.assert_array_equal(dXr, bwd["dX"][rows])


def test_against_autograd_random_inputs_within_bf16_error():
    c = synth.tiny_case(seed=0, M=16, K=64, N=96, r_s=4, r_l=4)
    cc = dict(X=c.X, W=c.W_res, L1=c.L1, L2=c.L2, A=c.A, B=c.B, dY=c.dY)
    wc, ws = q.quantize_tile32(c.W_res)
    fwd = L.linear_fwd(c.X, wc, ws, c.L1, c.L2, c.A, c.B, out_dtype="f64")
    bwd = L.linear_bwd(c.dY, c.X, fwd["U"], wc, ws, c.L1, c.L2, c.A, c.B,
                       out_dtype="f64", grad_dtype="f64")
    # Autograd of the unquantized layer differs by the 4-bit quantization
    # error of the backbone; compare the low-rank gradients (no quantizer in
    # their path) tightly and the full outputs loosely.
    _, _, dA, dB = _autograd(cc)
    assert L.rel_frobenius(bwd["dA"], dA) < 1e-2
    assert L.rel_frobenius(bwd["dB"], dB) < 1e-2


def _exact(b):
    return [[Fraction(float(v)) for v in row] for row in q.bf16_bits_to_f64(b)]


def test_brute_force_backbone_triple_loop():
    rng = np.random.default_rng(21)
    M, K, N = 3, 64, 32
    X = synth.to_bf16_bits(rng.standard_normal((M, K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.1)
    wc, ws = q.quantize_tile32(W)
    xc, xs = q.quantize_row32(X)
    z = lambda r, c: np.zeros((r, c), dtype=np.uint16)
    fwd = L.linear_fwd(X, wc, ws, z(K, 0), z(0, N), z(K, 0), z(0, N), out_dtype="f64")
    # decode each 4-bit code by hand from its nibble and its block's scale byte
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]

    def val(code, sc):
        v = grid[code & 7] * (Fraction(2) ** (int(sc) - 127))
        return -v if code & 8 else v

    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                cx = (int(xc[m, k // 2]) >> (4 * (k % 2))) & 0xF
                cw = (int(wc[n, k // 2]) >> (4 * (k % 2))) & 0xF
                acc += val(cx, xs[m, k // 32]) * val(cw, ws[n // 32, k // 32])
            assert float(acc) == fwd["Y"][m, n]


def test_brute_force_low_rank_branches():
    rng = np.random.default_rng(22)
    M, K, N, r_s, r_l = 2, 32, 32, 2, 3
    X = synth.to_bf16_bits(rng.standard_normal((M, K)))
    L1 = synth.to_bf16_bits(rng.standard_normal((K, r_s)))
    L2 = synth.to_bf16_bits(rng.standard_normal((r_s, N)))
    A = synth.to_bf16_bits(rng.standard_normal((K, r_l)))
    B = synth.to_bf16_bits(rng.standard_normal((r_l, N)))
    W0 = np.zeros((N, K), dtype=np.uint16)
    wc, ws = q.quantize_tile32(W0)
    fwd = L.linear_fwd(X, wc, ws, L1, L2, A, B, out_dtype="f64")
    Xe, L1e, L2e, Ae, Be = map(_exact, (X, L1, L2, A, B))
    for m in range(M):
        u = [sum(Xe[m][k] * L1e[k][j] for k in range(K)) for j in range(r_s)] + \
            [sum(Xe[m][k] * Ae[k][j] for k in range(K)) for j in range(r_l)]
        # U is rounded to bf16 once
        u16 = q.f64_to_bf16_bits(np.array([float(x) for x in u]))
        np.testing.assert_array_equal(fwd["U"][m], u16)
        ue = [Fraction(float(x)) for x in q.bf16_bits_to_f64(u16)]
        Ve = L2e + Be
        for n in range(N):
            y = sum(ue[j] * Ve[j][n] for j in range(r_s + r_l))
            assert abs(float(y) - fwd["Y"][m, n]) <= 1e-12 * max(1.0, abs(float(y)))


def test_zero_ranks_is_pure_backbone_and_zero_residual_is_pure_low_rank():
    c = synth.tiny_case(seed=3, M=8, K=64, N=64, r_s=4, r_l=2)
    wc, ws = q.quantize_tile32(c.W_res)
    z = lambda r, cc: np.zeros((r, cc), dtype=np.uint16)
    f0 = L.linear_fwd(c.X, wc, ws, z(64, 0), z(0, 64), z(64, 0), z(0, 64), out_dtype="f64")
    xc, xs = q.quantize_row32(c.X)
    np.testing.assert_array_equal(f0["Y"], q.dequantize_row32(xc, xs) @ q.dequantize_tile32(wc, ws).T)
    wz, sz = q.quantize_tile32(np.zeros_like(c.W_res))
    f1 = L.linear_fwd(c.X, wz, sz, c.L1, c.L2, c.A, c.B, out_dtype="f64")
    np.testing.assert_allclose(f1["Y"], q.bf16_bits_to_f64(f1["U"]) @
                               np.concatenate([q.bf16_bits_to_f64(c.L2), q.bf16_bits_to_f64(c.B)]),
                               rtol=0, atol=1e-12)


def test_backbone_adjoint_identity():
    # <G, Xh Wh^T> == <G Wh, Xh> with the dequantized operands (float64).
    c = synth.tiny_case(seed=4, M=32, K=96, N=64, r_s=0, r_l=0)
    wc, ws = q.quantize_tile32(c.W_res)
    f = L.linear_fwd(c.X, wc, ws, c.L1, c.L2, c.A, c.B, out_dtype="f64")
    b = L.linear_bwd(c.dY, c.X, f["U"], wc, ws, c.L1, c.L2, c.A, c.B, out_dtype="f64",
                     grad_dtype="f64")
    Gh = q.dequantize_row32(b["gq_codes"], b["gq_scales"])
    Xh = q.dequantize_row32(f["xq_codes"], f["xq_scales"])
    lhs = np.sum(Gh * f["Y"])
    rhs = np.sum(b["dX"] * Xh)
    assert abs(lhs - rhs) <= 1e-12 * (abs(lhs) + 1e-30)


def test_row_sampled_forms_match_full():
    c = synth.tiny_case(seed=5, M=40, K=64, N=96, r_s=4, r_l=4)
    wc, ws = q.quantize_tile32(c.W_res)
    f = L.linear_fwd(c.X, wc, ws, c.L1, c.L2, c.A, c.B, out_dtype="f64")
    b = L.linear_bwd(c.dY, c.X, f["U"], wc, ws, c.L1, c.L2, c.A, c.B, out_dtype="f64")
    rows = np.array([0, 7, 39])
    Y, U = L.linear_fwd_rows(rows, c.X, wc, ws, c.L1, c.L2, c.A, c.B)
    dX, P = L.linear_bwd_rows(rows, c.dY, wc, ws, c.L1, c.L2, c.A, c.B)
    np.testing.assert_array_equal(Y, f["Y"][rows])
    np.testing.assert_array_equal(U, f["U"][rows])
    np.testing.assert_array_equal(dX, b["dX"][rows])
    np.testing.assert_array_equal(P, b["P"][rows])


def test_gelu_against_torch():
    # Where torch's float64 1 + tanh(u) does not cancel (h > -5) its tanh-GELU
    # and autograd must round to the same bf16; in the far negative tail the
    # values are checked against a scalar high-precision evaluation instead.
    rng = np.random.default_rng(30)
    h = synth.to_bf16_bits(rng.standard_normal(50000) * 4)
    hf = q.bf16_bits_to_f64(h)
    ok = hf > -5.0
    ht = torch.from_numpy(hf).requires_grad_(True)
    g = torch.nn.functional.gelu(ht, approximate="tanh")
    np.testing.assert_array_equal(L.gelu_tanh(h)[ok], q.f64_to_bf16_bits(g.detach().numpy())[ok])
    up = synth.to_bf16_bits(rng.standard_normal(50000))
    g.backward(torch.from_numpy(q.bf16_bits_to_f64(up)))
    np.testing.assert_array_equal(L.gelu_tanh_grad(h, up)[ok],
                                  q.f64_to_bf16_bits(ht.grad.numpy())[ok])
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    c = (Decimal(2) / Decimal(str(np.pi))).sqrt()
    for x in hf[~ok][:200]:
        d = Decimal(float(x))
        u = c * (d + Decimal("0.044715") * d ** 3)
        tanh = ((2 * u).exp() - 1) / ((2 * u).exp() + 1)
        ref = float(Decimal("0.5") * d * (1 + tanh))
        got = q.bf16_bits_to_f64(L.gelu_tanh(synth.to_bf16_bits(np.array([x]))))[0]
        assert got == q.bf16_bits_to_f64(q.f64_to_bf16_bits(np.array([ref])))[0]


def test_rel_frobenius_basic():
    a = np.array([3.0, 4.0])
    assert L.rel_frobenius(a, a) == 0.0
    assert abs(L.rel_frobenius(np.array([3.0, 4.5]), a) - 0.1) < 1e-15


# ---------------------------------------------------------------- row32 weights
def _val(code, sc):
    """One E2M1 code times its E8M0 scale, decoded by hand (exact)."""
    grid = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
            Fraction(3), Fraction(4), Fraction(6)]
    v = grid[code & 7] * (Fraction(2) ** (int(sc) - 127))
    return -v if code & 8 else v


def _nib(codes, r, c):
    return (int(codes[r, c // 2]) >> (4 * (c % 2))) & 0xF


def test_row32_weights_brute_force_both_products():
    # Group-wise weights (the block-shape ablation's alternative): the forward
    # reads Q_row32(W) with blocks along K, the dgrad Q_row32(W^T) with blocks
    # along N; both decoded here nibble by nibble.
    rng = np.random.default_rng(31)
    M, K, N = 3, 64, 64
    X = synth.to_bf16_bits(rng.standard_normal((M, K)))
    dY = synth.to_bf16_bits(rng.standard_normal((M, N)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.1 *
                           np.exp2(rng.integers(-6, 6, size=(N, 1))))    # rows of different scale
    wc, ws = q.quantize_row32(W)
    wt = q.quantize_row32(np.ascontiguousarray(W.T))
    z = lambda r, c: np.zeros((r, c), dtype=np.uint16)
    fwd = L.linear_fwd(X, wc, ws, z(K, 0), z(0, N), z(K, 0), z(0, N), out_dtype="f64",
                       w_block="row32")
    bwd = L.linear_bwd(dY, X, fwd["U"], wc, ws, z(K, 0), z(0, N), z(K, 0), z(0, N),
                       out_dtype="f64", w_block="row32", wt=wt)
    xc, xs = q.quantize_row32(X)
    gc, gs = q.quantize_row32(dY)
    for m in range(M):
        for n in range(N):
            acc = sum(_val(_nib(xc, m, k), xs[m, k // 32]) * _val(_nib(wc, n, k), ws[n, k // 32])
                      for k in range(K))
            assert float(acc) == fwd["Y"][m, n]
        for k in range(K):
            acc = sum(_val(_nib(gc, m, n), gs[m, n // 32]) * _val(_nib(wt[0], k, n), wt[1][k, n // 32])
                      for n in range(N))
            assert float(acc) == bwd["dX"][m, k]
    # rows of different scale make the two groupings differ: the dgrad reads
    # its own quantization of W^T, not the forward's numbers
    assert not np.array_equal(L.weight_dgrad(wc, ws, "row32", wt), L.weight_fwd(wc, ws, "row32"))


def test_row32_weights_exact_on_ternary_inputs():
    c = _case_ternary(13, 8, 64, 96, 4, 3)
    wc, ws = q.quantize_row32(c["W"])
    wt = q.quantize_row32(np.ascontiguousarray(c["W"].T))
    fwd = L.linear_fwd(c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], out_dtype="f64",
                       w_block="row32")
    bwd = L.linear_bwd(c["dY"], c["X"], fwd["U"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                       out_dtype="f64", grad_dtype="f64", w_block="row32", wt=wt)
    Y, dX, dA, dB = _autograd(c)
    np.testing.assert_array_equal(fwd["Y"], Y)
    np.testing.assert_array_equal(bwd["dX"], dX)
    np.testing.assert_array_equal(bwd["dA"], dA)
    np.testing.assert_array_equal(bwd["dB"], dB)
    rows = np.array([1, 6])
    Yr, _ = L.linear_fwd_rows(rows, c["X"], wc, ws, c["L1"], c["L2"], c["A"], c["B"], w_block="row32")
    dXr, _ = L.linear_bwd_rows(rows, c["dY"], wc, ws, c["L1"], c["L2"], c["A"], c["B"],
                               w_block="row32", wt=wt)
    np.testing.assert_array_equal(Yr, Y[rows])
    np.testing.assert_array_equal(dXr, dX[rows])
    with pytest.raises(ValueError):
        L.weight_dgrad(wc, ws, "row32")
