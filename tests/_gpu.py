"""Helpers for the GPU parity tests: upload a synthetic case, run the layer
through the C ABI, and compare with the CPU oracle."""
import sys

import numpy as np
import pytest
import torch

from bit_quantized_amd import ops
from bit_quantized_amd.layer import QuantizedLinear, bf16_tensor, bits_of
from oracle import linear as OL
from oracle import mxfp4 as OQ

DEV = torch.device("cuda:0")
REL_TOL = 1e-3          # relative Frobenius bar for Y, dX, dA, dB


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ops.lib()  # fail loudly when the library is missing


def up(bits):
    return bf16_tensor(bits, DEV)


def u8(t):
    return None if t is None else t.detach().cpu().numpy()


class GpuCase:
    """A LinearCase resident on the device with its quantized weight."""

    def __init__(self, case, precision="W4A4G4", w_block="tile32"):
        self.c = case
        self.precision = precision
        self.w_block = w_block
        self.X = up(case.X)
        self.dY = up(case.dY)
        W = up(case.W_res)
        opt = lambda a: up(a) if a.size else None
        self.layer = QuantizedLinear.from_factors(W, opt(case.L1) if case.r_s else None,
                                                  opt(case.L2) if case.r_s else None,
                                                  opt(case.A) if case.r_l else None,
                                                  opt(case.B) if case.r_l else None,
                                                  precision=precision, w_block=w_block)
        del W

    def run(self, grad_f32=False):
        Y, U, xc, xs = self.layer.forward(self.X, want_codes=True)
        dX, dA, dB, P, gc, gs = self.layer.backward(self.dY, self.X, U, grad_f32=grad_f32,
                                                    want_codes=True)
        torch.cuda.synchronize()
        out = dict(Y=bits_of(Y), U=bits_of(U)[:, :self.c.R] if self.c.R else None,
                   xq_codes=u8(xc), xq_scales=u8(xs), dX=bits_of(dX),
                   P=bits_of(P)[:, :self.c.R] if self.c.R else None, gq_codes=u8(gc),
                   gq_scales=u8(gs), w_codes=u8(self.layer.w_codes),
                   w_scales=u8(self.layer.w_scales), wt_codes=u8(self.layer.wt_codes),
                   wt_scales=u8(self.layer.wt_scales), w_block=self.w_block)
        # dA comes back as dA^T [r_l, K] (the layout of the stored A^T)
        if self.c.r_l:
            if grad_f32:
                out["dA"] = np.ascontiguousarray(dA.cpu().numpy().T)
                out["dB"] = dB.cpu().numpy()
            else:
                out["dA"] = np.ascontiguousarray(bits_of(dA).T)
                out["dB"] = bits_of(dB)
        return out


def bit_agreement(a, b):
    if a is None or a.size == 0:
        return 1.0
    return float(np.mean(a == b))


def _ordinal(x):
    """Output values as integers ordered like the values, one apart for
    neighbouring representable numbers (bf16 bits or float32; +0 == -0)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        b = x.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    b = x.astype(np.float32).view(np.int32).astype(np.int64)
    return np.where(b < 0, -(b & 0x7FFFFFFF), b)


def _values(x):
    x = np.asarray(x)
    return OQ.bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _half_ulp(v, mant):
    """Half the spacing of the output type at |v| (upper spacing of its binade)."""
    return np.ldexp(1.0, np.frexp(np.maximum(np.abs(v), 1e-300))[1] - mant - 1)


def check_rounding_flips(got, exact, name, absdot, n_terms, max_frac=0.001):
    """Elementwise bound.  Every output is one rounding (to bf16, or to fp32
    in the fp32 gradient mode) of a sum that the GPU accumulates in fp32 and
    the oracle forms exactly (float64 `exact`, from the same operands).  The
    GPU's fp32 sum s is within e = depth * 2^-24 * sum_k |terms| (absdot) of
    the exact sum, with depth = n/16 + 64 an upper bound on the rounded fp32
    additions any one term goes through in these kernels (every
    matrix-core instruction sums at least 16 products before touching its
    accumulator, at most 64 inside it; the partial-sum reductions are
    shorter than the accumulation chains).  So every element must lie within
    e plus half an output ulp of the exact sum.  For bf16 outputs, elements
    that are not the correctly rounded exact sum (those within e of a
    rounding midpoint) may be at most max_frac of the total (two always
    allowed)."""
    if got is None or got.size == 0:
        return
    got = np.asarray(got)
    exact = np.asarray(exact, dtype=np.float64)
    assert got.shape == exact.shape, (name, got.shape, exact.shape)
    bf = got.dtype == np.uint16
    mant = 8 if bf else 24
    ref = OQ.f64_to_bf16_bits(exact) if bf else OQ.f64_to_f32(exact)
    g = _values(got)
    eps = (n_terms / 16.0 + 64.0) * 2.0 ** -24 * np.asarray(absdot)
    far = np.abs(g - exact) > eps + _half_ulp(g, mant) + _half_ulp(exact, mant) * 1e-6
    if far.any():
        idx = np.argwhere(far)[:5]
        raise AssertionError((name, "beyond accumulation error of the exact sum", int(far.sum()),
                              [tuple(int(v) for v in i) for i in idx], g[far][:5],
                              exact[far][:5], eps[far][:5]))
    # (fp32 outputs: the accumulation error is of the order of the output's
    # own rounding step, so most elements may legitimately round the other
    # way; the bound above is the check there)
    if bf:
        n = int((_ordinal(got) != _ordinal(ref)).sum())
        assert n <= max(2, max_frac * got.size), (name, "not correctly rounded", n, got.size)


def _exact_terms(c, rows, wc, ws, fkw, bkw, precision, U, P):
    """Exact float64 sums (and sum_k |terms|) of Y and dX on the given rows,
    from the dequantized backbone operands and the GPU's own U and P (the
    low-rank up-projections read the bf16 values the first kernels wrote)."""
    X, dY = np.asarray(c.X)[rows], np.asarray(c.dY)[rows]
    if "A16" in precision:
        Xh = OQ.bf16_bits_to_f64(X)
    else:
        Xh = OQ.dequantize_row32(*OQ.quantize_row32(X))
    if "G16" in precision:
        Gh = OQ.bf16_bits_to_f64(dY)
    else:
        Gh = OQ.dequantize_row32(*OQ.quantize_row32(dY))
    Wf = OL.weight_fwd(wc, ws, fkw.get("w_block", "tile32"))
    Wd = OL.weight_dgrad(wc, ws, bkw.get("w_block", "tile32"), bkw.get("wt"))
    D = OL.stack_down(c.L1, c.A)
    V = OL.stack_up(c.L2, c.B)
    Uv = OQ.bf16_bits_to_f64(U) if c.R else np.zeros((len(rows), 0))
    Pv = OQ.bf16_bits_to_f64(P) if c.R else np.zeros((len(rows), 0))
    ey = Xh @ Wf.T + Uv @ V
    edx = Gh @ Wd + Pv @ D.T
    ty = np.abs(Xh) @ np.abs(Wf).T + np.abs(Uv) @ np.abs(V)
    tdx = np.abs(Gh) @ np.abs(Wd) + np.abs(Pv) @ np.abs(D).T
    return ey, ty, edx, tdx


def _exact_grads(c, U, P):
    """Exact dA, dB and their sum_k |terms| from the GPU's U and P."""
    X, G = OQ.bf16_bits_to_f64(c.X), OQ.bf16_bits_to_f64(c.dY)
    Pl = OQ.bf16_bits_to_f64(P)[:, c.r_s:]
    Ul = OQ.bf16_bits_to_f64(U)[:, c.r_s:]
    return X.T @ Pl, np.abs(X).T @ np.abs(Pl), Ul.T @ G, np.abs(Ul).T @ np.abs(G)


def _check_down_proj(c, got):
    """U and P against their exact sums X D and dY V^T."""
    D = OL.stack_down(c.L1, c.A)
    V = OL.stack_up(c.L2, c.B)
    X, G = OQ.bf16_bits_to_f64(c.X), OQ.bf16_bits_to_f64(c.dY)
    check_rounding_flips(got["U"], X @ D, "U", np.abs(X) @ np.abs(D), c.K)
    check_rounding_flips(got["P"], G @ V.T, "P", np.abs(G) @ np.abs(V).T, c.N)


def _check_outputs_elementwise(c, got, rows, wc, ws, fkw, bkw, precision, grads=True):
    """Y and dX on `rows` and (grads) dA, dB in full, elementwise against the
    oracle fed the GPU's U and P."""
    U = got["U"][rows] if c.R else None
    P = got["P"][rows] if c.R else None
    ey, ty, edx, tdx = _exact_terms(c, rows, wc, ws, fkw, bkw, precision, U, P)
    check_rounding_flips(got["Y"][rows], ey, "Y", ty, c.K + c.R)
    check_rounding_flips(got["dX"][rows], edx, "dX", tdx, c.N + c.R)
    if grads and c.r_l:
        ea, ta, eb, tb = _exact_grads(c, got["U"], got["P"])
        check_rounding_flips(got["dA"], ea, "dA", ta, c.M)
        check_rounding_flips(got["dB"], eb, "dB", tb, c.M)


def check_weight_codes(c, got):
    """Qtile(W): the method stores it once and the backward reads the same
    bytes transposed.  With the stored transposed copy (tile32_t) the copy
    must be Qtile(W^T): the same numbers, since a 32x32 tile has one scale.
    With group-wise weights: Qrow32(W) and the separate Qrow32(W^T).
    Returns the oracle's (codes, scales) and the keyword arguments of its
    weight."""
    blk = got.get("w_block", "tile32")
    row = blk == "row32"
    quant = OQ.quantize_row32 if row else OQ.quantize_tile32
    wc, ws = quant(c.W_res)
    np.testing.assert_array_equal(got["w_codes"], wc)
    np.testing.assert_array_equal(got["w_scales"], ws)
    if blk == "tile32":
        assert got["wt_codes"] is None and got["wt_scales"] is None
    else:
        wtc, wts = quant(np.ascontiguousarray(c.W_res.T))
        np.testing.assert_array_equal(got["wt_codes"], wtc)
        np.testing.assert_array_equal(got["wt_scales"], wts)
    kw = dict(w_block="row32") if row else {}
    return wc, ws, kw, (dict(w_block="row32", wt=(wtc, wts)) if row else {})


def _codes_equal(got, ref, name):
    """Codes and scales bit for bit; a 16-bit side has none on either side."""
    assert (got is None) == (ref is None), name
    if ref is not None:
        np.testing.assert_array_equal(got, ref, err_msg=name)


def check_full(case, got, grad_f32=False, precision="W4A4G4"):
    """Full-size oracle comparison for cases the oracle finishes in seconds."""
    c = case
    wc, ws, fkw, bkw = check_weight_codes(c, got)
    f = OL.linear_fwd(c.X, wc, ws, c.L1, c.L2, c.A, c.B, precision=precision, **fkw)
    b = OL.linear_bwd(c.dY, c.X, f["U"], wc, ws, c.L1, c.L2, c.A, c.B,
                      grad_dtype="f32" if grad_f32 else "bf16", precision=precision, **bkw)
    for k in ("xq_codes", "xq_scales"):
        _codes_equal(got[k], f[k], k)
    for k in ("gq_codes", "gq_scales"):
        _codes_equal(got[k], b[k], k)
    res = {}
    if c.R:
        res["U_bits"] = bit_agreement(got["U"], f["U"])
        res["P_bits"] = bit_agreement(got["P"], b["P"])
        res["U"] = OL.rel_frobenius(got["U"], f["U"])
        res["P"] = OL.rel_frobenius(got["P"], b["P"])
    res["Y"] = OL.rel_frobenius(got["Y"], f["Y"])
    res["dX"] = OL.rel_frobenius(got["dX"], b["dX"])
    if c.r_l:
        res["dA"] = OL.rel_frobenius(got["dA"], b["dA"])
        res["dB"] = OL.rel_frobenius(got["dB"], b["dB"])
    say(c.name, {k: (round(v, 7) if isinstance(v, float) else v) for k, v in res.items()})
    for k in ("Y", "dX", "dA", "dB"):
        if k in res:
            assert res[k] <= REL_TOL, (k, res[k])
    for k in ("U", "P"):
        if k in res:
            assert res[k] <= REL_TOL, (k, res[k])
    if c.R:
        _check_down_proj(c, got)
    # elementwise: each output a correct rounding but for accumulation order
    _check_outputs_elementwise(c, got, np.arange(c.M), wc, ws, fkw, bkw, precision)
    return res


def check_sampled(case, got, rows, precision="W4A4G4"):
    """Large cases: outputs of sampled rows, and the adapter gradients in full."""
    c = case
    wc, ws, fkw, bkw = check_weight_codes(c, got)
    if "A16" in precision:
        assert got["xq_codes"] is None
    else:
        xc, xs = OQ.quantize_row32(c.X[rows])
        np.testing.assert_array_equal(got["xq_codes"][rows], xc)
        np.testing.assert_array_equal(got["xq_scales"][rows], xs)
    if "G16" in precision:
        assert got["gq_codes"] is None
    else:
        gc, gs = OQ.quantize_row32(c.dY[rows])
        np.testing.assert_array_equal(got["gq_codes"][rows], gc)
        np.testing.assert_array_equal(got["gq_scales"][rows], gs)
    Y, U = OL.linear_fwd_rows(rows, c.X, wc, ws, c.L1, c.L2, c.A, c.B, precision=precision, **fkw)
    dX, P = OL.linear_bwd_rows(rows, c.dY, wc, ws, c.L1, c.L2, c.A, c.B, precision=precision,
                               **bkw)
    res = {"Y": OL.rel_frobenius(got["Y"][rows], OQ.f64_to_bf16_bits(Y)),
           "dX": OL.rel_frobenius(got["dX"][rows], OQ.f64_to_bf16_bits(dX))}
    if c.R:
        # the rank-R down-projections are cheap: check them over all tokens
        D = OL.stack_down(c.L1, c.A)
        V = OL.stack_up(c.L2, c.B)
        Uf = OL.down_proj(c.X, D)
        Pf = OL.down_proj(c.dY, V.T)
        np.testing.assert_array_equal(Uf[rows], U)
        np.testing.assert_array_equal(Pf[rows], P)
        res["U_bits"] = bit_agreement(got["U"], Uf)
        res["P_bits"] = bit_agreement(got["P"], Pf)
        res["U"] = OL.rel_frobenius(got["U"], Uf)
        res["P"] = OL.rel_frobenius(got["P"], Pf)
    if c.r_l:
        dA = OQ.bf16_bits_to_f64(c.X).T @ OQ.bf16_bits_to_f64(Pf)[:, c.r_s:]
        dB = OQ.bf16_bits_to_f64(Uf)[:, c.r_s:].T @ OQ.bf16_bits_to_f64(c.dY)
        res["dA"] = OL.rel_frobenius(got["dA"], OQ.f64_to_bf16_bits(dA))
        res["dB"] = OL.rel_frobenius(got["dB"], OQ.f64_to_bf16_bits(dB))
    say(c.name, {k: round(v, 7) for k, v in res.items()})
    for k in ("Y", "dX", "dA", "dB", "U", "P"):
        if k in res:
            assert res[k] <= REL_TOL, (k, res[k])
    if c.R:
        _check_down_proj(c, got)
    # elementwise on the sampled rows, and on the whole adapter gradients
    _check_outputs_elementwise(c, got, rows, wc, ws, fkw, bkw, precision)
    return res
