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


def check_rounding_flips(got, ref, name, absdot, n_terms):
    """U and P are bf16 roundings of long fp32 (GPU) vs fp64 (oracle) sums.
    They may differ only where the exact sum lies within fp32 accumulation
    error of a bf16 rounding boundary: in at most 0.1% of the elements (two
    are always allowed), and each by at most one bf16 ulp plus the
    recursive-summation bound n * 2^-24 * sum_k |x_k d_k| (absdot)."""
    if got is None or got.size == 0:
        return
    diff = got != ref
    n = int(diff.sum())
    assert n <= max(2, 0.001 * got.size), (name, n, got.size)
    g = OQ.bf16_bits_to_f64(got[diff])
    r = OQ.bf16_bits_to_f64(ref[diff])
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(r), 1e-38))[1] - 8)
    bound = ulp + n_terms * 2.0 ** -24 * absdot[diff]
    assert np.all(np.abs(g - r) <= bound), (name, np.abs(g - r).max())


def _absdots(c):
    D = np.abs(OL.stack_down(c.L1, c.A))
    V = np.abs(OL.stack_up(c.L2, c.B))
    return (np.abs(OQ.bf16_bits_to_f64(c.X)) @ D, np.abs(OQ.bf16_bits_to_f64(c.dY)) @ V.T)


def check_weight_codes(c, got):
    """Qtile(W) and the transposed copy the backward reads, which must be
    Qtile(W^T): the same numbers, since a 32x32 tile has one scale.  With
    group-wise weights: Qrow32(W) and the separate Qrow32(W^T).  Returns
    the oracle's (codes, scales) and the keyword arguments of its weight."""
    row = got.get("w_block", "tile32") == "row32"
    quant = OQ.quantize_row32 if row else OQ.quantize_tile32
    wc, ws = quant(c.W_res)
    np.testing.assert_array_equal(got["w_codes"], wc)
    np.testing.assert_array_equal(got["w_scales"], ws)
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
    if c.R:
        ua, pa = _absdots(c)
        check_rounding_flips(got["U"], f["U"], "U", ua, c.K)
        check_rounding_flips(got["P"], b["P"], "P", pa, c.N)
    for k in ("U", "P"):
        if k in res:
            assert res[k] <= REL_TOL, (k, res[k])
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
        ua, pa = _absdots(c)
        check_rounding_flips(got["U"], Uf, "U", ua, c.K)
        check_rounding_flips(got["P"], Pf, "P", pa, c.N)
    return res
