"""GPU parity of the MLP glue around the GELU (two linears with the
activation between them), through the C ABI.

FourTune, "3.3 Kernel Fusion for Efficiency / MLP Fusion": GeLU sits on the
wide intermediate between the two linears of an MLP block.  The first
linear's output h is kept; the second linear takes gelu(h) as its input
(applied as its quantizer reads h), and in the backward the first linear's
incoming gradient is dX2 * gelu'(h) (applied as its quantizer and its dB
read dX2 and h).

The GPU evaluates GELU in fp32 and the oracle in float64; both round to
bf16, so a value lying within fp32 error of a rounding boundary may round
the other way.  The activation entry points (the same device functions the
fused kernels call) are therefore checked against the oracle's GELU to
within one bf16 ulp, and each linear is then checked against the oracle fed
the GPU's bf16 activation values, so that the codes compare bit for bit.
"""
import copy

import numpy as np
import pytest
import torch

from bit_quantized_amd import ops, synth
from bit_quantized_amd.layer import QuantizedLinear, bits_of, mlp_backward, mlp_forward
from oracle import linear as OL
from oracle import mxfp4 as OQ

from _gpu import (DEV, REL_TOL, _check_down_proj, _check_outputs_elementwise,
                  check_rounding_flips, require_gpu, say, up)

pytestmark = pytest.mark.gpu
G = ops.FT_ACT_GELU_TANH


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _ord(bits):
    """bf16 bit patterns as integers ordered like their values (+0 == -0)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def check_ulps(got, ref, name, min_exact=0.999):
    """got within one bf16 ulp of ref everywhere (values below 2^-126 in
    magnitude on both sides count as equal: fp32's flush region), and
    bit-identical in at least `min_exact` of the elements."""
    d = np.abs(_ord(got) - _ord(ref))
    tiny = (np.abs(OQ.bf16_bits_to_f64(got)) < 2.0 ** -126) & (np.abs(OQ.bf16_bits_to_f64(ref)) < 2.0 ** -126)
    bad = (d > 1) & ~tiny
    assert not bad.any(), (name, int(bad.sum()), got[bad][:5], ref[bad][:5])
    exact = float(np.mean(d == 0))
    say(name, "bit-identical fraction", exact)
    assert exact >= min_exact, (name, exact)


def _gelu_gpu(h_bits):
    h = up(h_bits)
    out = torch.empty_like(h)
    ops.fourtune_act_fwd(G, h, h.numel(), out)
    torch.cuda.synchronize()
    return bits_of(out)


def _gelu_grad_gpu(h_bits, g_bits):
    h, g = up(h_bits), up(g_bits)
    out = torch.empty_like(h)
    ops.fourtune_act_bwd(G, h, g, h.numel(), out)
    torch.cuda.synchronize()
    return bits_of(out)


def _finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7F80) != 0x7F80]          # drop Inf and NaN


def test_gelu_every_bf16_value():
    h = _finite_bf16()
    say("case gelu over", h.size, "bf16 values")
    check_ulps(_gelu_gpu(h), OL.gelu_tanh(h), "gelu")


@pytest.mark.parametrize("g", [1.0, -0.3711, 1.5e-3, -2.75e4])
def test_gelu_grad_every_bf16_value(g):
    h = _finite_bf16()
    gb = synth.to_bf16_bits(np.full(h.size, g, dtype=np.float32))
    say("case gelu' over", h.size, "bf16 values, g =", g)
    check_ulps(_gelu_grad_gpu(h, gb), OL.gelu_tanh_grad(h, gb), f"gelu_grad g={g}")


def test_gelu_odd_length_tail():
    rng = np.random.default_rng(3)
    h = synth.to_bf16_bits(rng.standard_normal(1003).astype(np.float32) * 3)
    # the entry points take any n; the last n % 8 values go through the tail path
    hb = up(np.concatenate([h, np.zeros(5, np.uint16)]))
    out = torch.zeros_like(hb)
    ops.fourtune_act_fwd(G, hb, 1003, out)
    torch.cuda.synchronize()
    got = bits_of(out)
    check_ulps(got[:1003], OL.gelu_tanh(h), "gelu tail")
    assert np.all(got[1003:] == 0)


# ------------------------------------------------------------------ the MLP pair
class MlpPair:
    """FC1 (K -> F, act_out = GELU) and FC2 (F -> K, act_in = GELU) on the GPU."""

    def __init__(self, M, K, F, rs, rl, seed, precision="W4A4G4"):
        self.c1 = synth.flux_linear_case(f"fc1_{M}x{K}x{F}", M, K, F, rs, rl, seed)
        self.c2 = synth.flux_linear_case(f"fc2_{M}x{F}x{K}", M, F, K, rs, rl, seed + 1)
        opt = lambda a: up(a) if a.size else None
        mk = lambda c, **kw: QuantizedLinear.from_factors(
            up(c.W_res), opt(c.L1), opt(c.L2), opt(c.A), opt(c.B), **kw)
        self.fc1 = mk(self.c1, act_out=G, precision=precision)
        self.fc2 = mk(self.c2, act_in=G, precision=precision)

    def run(self):
        c1, c2 = self.c1, self.c2
        X1, dY2 = up(c1.X), up(c2.dY)
        h, U1, xc1, xs1 = self.fc1.forward(X1, want_codes=True)
        Y2, U2, xc2, xs2 = self.fc2.forward(h, want_codes=True)
        dX2, dA2, dB2, P2, gc2, gs2 = self.fc2.backward(dY2, h, U2, want_codes=True)
        dX1, dA1, dB1, P1, gc1, gs1 = self.fc1.backward(dX2, X1, U1, want_codes=True, H=h)
        torch.cuda.synchronize()
        u8 = lambda t: None if t is None else t.cpu().numpy()
        R = lambda t, c: bits_of(t)[:, :c.R] if c.R else None
        T = lambda t: None if t is None else np.ascontiguousarray(bits_of(t).T)
        Bb = lambda t: None if t is None else bits_of(t)
        return dict(h=bits_of(h), U1=R(U1, c1), xc1=u8(xc1), xs1=u8(xs1),
                    Y2=bits_of(Y2), U2=R(U2, c2), xc2=u8(xc2), xs2=u8(xs2),
                    dX2=bits_of(dX2), dA2=T(dA2), dB2=Bb(dB2),
                    P2=R(P2, c2), gc2=u8(gc2), gs2=u8(gs2),
                    dX1=bits_of(dX1), dA1=T(dA1), dB1=Bb(dB1),
                    P1=R(P1, c1), gc1=u8(gc1), gs1=u8(gs1))


def _check_layer_full(tag, c, X, dY, got_fwd, got_bwd, Y_name, precision="W4A4G4"):
    """One linear against the oracle in full, given the operands the GPU saw.
    got_fwd = (Y, U, xc, xs); got_bwd = (dX, dA, dB, P, gc, gs)."""
    wc, ws = OQ.quantize_tile32(c.W_res)
    f = OL.linear_fwd(X, wc, ws, c.L1, c.L2, c.A, c.B, precision=precision)
    b = OL.linear_bwd(dY, X, f["U"], wc, ws, c.L1, c.L2, c.A, c.B, precision=precision)
    Y, U, xc, xs = got_fwd
    dX, dA, dB, P, gc, gs = got_bwd
    for got_c, ref_c, name in ((xc, f["xq_codes"], "xq codes"), (xs, f["xq_scales"], "xq scales"),
                               (gc, b["gq_codes"], "gq codes"), (gs, b["gq_scales"], "gq scales")):
        assert (got_c is None) == (ref_c is None), tag + " " + name
        if ref_c is not None:
            np.testing.assert_array_equal(got_c, ref_c, err_msg=tag + " " + name)
    res = {Y_name: OL.rel_frobenius(Y, f["Y"]), "dX": OL.rel_frobenius(dX, b["dX"])}
    if c.r_l:
        res["dA"] = OL.rel_frobenius(dA, b["dA"])
        res["dB"] = OL.rel_frobenius(dB, b["dB"])
    if c.R:
        res["U"] = OL.rel_frobenius(U, f["U"])
        res["P"] = OL.rel_frobenius(P, b["P"])
    say(tag, {k: round(v, 8) for k, v in res.items()})
    for k, v in res.items():
        assert v <= REL_TOL, (tag, k, v)
    # elementwise, against the oracle fed the operands the GPU saw
    cc = copy.copy(c)
    cc.X, cc.dY = X, dY
    got = {"Y": Y, "dX": dX, "dA": dA, "dB": dB, "U": U, "P": P}
    if c.R:
        _check_down_proj(cc, got)
    wkw = {}
    _check_outputs_elementwise(cc, got, np.arange(c.M), wc, ws, wkw, wkw, precision)
    return f


@pytest.mark.parametrize("shape", [
    (300, 288, 544, 16, 8),     # ragged tokens, several tiles, F not a multiple of 128
    (130, 256, 1024, 32, 32),   # R = 64
    (64, 160, 320, 0, 8),       # adapter only
    (40, 96, 192, 0, 0),        # no low-rank branches (plain quantizer with the activation)
])
def test_mlp_pair_chain_full(shape, precision="W4A4G4"):
    M, K, F, rs, rl = shape
    say("case mlp pair", shape, precision)
    mp = MlpPair(M, K, F, rs, rl, seed=M + F, precision=precision)
    got = mp.run()
    c1, c2 = mp.c1, mp.c2
    a_gpu = _gelu_gpu(got["h"])
    check_ulps(a_gpu, OL.gelu_tanh(got["h"]), "a = gelu(h)", min_exact=0.99)
    dh_gpu = _gelu_grad_gpu(got["h"], got["dX2"])
    check_ulps(dh_gpu, OL.gelu_tanh_grad(got["h"], got["dX2"]), "dh", min_exact=0.99)
    # FC2 consumes gelu(h): the oracle is fed the GPU's bf16 activation
    _check_layer_full("fc2", c2, a_gpu, c2.dY,
                      (got["Y2"], got["U2"], got["xc2"], got["xs2"]),
                      (got["dX2"], got["dA2"], got["dB2"], got["P2"], got["gc2"], got["gs2"]), "Y2",
                      precision)
    # FC1's incoming gradient is dX2 * gelu'(h)
    _check_layer_full("fc1", c1, c1.X, dh_gpu,
                      (got["h"], got["U1"], got["xc1"], got["xs1"]),
                      (got["dX1"], got["dA1"], got["dB1"], got["P1"], got["gc1"], got["gs1"]), "h",
                      precision)


@pytest.mark.parametrize("shape", [(300, 288, 544, 16, 8), (40, 96, 192, 0, 0)])
def test_mlp_pair_chain_w4a16g16_full(shape):
    """The 16-bit setting around the GELU: FC2's bf16 input gelu(h) and FC1's
    bf16 incoming gradient dX2 * gelu'(h) are made by the activation kernels
    before the 16-bit products."""
    test_mlp_pair_chain_full(shape, precision="W4A16G16")


def test_mlp_pair_chain_full_size_sampled():
    """FLUX MLP at full size: 4608 tokens, 3072 -> 12288 -> GELU -> 3072, ranks 32/32.
    Row outputs on sampled rows; codes of the sampled rows; adapter gradients and
    the down-projections over all rows."""
    M, K, F = 4608, 3072, 12288
    say("case mlp pair full size")
    mp = MlpPair(M, K, F, 32, 32, seed=2)
    got = mp.run()
    c1, c2 = mp.c1, mp.c2
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([rng.choice(M, 40, replace=False), [0, M - 1]]))
    a_gpu = _gelu_gpu(got["h"])
    check_ulps(a_gpu[rows], OL.gelu_tanh(got["h"][rows]), "a rows")
    dh_gpu = _gelu_grad_gpu(got["h"], got["dX2"])
    check_ulps(dh_gpu[rows], OL.gelu_tanh_grad(got["h"][rows], got["dX2"][rows]), "dh rows")
    for tag, c, X, dY, Yk, Uk, xk, gk, Pk, dXk, dAk, dBk in (
            ("fc2", c2, a_gpu, c2.dY, "Y2", "U2", "2", "2", "P2", "dX2", "dA2", "dB2"),
            ("fc1", c1, c1.X, dh_gpu, "h", "U1", "1", "1", "P1", "dX1", "dA1", "dB1")):
        wc, ws = OQ.quantize_tile32(c.W_res)
        xc, xs = OQ.quantize_row32(X[rows])
        np.testing.assert_array_equal(got["xc" + xk][rows], xc, err_msg=tag)
        np.testing.assert_array_equal(got["xs" + xk][rows], xs, err_msg=tag)
        gc, gs = OQ.quantize_row32(dY[rows])
        np.testing.assert_array_equal(got["gc" + gk][rows], gc, err_msg=tag)
        np.testing.assert_array_equal(got["gs" + gk][rows], gs, err_msg=tag)
        Y, U = OL.linear_fwd_rows(rows, X, wc, ws, c.L1, c.L2, c.A, c.B)
        dX, P = OL.linear_bwd_rows(rows, dY, wc, ws, c.L1, c.L2, c.A, c.B)
        D = OL.stack_down(c.L1, c.A)
        V = OL.stack_up(c.L2, c.B)
        Uf = OL.down_proj(X, D)
        Pf = OL.down_proj(dY, V.T)
        dA = OQ.bf16_bits_to_f64(X).T @ OQ.bf16_bits_to_f64(Pf)[:, c.r_s:]
        dB = OQ.bf16_bits_to_f64(Uf)[:, c.r_s:].T @ OQ.bf16_bits_to_f64(dY)
        res = {"Y": OL.rel_frobenius(got[Yk][rows], OQ.f64_to_bf16_bits(Y)),
               "dX": OL.rel_frobenius(got[dXk][rows], OQ.f64_to_bf16_bits(dX)),
               "U": OL.rel_frobenius(got[Uk], Uf), "P": OL.rel_frobenius(got[Pk], Pf),
               "dA": OL.rel_frobenius(got[dAk], OQ.f64_to_bf16_bits(dA)),
               "dB": OL.rel_frobenius(got[dBk], OQ.f64_to_bf16_bits(dB))}
        say(tag, {k: round(v, 8) for k, v in res.items()})
        for k, v in res.items():
            assert v <= REL_TOL, (tag, k, v)
        cc = copy.copy(c)
        cc.X, cc.dY = X, dY
        g = {"Y": got[Yk], "dX": got[dXk], "dA": got[dAk], "dB": got[dBk], "U": got[Uk],
             "P": got[Pk]}
        _check_down_proj(cc, g)
        _check_outputs_elementwise(cc, g, rows, wc, ws, {}, {}, "W4A4G4")


# ------------------------------------------------------------------ the fused MLP forward
# FourTune, "3.3 Kernel Fusion for Efficiency / MLP Fusion": FC1's GEMM
# epilogue applies the GeLU to the h it holds and writes FC2's quantized
# input and FC2's down-projection partials (fourtune_mlp_fwd).
def _fused_kernels():
    """Launch counts per kernel name since the last timing reset."""
    return {k: cnt for k, (tot, cnt) in ops.fourtune_timing_read().items() if cnt}


def _run_fused(mp, X1):
    """Both paths on the same input: the two forwards one after the other,
    then the fused call (its kernel names recorded, to show that the
    epilogue fusion ran)."""
    h_u, U1_u, _, _ = mp.fc1.forward(X1, want_codes=True)
    Y_u, U2_u, ac_u, as_u = mp.fc2.forward(h_u, want_codes=True)
    torch.cuda.synchronize()
    ops.fourtune_timing_reset()
    ops.fourtune_timing_enable(True)
    try:
        h, U1, Y, U2, ac, as_ = mlp_forward(mp.fc1, mp.fc2, X1, want_codes=True)
        torch.cuda.synchronize()
    finally:
        ops.fourtune_timing_enable(False)
    names = _fused_kernels()
    ops.fourtune_timing_reset()
    R = lambda t, c: bits_of(t)[:, :c.R] if c.R else None
    fused = dict(h=bits_of(h), U1=R(U1, mp.c1), Y=bits_of(Y), U2=R(U2, mp.c2),
                 ac=ac.cpu().numpy(), as_=as_.cpu().numpy())
    plain = dict(h=bits_of(h_u), U1=R(U1_u, mp.c1), Y=bits_of(Y_u), U2=R(U2_u, mp.c2),
                 ac=ac_u.cpu().numpy(), as_=as_u.cpu().numpy())
    return fused, plain, names


def _same_bits(a, b, name):
    if a is None:
        assert b is None, name
        return
    np.testing.assert_array_equal(a, b, err_msg=name)


@pytest.mark.parametrize("shape", [
    (300, 256, 544, 16, 8),     # ragged rows (2 row tiles), F = 544: last column tile of 32
    (520, 384, 1280, 32, 32),   # R2 = 64: four rank groups, two per wave
    (600, 128, 2304, 32, 16),   # R2 = 48: three rank groups (the second wave's second empty)
    (130, 256, 768, 0, 8),      # adapter only, R2 = 8: one rank group
    (272, 128, 288, 0, 0),      # no ranks: codes and scales only
    (1040, 128, 16384, 16, 16), # 5 x 64 = 320 tiles: workgroups that walk two tiles
])
def test_mlp_fused_forward_full(shape):
    M, K, F, rs, rl = shape
    say("case fused mlp forward", shape)
    mp = MlpPair(M, K, F, rs, rl, seed=3 * M + F)
    X1 = up(mp.c1.X)
    got, ref, names = _run_fused(mp, X1)
    say("kernels", names)
    # FC1's kernel 1, its fused GEMM, the partials' sum, FC2's GEMM: FC2's
    # quantize kernel does not run
    assert names.get("fwd_gemm_mlp") == 1 and names.get("fwd_gemm") == 1, names
    assert names.get("fwd_quant_down") == 1, names
    assert names.get("fwd_rank_reduce", 0) == (1 if mp.c2.R else 0), names
    # h and U1 come out of the same kernels as the unfused forward
    _same_bits(got["h"], ref["h"], "h")
    _same_bits(got["U1"], ref["U1"], "U1")
    # FC2's quantized input: the unfused quantizer's bits, and the oracle's
    # quantization of the GPU's bf16 gelu(h)
    _same_bits(got["ac"], ref["ac"], "aq codes")
    _same_bits(got["as_"], ref["as_"], "aq scales")
    a_gpu = _gelu_gpu(got["h"])
    xc, xs = OQ.quantize_row32(a_gpu)
    np.testing.assert_array_equal(got["ac"], xc, err_msg="aq codes vs oracle")
    np.testing.assert_array_equal(got["as_"], xs, err_msg="aq scales vs oracle")
    c2 = copy.copy(mp.c2)
    c2.X = a_gpu
    if c2.R:
        # U2 = bf16(gelu(h) D2): a correct rounding of the exact sum but for
        # the fp32 accumulation order
        D = OL.stack_down(c2.L1, c2.A)
        A = OQ.bf16_bits_to_f64(a_gpu)
        check_rounding_flips(got["U2"], A @ D, "U2", np.abs(A) @ np.abs(D), c2.K)
    # Y against the oracle fed the GPU's activation and U2: exact sums of
    # the dequantized operands plus U2 V2
    wc, ws = OQ.quantize_tile32(c2.W_res)
    Xh = OQ.dequantize_row32(xc, xs)
    Wf = OL.weight_fwd(wc, ws, "tile32")
    Uv = OQ.bf16_bits_to_f64(got["U2"]) if c2.R else np.zeros((M, 0))
    V = OL.stack_up(c2.L2, c2.B)
    ey = Xh @ Wf.T + Uv @ V
    ty = np.abs(Xh) @ np.abs(Wf).T + np.abs(Uv) @ np.abs(V)
    check_rounding_flips(got["Y"], ey, "Y", ty, c2.K + c2.R)
    res = {"Y": OL.rel_frobenius(got["Y"], OQ.f64_to_bf16_bits(ey))}
    say("rel", res)
    assert res["Y"] <= REL_TOL


def test_mlp_fused_forward_full_size():
    """FLUX MLP forward at full size (4608 tokens, 3072 -> 12288 -> GELU ->
    3072, ranks 32/32; 864 output tiles, 3-4 per workgroup): the fused call
    gives the unfused forwards' bits (FC2's quantizer sums 256-column splits
    at this size), and FC2's codes and U2 agree with the oracle on sampled rows."""
    M, K, F = 4608, 3072, 12288
    say("case fused mlp forward full size")
    mp = MlpPair(M, K, F, 32, 32, seed=2)
    got, ref, names = _run_fused(mp, up(mp.c1.X))
    assert names.get("fwd_gemm_mlp") == 1 and names.get("fwd_rank_reduce") == 1, names
    assert names.get("fwd_quant_down") == 1, names
    for k in ("h", "U1", "ac", "as_", "U2", "Y"):
        _same_bits(got[k], ref[k], k)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.choice(M, 24, replace=False), [0, M - 1]]))
    a_rows = _gelu_gpu(got["h"][rows])
    xc, xs = OQ.quantize_row32(a_rows)
    np.testing.assert_array_equal(got["ac"][rows], xc)
    np.testing.assert_array_equal(got["as_"][rows], xs)
    D = OL.stack_down(mp.c2.L1, mp.c2.A)
    A = OQ.bf16_bits_to_f64(a_rows)
    check_rounding_flips(got["U2"][rows], A @ D, "U2 rows", np.abs(A) @ np.abs(D), F)


# ------------------------------------------------------------------ the mirrored MLP backward
# FC2's input-gradient GEMM forms FC1's incoming gradient dY1 = dX2 gelu'(h)
# in its epilogue and quantizes and projects it for FC1 (fourtune_mlp_bwd).
def _run_bwd_both(mp, full_size=False):
    c1, c2 = mp.c1, mp.c2
    X1, dY2 = up(c1.X), up(c2.dY)
    h, U1, _, U2 = mlp_forward(mp.fc1, mp.fc2, X1)
    torch.cuda.synchronize()
    # unfused: the two backwards through dX2
    dX2, dA2u, dB2u, _ = mp.fc2.backward(dY2, h, U2)
    dX1u, dA1u, dB1u, _ = mp.fc1.backward(dX2, X1, U1, H=h)
    torch.cuda.synchronize()
    ops.fourtune_timing_reset()
    ops.fourtune_timing_enable(True)
    try:
        dX1, dA1, dB1, dA2, dB2 = mlp_backward(mp.fc1, mp.fc2, dY2, X1, h, U1, U2)
        torch.cuda.synchronize()
    finally:
        ops.fourtune_timing_enable(False)
    names = _fused_kernels()
    ops.fourtune_timing_reset()
    T = lambda t: None if t is None else np.ascontiguousarray(bits_of(t).T)
    Bb = lambda t: None if t is None else bits_of(t)
    got = dict(dX1=bits_of(dX1), dA1=T(dA1), dB1=Bb(dB1), dA2=T(dA2), dB2=Bb(dB2))
    ref = dict(dX1=bits_of(dX1u), dA1=T(dA1u), dB1=Bb(dB1u), dA2=T(dA2u), dB2=Bb(dB2u))
    return got, ref, names, bits_of(h), bits_of(dX2), bits_of(U1)


def _check_db1(mp, got, h_bits, dx2_bits, u1_bits):
    """dB1 = U1[:, r_s:]^T dY1 with dY1 = gelu'(h) dX2 as the GPU forms it:
    a correct rounding of the exact sum but for the fp32 accumulation order."""
    c1 = mp.c1
    if not c1.r_l:
        return
    dy1 = _gelu_grad_gpu(h_bits, dx2_bits)
    Ul = OQ.bf16_bits_to_f64(u1_bits[:, c1.r_s:c1.R])
    G = OQ.bf16_bits_to_f64(dy1)
    check_rounding_flips(got["dB1"], Ul.T @ G, "dB1", np.abs(Ul).T @ np.abs(G), c1.M)


@pytest.mark.parametrize("shape", [
    (300, 256, 544, 16, 8),     # ragged rows, F = 544: last column tile of 32
    (520, 384, 1280, 32, 32),   # R1 = 64: four rank groups
    (600, 128, 2304, 32, 16),   # R1 = 48: three rank groups
    (130, 256, 768, 0, 8),      # adapter only
    (272, 128, 288, 0, 0),      # no ranks: dY1's codes only
])
def test_mlp_mirrored_backward_full(shape):
    M, K, F, rs, rl = shape
    say("case mirrored mlp backward", shape)
    mp = MlpPair(M, K, F, rs, rl, seed=5 * M + F)
    got, ref, names, h, dx2, u1 = _run_bwd_both(mp)
    say("kernels", names)
    # FC2's quantizer, its mirrored dgrad, FC1's dgrad: FC1's quantizer does not run
    assert names.get("bwd_gemm_dgrad_mlp") == 1 and names.get("bwd_gemm_dgrad") == 1, names
    assert names.get("bwd_quant_down") == 1, names
    assert names.get("bwd_rank_reduce", 0) == (1 if mp.c1.R else 0), names
    # FC2's adapter gradients come out of the same kernels
    for k in ("dA2", "dB2"):
        _same_bits(got[k], ref[k], k)
    # dX1 and dA1 read P1, whose fp32 sums may round the other way where
    # the unfused quantizer takes 128-column splits: compared to the unfused
    # result within the accumulation bound of the exact sums
    res = {k: OL.rel_frobenius(got[k], ref[k]) for k in ("dX1", "dA1") if got[k] is not None}
    say("rel vs unfused", res)
    for k, v in res.items():
        assert v <= 1e-4, (k, v)
    _check_db1(mp, got, h, dx2, u1)


def test_mlp_mirrored_backward_full_size():
    """FLUX MLP backward at full size (4608 tokens, 3072 -> 12288 -> 3072,
    ranks 32/32): the mirrored backward gives the unfused backwards' dX1,
    dA1, dA2 and dB2 bit for bit (FC1's quantizer sums 256-column splits at
    this size) and dB1 within its accumulation bound."""
    M, K, F = 4608, 3072, 12288
    say("case mirrored mlp backward full size")
    mp = MlpPair(M, K, F, 32, 32, seed=2)
    got, ref, names, h, dx2, u1 = _run_bwd_both(mp)
    assert names.get("bwd_gemm_dgrad_mlp") == 1 and names.get("bwd_rank_reduce") == 1, names
    for k in ("dX1", "dA1", "dA2", "dB2"):
        _same_bits(got[k], ref[k], k)
    _check_db1(mp, got, h, dx2, u1)
