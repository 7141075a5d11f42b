"""Layer-level ablations on synthetic weights, with the oracle (CPU).

The layer analog of two comparisons in FourTune (arXiv 2607.05711):
* the stabilizer (section 3.1, and the gradient-norm curves of Fig. 8):
  the top singular directions of the weight stay in bf16 as L1 L2, so only
  the residual is quantized; on a weight whose few outlier columns set the
  scale of every 32x32 tile they touch, the forward and input-gradient
  errors drop several-fold;
* the weight block shape (Table 5, group-wise vs square blocks): 1x32 blocks
  along K never have a larger amax than the 32x32 tile that holds them, so
  the weight quantization error is lower, most of all with outlier rows.
The errors are measured against the unquantized layer X W^T (and dY W)."""
import numpy as np

from bit_quantized_amd import synth
from oracle import linear as OL
from oracle import mxfp4 as q


def _exact(case):
    W = q.bf16_bits_to_f64(case.meta["W"])
    return q.bf16_bits_to_f64(case.X) @ W.T, q.bf16_bits_to_f64(case.dY) @ W


def _layer_errors(case):
    Y_ref, dX_ref = _exact(case)
    wc, ws = q.quantize_tile32(case.W_res)
    f = OL.linear_fwd(case.X, wc, ws, case.L1, case.L2, case.A, case.B)
    b = OL.linear_bwd(case.dY, case.X, f["U"], wc, ws, case.L1, case.L2, case.A, case.B)
    return (OL.rel_frobenius(OL.out_to_f64(f["Y"]), Y_ref),
            OL.rel_frobenius(OL.out_to_f64(b["dX"]), dX_ref))


def test_stabilizer_ablation():
    with_stab, without = synth.outlier_weight_cases()
    ey1, ed1 = _layer_errors(with_stab)
    ey0, ed0 = _layer_errors(without)
    print(f"Y error {ey0:.3f} -> {ey1:.3f}; dX error {ed0:.3f} -> {ed1:.3f}")
    assert ey1 < ey0 / 3 and ed1 < ed0 / 3


def _weight_errors(w_bits):
    W = q.bf16_bits_to_f64(w_bits)
    ct, st = q.quantize_tile32(w_bits)
    cr, sr = q.quantize_row32(w_bits)
    n = np.linalg.norm(W)
    return (np.linalg.norm(q.dequantize_tile32(ct, st) - W) / n,
            np.linalg.norm(q.dequantize_row32(cr, sr) - W) / n)


def test_weight_block_ablation():
    rng = np.random.Generator(np.random.PCG64(7))
    gauss = synth.to_bf16_bits(0.02 * rng.standard_normal((256, 256)))
    rows = 0.02 * rng.standard_normal((256, 256))
    rows[rng.choice(256, 4, replace=False)] *= 20.0
    t_g, r_g = _weight_errors(gauss)
    t_r, r_r = _weight_errors(synth.to_bf16_bits(rows))
    print(f"gaussian: tile32 {t_g:.4f} row32 {r_g:.4f}; outlier rows: tile32 {t_r:.4f} row32 {r_r:.4f}")
    assert r_g < t_g
    assert r_r < t_r / 1.5
    # per block, a 1x32 row block's scale never exceeds its tile's
    ct, st = q.quantize_tile32(gauss)
    cr, sr = q.quantize_row32(gauss)
    tile_of_block = np.repeat(st, 32, axis=0)                             # [N, K/32]
    assert np.all(sr <= tile_of_block)
