"""Checks of the seeded input generators (CPU only)."""
import numpy as np

from bit_quantized_amd import synth


def _f(b):
    return synth.bf16_bits_to_f32(b).astype(np.float64)


def test_tiny_case_shapes_and_spectral_split():
    c = synth.tiny_case(0)
    assert (c.M, c.K, c.N, c.r_s, c.r_l) == (128, 256, 256, 16, 8)
    assert c.X.shape == (128, 256) and c.W_res.shape == (256, 256)
    assert c.L1.shape == (256, 16) and c.L2.shape == (16, 256)
    assert c.A.shape == (256, 8) and c.B.shape == (8, 256) and c.dY.shape == (128, 256)
    # The residual no longer holds the top singular directions: its spectral
    # norm is close to the noise level, far below the planted 5.0.
    s = np.linalg.svd(_f(c.W_res), compute_uv=False)
    assert s[0] < 1.0
    # Two outlier channels x40.
    col_std = _f(c.X).std(axis=0)
    assert np.sum(col_std > 10) == 2


def test_seeded_and_reproducible():
    a = synth.tiny_case(0)
    b = synth.tiny_case(0)
    for k in ("X", "W_res", "L1", "L2", "A", "B", "dY"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    c = synth.tiny_case(1)
    assert not np.array_equal(a.X, c.X)


def test_flux_case_small_shape_properties():
    c = synth.flux_linear_case("t", 64, 320, 96, 8, 4, seed=1)
    X = _f(c.X)
    assert np.sum(X.std(axis=0) > 10) == 3          # round(1% of 320) channels x50
    g = synth.flux_linear_case("g", 64, 320, 96, 8, 4, seed=1, x_kind="gated")
    assert _f(g.X).min() > -0.5
    L1 = _f(c.L1)
    n = np.linalg.norm(L1, axis=0) ** 2
    np.testing.assert_allclose(n, 8 * 0.8 ** np.arange(8), rtol=2e-2)


def test_stress_activation_has_zero_tiles_small():
    T = synth.stress_activation(4, rows=256, cols=512, zero_tile_frac=0.05)
    Tf = _f(T).reshape(8, 32, 16, 32)
    zero_tiles = np.all(Tf == 0, axis=(1, 3))
    assert zero_tiles.sum() == round(0.05 * 128)


def test_dit_block_shapes():
    shapes = synth.dit_block_linears()
    assert len(shapes) == 10
    assert ("img_qkv", 8192, 3072, 9216) in shapes and ("txt_mod", 2, 3072, 18432) in shapes
