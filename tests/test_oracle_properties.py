"""Property tests of the oracle's MXFP4 block quantizer (CPU, hypothesis).

Blocks of 32 bf16 values are drawn with an anchor element that fixes the
block exponent E (amax in [4, 8) * 2^E, so the OCP MX scale is 2^E) and the
other elements drawn from: exact ties between neighbouring E2M1 values
(0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 times 2^E), signed zeros, values far
below the block's smallest step, values beyond 6 * 2^E (saturation), and
random values.  Each element's code is checked against a brute-force
nearest search over the signed E2M1 grid times the block scale, ties to the
even code, saturating at +-6, sign kept ("2.3 Model Quantization": Round(W/s)
with the block scale; the MX element rounding)."""
import numpy as np
from hypothesis import given, settings, strategies as st

from bit_quantized_amd import synth
from oracle import mxfp4 as q

GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)
TIES = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


@st.composite
def blocks(draw):
    E = draw(st.integers(min_value=-118, max_value=118))
    anchor = draw(st.sampled_from((4.0, 5.0, 6.0, 7.0, 7.5)))
    vals = [anchor * 2.0 ** E * draw(st.sampled_from((1.0, -1.0)))]
    for _ in range(31):
        kind = draw(st.sampled_from(("tie", "tie", "zero", "negzero", "tiny", "sat", "rand")))
        sign = draw(st.sampled_from((1.0, -1.0)))
        if kind == "tie":
            v = sign * draw(st.sampled_from(TIES)) * 2.0 ** E
        elif kind == "zero":
            v = 0.0
        elif kind == "negzero":
            v = -0.0
        elif kind == "tiny":
            v = sign * draw(st.floats(min_value=0.0, max_value=0.2)) * 2.0 ** E
        elif kind == "sat":
            v = sign * draw(st.floats(min_value=6.0, max_value=7.9)) * 2.0 ** E
        else:
            v = sign * draw(st.floats(min_value=0.0, max_value=6.0)) * 2.0 ** E
        vals.append(v)
    perm = draw(st.permutations(range(32)))
    return np.array([vals[i] for i in perm], dtype=np.float64)


def _nearest_even(x, scale):
    """Brute force: the E2M1 code whose value times scale is nearest to x;
    ties to the even code; beyond the grid, the largest magnitude."""
    mags = [g * scale for g in GRID]
    a = abs(x)
    best = min(range(8), key=lambda c: (abs(a - mags[c]), c & 1))
    neg = np.signbit(x)
    return best | (8 if neg else 0)


@settings(max_examples=300, deadline=None)
@given(blocks())
def test_row32_block_is_nearest_even_under_block_scale(vals):
    bits = synth.to_bf16_bits(vals.astype(np.float32))[None, :]
    x = q.bf16_bits_to_f64(bits)[0]
    codes, scales = q.quantize_row32(bits)
    s = int(scales[0, 0])
    # the anchor fixes the scale: amax in [4, 8) * 2^E gives 2^E
    amax = np.max(np.abs(x))
    assert 4.0 <= amax / 2.0 ** (s - 127) < 8.0
    c = q.unpack_nibbles(codes)[0]
    for i in range(32):
        assert int(c[i]) == _nearest_even(x[i], 2.0 ** (s - 127)), (i, x[i], int(c[i]))


@settings(max_examples=100, deadline=None)
@given(blocks(), st.integers(min_value=-3, max_value=3))
def test_block_scale_equivariance_and_sign_symmetry(vals, k):
    bits = synth.to_bf16_bits(vals.astype(np.float32))[None, :]
    c0, s0 = q.quantize_row32(bits)
    # multiplying a block by 2^k only moves its scale; negating it only flips
    # the sign bits
    c1, s1 = q.quantize_row32(synth.to_bf16_bits((vals * 2.0 ** k).astype(np.float32))[None, :])
    np.testing.assert_array_equal(c0, c1)
    assert int(s1[0, 0]) == int(s0[0, 0]) + k
    cn, sn = q.quantize_row32(synth.to_bf16_bits((-vals).astype(np.float32))[None, :])
    np.testing.assert_array_equal(q.unpack_nibbles(cn), q.unpack_nibbles(c0) ^ 8)
    assert int(sn[0, 0]) == int(s0[0, 0])
