"""The GPU tests' elementwise checker, exercised on the CPU: results summed
in fp32 (numpy's float32 matrix product, another accumulation order than
the oracle's float64) pass, and a planted error fails."""
import numpy as np
import pytest

from oracle import mxfp4 as OQ

from _gpu import check_rounding_flips


def _case(seed, m=64, k=3072, n=48, cancel=False):
    rng = np.random.default_rng(seed)
    x = OQ.f64_to_bf16_bits(rng.standard_normal((m, k)))
    d = OQ.f64_to_bf16_bits(rng.standard_normal((k, n)) * (0.05 if cancel else 1.0))
    xf, df = OQ.bf16_bits_to_f64(x), OQ.bf16_bits_to_f64(d)
    exact = xf @ df
    absdot = np.abs(xf) @ np.abs(df)
    f32 = (xf.astype(np.float32) @ df.astype(np.float32)).astype(np.float64)
    return OQ.f64_to_bf16_bits(f32), exact, absdot, k


@pytest.mark.parametrize("seed", range(4))
def test_fp32_accumulated_sums_pass(seed):
    got, exact, absdot, k = _case(seed, cancel=seed % 2 == 1)
    check_rounding_flips(got, exact, "fp32 sum", absdot, k)
    f32 = OQ.f64_to_f32(exact)                     # the fp32 output mode
    check_rounding_flips(f32, exact, "fp32 out", absdot, k)


def test_planted_errors_fail():
    got, exact, absdot, k = _case(7)
    bad = got.copy()
    bad[3, 5] = OQ.f64_to_bf16_bits(OQ.bf16_bits_to_f64(bad[3, 5]) * 1.03)   # a few ulps off
    with pytest.raises(AssertionError):
        check_rounding_flips(bad, exact, "planted", absdot, k)
    bad = got.copy()
    bad[0, 0] ^= 0x8000                                                         # sign flip
    with pytest.raises(AssertionError):
        check_rounding_flips(bad, exact, "planted sign", absdot, k)
    # one step off where the exact sum is close to a representable value and
    # the accumulation error is small against the spacing
    ref = OQ.f64_to_bf16_bits(exact)
    rv = OQ.bf16_bits_to_f64(ref)
    spacing = np.ldexp(1.0, np.frexp(np.abs(rv))[1] - 8)
    eps = (k / 16.0 + 64.0) * 2.0 ** -24 * absdot
    score = np.where(eps < 0.2 * spacing, np.abs(exact - rv) / spacing, np.inf)
    i = np.unravel_index(np.argmin(score), exact.shape)
    assert np.isfinite(score[i])
    bad = ref.copy()
    bad[i] = bad[i] + 1
    with pytest.raises(AssertionError):
        check_rounding_flips(bad, exact, "planted step", absdot, k)
