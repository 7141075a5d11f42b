"""The stabilizer ablation through the C ABI: the same outlier-laden weight
run with its top-16 SVD as the stabilizer and without it.  Each run matches
the oracle to the usual bar, and against the unquantized layer the
stabilizer cuts the Y and dX errors several-fold (FourTune section 3.1;
the CPU version of this comparison is in test_ablations.py)."""
import pytest

from bit_quantized_amd import synth
from oracle import linear as OL
from oracle import mxfp4 as q

from _gpu import GpuCase, check_full, require_gpu, say

pytestmark = pytest.mark.gpu


def test_stabilizer_ablation_gpu():
    require_gpu()
    with_stab, without = synth.outlier_weight_cases()
    W = q.bf16_bits_to_f64(with_stab.meta["W"])
    Y_ref = q.bf16_bits_to_f64(with_stab.X) @ W.T
    dX_ref = q.bf16_bits_to_f64(with_stab.dY) @ W
    err = {}
    for c in (with_stab, without):
        say("case", c.name)
        got = GpuCase(c).run()
        check_full(c, got)
        err[c.name] = (OL.rel_frobenius(got["Y"], Y_ref), OL.rel_frobenius(got["dX"], dX_ref))
    say(err)
    (y1, d1), (y0, d0) = err["outlier_w_stab"], err["outlier_w_nostab"]
    assert y1 < y0 / 3 and d1 < d0 / 3
