"""Oracle for FourTune's W4A4G4 triple-branch linear (arXiv 2607.05711).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  A plain, slow, float64 CPU
implementation written from the paper's equations and the OCP MX format
definition it cites.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import it.  It shares no code, tables or helpers
with the HIP path in bit_quantized_amd/; the only thing both sides see is
the seeded synthetic input from bit_quantized_amd.synth.

Parity status of every function: pinned by the non-GPU tests in
tests/test_oracle_*.py (closed forms, hand-worked blocks under
tests/golden/, invariants, brute force, autograd).  gelu_tanh and
gelu_tanh_grad are checked against torch's float64 GELU.
"""
from . import mxfp4, linear  # noqa: F401
