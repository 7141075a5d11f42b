"""GPU parity of the triple-branch linear (forward, dgrad, adapter
gradients) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from bit_quantized_amd import synth
from bit_quantized_amd.layer import FourTuneLinearFunction, bits_of

from _gpu import GpuCase, check_full, check_sampled, require_gpu, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_tiny_case_full():
    c = synth.tiny_case(0)
    say("case tiny", c.M, c.K, c.N, c.r_s, c.r_l)
    check_full(c, GpuCase(c).run())


@pytest.mark.parametrize("shape", [
    (300, 288, 544, 16, 8),      # ragged in every dimension, several tiles
    (257, 160, 96, 0, 0),        # no low-rank branches
    (64, 256, 320, 0, 8),        # adapter only
    (96, 384, 256, 16, 0),       # stabilizer only
    (130, 512, 288, 32, 32),     # R = 64
    (33, 224, 352, 24, 16),      # R = 40
    (1, 128, 64, 8, 8),          # a single token
    (2, 3072, 1024, 32, 16),     # modulation-like: two tokens, long reduction
    (520, 1024, 768, 32, 16),    # several k steps, aligned scales
    (4200, 1120, 800, 32, 16),   # several column splits of 256 with a ragged last one
    (96, 256, 320, 5, 3),        # ranks that are not multiples of 8
    (200, 640, 384, 0, 0),       # odd 128-step counts both ways (padded step), no ranks
    (200, 640, 384, 16, 8),      # the same with rank steps
])
def test_ragged_shapes_full(shape):
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"ragged_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + K)
    say("case", c.name)
    check_full(c, GpuCase(c).run())


@pytest.mark.parametrize("precision", ["W4A16G4", "W4A4G16", "W4A16G16"])
@pytest.mark.parametrize("shape", [
    (300, 288, 544, 16, 8),      # ragged, several tiles and 32-element bf16 steps
    (200, 640, 384, 0, 0),       # no low-rank branches, odd step count padded
    (2, 3072, 1024, 32, 16),     # two tokens, long reduction
])
def test_precision_settings_full(shape, precision):
    """The 16-bit settings of the precision ablation: the bf16 side is
    multiplied by the weight tiles dequantized to bf16, the rest as in
    W4A4G4."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"{precision}_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + N)
    say("case", c.name)
    check_full(c, GpuCase(c, precision).run(), precision=precision)


def test_precision_w4a16g16_qkv_full_size_sampled():
    c = synth.qkv_case()
    say("case", c.name, "W4A16G16")
    check_sampled(c, GpuCase(c, "W4A16G16").run(), _rows(c.M, seed=3), precision="W4A16G16")


@pytest.mark.parametrize("shape", [
    (300, 288, 544, 16, 8),      # ragged; K % 128 != 0: the register-staged kernel both ways
    (520, 1024, 768, 32, 16),    # the pipelined kernel both ways
    (200, 640, 384, 0, 0),       # odd step counts (padded step), no ranks
])
def test_row32_weights_full(shape):
    """Group-wise (1x32) weights, the block-shape ablation's alternative: the
    GEMMs read per-row weight scales, the dgrad a separate quantization of
    W^T (both written by one FT_Q_ROW32_T pass, checked bit for bit)."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"row32w_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + 2 * N)
    say("case", c.name)
    check_full(c, GpuCase(c, w_block="row32").run())


def test_row32_weights_qkv_full_size_sampled():
    c = synth.qkv_case()
    say("case", c.name, "row32 weights")
    check_sampled(c, GpuCase(c, w_block="row32").run(), _rows(c.M, seed=4))


def _random_shapes(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M = int(rng.integers(1, 700))
        K = 32 * int(rng.integers(1, 40))
        N = 32 * int(rng.integers(1, 40))
        rs = int(rng.integers(0, 33))
        rl = int(rng.integers(0, 65 - rs)) if rng.random() < 0.8 else 0
        out.append((M, K, N, rs, min(rl, 64 - rs)))
    return out


@pytest.mark.parametrize("shape", _random_shapes(10, 2027))
def test_random_shapes_full(shape):
    """A seeded sweep of shapes: any M, K and N multiples of 32 (so both GEMM
    kernels and every split width of the fused quantizer), ranks 0..64."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"rand_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M * 7 + K + N)
    say("case", c.name)
    check_full(c, GpuCase(c).run())


def test_fp32_adapter_gradients():
    c = synth.flux_linear_case("f32grads", 200, 256, 320, 8, 16, seed=5)
    say("case", c.name)
    check_full(c, GpuCase(c).run(grad_f32=True), grad_f32=True)


def test_zero_input_and_zero_residual():
    c = synth.flux_linear_case("zeros", 64, 128, 96, 8, 8, seed=6)
    c.X[:] = 0
    c.W_res[:] = 0
    say("case zeros")
    got = GpuCase(c).run()
    assert np.all(got["xq_codes"] == 0) and np.all(got["xq_scales"] == 0)
    check_full(c, got)


def test_deterministic():
    c = synth.flux_linear_case("det", 1000, 768, 1024, 32, 16, seed=7)
    say("case det")
    g = GpuCase(c)
    a = g.run()
    b = g.run()
    for k in ("Y", "U", "dX", "dA", "dB", "P", "xq_codes", "gq_codes"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_autograd_function_matches_library():
    c = synth.flux_linear_case("autograd", 128, 256, 192, 8, 8, seed=8)
    say("case autograd")
    g = GpuCase(c)
    X = g.X.clone().requires_grad_(True)
    At = g.layer.At.clone().requires_grad_(True)
    B = g.layer.B.clone().requires_grad_(True)
    Y = FourTuneLinearFunction.apply(X, At, B, g.layer)
    Y.backward(g.dY)
    ref = g.run()
    np.testing.assert_array_equal(bits_of(Y), ref["Y"])
    np.testing.assert_array_equal(bits_of(X.grad), ref["dX"])
    np.testing.assert_array_equal(bits_of(At.grad).T, ref["dA"])
    np.testing.assert_array_equal(bits_of(B.grad), ref["dB"])


def _rows(M, n=48, seed=0):
    rng = np.random.default_rng(seed)
    r = np.unique(np.concatenate([rng.choice(M, n, replace=False), [0, M - 1]]))
    return r


def test_qkv_full_size_sampled():
    """FLUX QKV linear at its full size (4608 x 3072 -> 9216, ranks 32/16), the
    configuration the benchmark times."""
    c = synth.qkv_case()
    say("case", c.name)
    check_sampled(c, GpuCase(c).run(), _rows(c.M))


def test_mlp_pair_full_size_sampled():
    up_c, down_c = synth.mlp_cases()
    for c in (up_c, down_c):
        say("case", c.name)
        check_sampled(c, GpuCase(c).run(), _rows(c.M, seed=1))


@pytest.mark.parametrize("name", ["img_out", "txt_qkv", "txt_mod", "img_mod"])
def test_dit_block_linears_sampled(name):
    c = synth.dit_block_case(name)
    say("case", c.name)
    check_sampled(c, GpuCase(c).run(), _rows(c.M, n=min(48, c.M - 1), seed=2) if c.M > 2
                  else np.arange(c.M))
