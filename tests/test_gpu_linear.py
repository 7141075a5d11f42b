"""GPU parity of the triple-branch linear (forward, dgrad, adapter
gradients) against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from bit_quantized_amd import ops, synth
from bit_quantized_amd.layer import FourTuneLinearFunction, QuantizedLinear, bits_of
from oracle import linear as OL
from oracle import mxfp4 as OQ

from _gpu import REL_TOL, GpuCase, check_full, check_sampled, require_gpu, say, up

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
    # the dgrad reads the forward's tiles transposed; K / 32 not a multiple
    # of 4 puts each reduction block's run of tile scales at a byte offset
    # inside its first word (pipelined dgrad: N % 128 == 0)
    (300, 288, 512, 16, 8),      # K / 32 = 9
    (96, 160, 256, 0, 0),        # K / 32 = 5, no ranks
    (260, 224, 384, 32, 16),     # K / 32 = 7
    # more than 64 ranks: four rank steps per GEMM tile, 5 to 8 rank groups
    # in the fused quantizer, dB fused up to r_l = 64, two adapter-gradient
    # passes above that
    (300, 288, 544, 32, 64),     # R = 96, ragged in every dimension
    (260, 224, 384, 32, 64),     # R = 96, pipelined dgrad on the packed weight
    (130, 512, 288, 64, 64),     # R = 128, the cap
    (200, 640, 384, 48, 40),     # R = 88 (run as 96), dB over 3 rank groups
    (96, 256, 320, 5, 70),       # r_l > 64, ranks not multiples of 8
    (64, 256, 256, 0, 128),      # adapter only, 128 ranks
    (4200, 1120, 800, 32, 64),   # several column splits with a ragged last one
    # few rows: both GEMMs split their reduction over units that write fp32
    # sums, added (with the rank part) by a second kernel
    (2, 3072, 18432, 32, 16),    # the modulation linear of a DiT block
    (16, 1024, 768, 32, 16),     # 3 output tiles each way
    (64, 2048, 4096, 16, 8),     # the largest row count that splits
    (5, 512, 288, 8, 8),         # ragged columns, 2 step pairs
    (16, 1152, 768, 0, 0),       # no ranks; odd step count: the last split pads
    (1024, 3072, 768, 32, 16),   # many rows, few tiles: the forward splits
    (600, 4096, 1024, 16, 8),    # ragged rows past a 256-row tile
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
    (2, 3072, 1024, 32, 16),     # two rows: the streaming kernel both ways (per-row b scales)
    (13, 1152, 640, 16, 8),      # 13 rows, 9 steps (a partial batch)
])
def test_row32_weights_full(shape):
    """Group-wise (1x32) weights, the block-shape ablation's alternative: the
    GEMMs read per-row weight scales, the dgrad a separate quantization of
    W^T (both written by one FT_Q_ROW32_T pass, checked bit for bit)."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"row32w_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + 2 * N)
    say("case", c.name)
    check_full(c, GpuCase(c, w_block="row32").run())


@pytest.mark.parametrize("shape", [
    (300, 288, 544, 16, 8),      # register-staged dgrad
    (520, 1024, 768, 32, 16),    # pipelined dgrad
    (96, 160, 256, 0, 0),        # pipelined, no ranks
    (2, 3072, 1024, 32, 16),     # two rows: the streaming kernel reads the copy
])
def test_tile32_transposed_copy_full(shape):
    """The measured alternative to the method's single weight: the tiles
    plus a stored transposed layout copy (FT_WBLOCK_TILE32_T), which the
    dgrad reads row-wise.  The copy must hold exactly Qtile(W^T) and give
    the same layer."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"tile32t_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + 3 * N)
    say("case", c.name)
    check_full(c, GpuCase(c, w_block="tile32_t").run())


def test_tile32_reads_agree_bitwise():
    """The dgrad on the one packed weight (transposing LDS reads) and on the
    stored transposed copy (row reads) add the same products in the same
    order: dX must agree bit for bit."""
    c = synth.flux_linear_case("tile32_vs_copy", 700, 1024, 1536, 32, 16, seed=11)
    say("case", c.name)
    a = GpuCase(c).run()
    b = GpuCase(c, w_block="tile32_t").run()
    for k in ("Y", "dX", "dA", "dB", "U", "P", "gq_codes"):
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_multi_tile_walk_full():
    """4608 x 4608 x 4608 (ranks 32/16): 324 output tiles each way on 256
    workgroups, so some workgroups of both GEMMs walk two tiles and the
    load pipeline runs across a tile boundary; compared in full."""
    c = synth.flux_linear_case("multi_tile_4608", 4608, 4608, 4608, 32, 16, seed=12)
    say("case", c.name)
    check_full(c, GpuCase(c).run())


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
        rs = int(rng.integers(0, 65))
        rl = int(rng.integers(0, 129 - rs)) if rng.random() < 0.8 else 0
        out.append((M, K, N, rs, min(rl, 128 - rs)))
    return out


@pytest.mark.parametrize("shape", _random_shapes(12, 2027))
def test_random_shapes_full(shape):
    """A seeded sweep of shapes: any M, K and N multiples of 32 (so both GEMM
    kernels and every split width of the fused quantizer), ranks 0..128."""
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


@pytest.mark.parametrize("shape", [
    (520, 1024, 768, 32, 16),    # 12 dgrad tiles: nearly every CU free
    (4608, 3072, 9216, 32, 16),  # the QKV layer: 216 dgrad tiles, 40 CUs free
    (300, 288, 512, 16, 64),     # 64 adapter ranks (4 rank groups), ragged rows
    (8192, 3072, 9216, 32, 16),  # 384 dgrad tiles: the extra workgroups take the
                                 # 128 CUs that finish a round early
])
def test_adapter_gradient_beside_dgrad(shape):
    """dA and dB made by the dgrad's launch on the CUs its tiles leave free
    (no adapter-gradient launch) against those of the adapter-gradient
    kernels themselves (the same backward without dX): bit for bit, and P
    unchanged.  The library's kernel timing names which path ran."""
    M, K, N, rs, rl = shape
    c = synth.flux_linear_case(f"beside_{M}x{K}x{N}_r{rs}_{rl}", M, K, N, rs, rl, seed=M + N)
    say("case", c.name)
    g = GpuCase(c)
    _, U = g.layer.forward(g.X)
    torch.cuda.synchronize()

    def bwd(need_dx):
        ops.fourtune_timing_reset()
        ops.fourtune_timing_enable(True)
        out = g.layer.backward(g.dY, g.X, U, need_dx=need_dx)
        torch.cuda.synchronize()
        ops.fourtune_timing_enable(False)
        names = {k for k, (_, n) in ops.fourtune_timing_read().items() if n}
        return out, names

    (dX, dA1, dB1, P1), n1 = bwd(True)
    (_, dA0, dB0, P0), n0 = bwd(False)
    assert "bwd_gemm_dgrad" in n1 and "bwd_lora_grads" not in n1, n1
    assert "bwd_lora_grads" in n0 and "bwd_gemm_dgrad" not in n0, n0
    np.testing.assert_array_equal(bits_of(dA1), bits_of(dA0))
    np.testing.assert_array_equal(bits_of(dB1), bits_of(dB0))
    np.testing.assert_array_equal(bits_of(P1), bits_of(P0))
    assert dX is not None


def test_adapter_gradient_own_launch_with_gelu_input():
    """A layer whose input is gelu(h) keeps its adapter gradients in their
    own launch (GELU on X is not recomputed beside the dgrad)."""
    c = synth.flux_linear_case("gelu_in_lora", 256, 512, 384, 16, 8, seed=10)
    say("case", c.name)
    g = GpuCase(c)
    layer = QuantizedLinear.from_factors(up(c.W_res), up(c.L1), up(c.L2), up(c.A), up(c.B),
                                         act_in=ops.FT_ACT_GELU_TANH)
    _, U = layer.forward(g.X)
    ops.fourtune_timing_reset()
    ops.fourtune_timing_enable(True)
    layer.backward(g.dY, g.X, U)
    torch.cuda.synchronize()
    ops.fourtune_timing_enable(False)
    names = {k for k, (_, n) in ops.fourtune_timing_read().items() if n}
    assert "bwd_lora_grads" in names, names


def test_autograd_function_act_in():
    """A layer whose input is gelu(h) used through the autograd Function:
    h's gradient is the layer's input gradient times gelu'(h).  Checked
    against the oracle fed the GPU's gelu(h) values, with the oracle's own
    gelu' applied to the oracle's input gradient."""
    c = synth.flux_linear_case("act_in_autograd", 256, 512, 384, 16, 8, seed=9)
    say("case act_in autograd")
    g = GpuCase(c)
    layer = QuantizedLinear.from_factors(up(c.W_res), up(c.L1), up(c.L2), up(c.A), up(c.B),
                                         act_in=ops.FT_ACT_GELU_TANH)
    h = g.X.clone().requires_grad_(True)
    At = layer.At.clone().requires_grad_(True)
    B = layer.B.clone().requires_grad_(True)
    Y = FourTuneLinearFunction.apply(h, At, B, layer)
    Y.backward(g.dY)
    torch.cuda.synchronize()
    a = torch.empty_like(g.X)
    ops.fourtune_act_fwd(ops.FT_ACT_GELU_TANH, g.X, g.X.numel(), a)
    torch.cuda.synchronize()
    a_bits = bits_of(a)
    wc, ws = OQ.quantize_tile32(c.W_res)
    f = OL.linear_fwd(a_bits, wc, ws, c.L1, c.L2, c.A, c.B)
    b = OL.linear_bwd(c.dY, a_bits, f["U"], wc, ws, c.L1, c.L2, c.A, c.B)
    dh_ref = OL.gelu_tanh_grad(c.X, b["dX"])
    errs = {"Y": OL.rel_frobenius(bits_of(Y), f["Y"]),
            "dh": OL.rel_frobenius(bits_of(h.grad), dh_ref),
            "dA": OL.rel_frobenius(np.ascontiguousarray(bits_of(At.grad).T), b["dA"]),
            "dB": OL.rel_frobenius(bits_of(B.grad), b["dB"])}
    say("act_in autograd", errs)
    for k, v in errs.items():
        assert v <= REL_TOL, (k, v)
    # the input gradient is not the library's dX itself
    dX_lib = layer.backward(g.dY, g.X, layer.forward(g.X)[1])[0]
    assert not np.array_equal(bits_of(h.grad), bits_of(dX_lib))


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


def test_qkv_full_size_rank96_sampled():
    """The QKV linear at its full size with an adapter of rank 64 (R = 96):
    four rank steps per GEMM tile, dB fused over four rank groups."""
    c = synth.flux_linear_case("qkv_4608x3072x9216_r32_64", 4608, 3072, 9216, 32, 64, seed=3)
    say("case", c.name)
    check_sampled(c, GpuCase(c).run(), _rows(c.M, seed=5))


def test_mlp_pair_full_size_sampled():
    up_c, down_c = synth.mlp_cases()
    for c in (up_c, down_c):
        say("case", c.name)
        check_sampled(c, GpuCase(c).run(), _rows(c.M, seed=1))


@pytest.mark.parametrize("name", [n for n, *_ in synth.dit_block_linears()])
def test_dit_block_linears_sampled(name):
    """Every linear of the double-stream DiT block at batch 2."""
    c = synth.dit_block_case(name)
    say("case", c.name)
    check_sampled(c, GpuCase(c).run(), _rows(c.M, n=min(48, c.M - 1), seed=2) if c.M > 2
                  else np.arange(c.M))
