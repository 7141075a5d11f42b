"""GPU parity of the MXFP4 quantizers against the CPU oracle: codes and
scales must match bit for bit."""
import numpy as np
import pytest
import torch

from bit_quantized_amd import ops, synth
from oracle import mxfp4 as OQ

from _gpu import DEV, require_gpu, say, u8, up

pytestmark = pytest.mark.gpu


def _run(mode, bits, ld=None, dual=False):
    rows, cols = bits.shape
    if ld is not None and ld != cols:
        padded = np.zeros((rows, ld), dtype=np.uint16)
        padded[:, :cols] = bits
        x = up(padded)
    else:
        ld = cols
        x = up(bits)
    c = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    if mode == ops.FT_Q_TILE32:
        s = torch.empty((rows // 32, cols // 32), dtype=torch.uint8, device=DEV)
    else:
        s = torch.empty((rows, cols // 32), dtype=torch.uint8, device=DEV)
    ct = st = None
    if mode == ops.FT_Q_ROW32_T:
        ct = torch.empty((cols, rows // 2), dtype=torch.uint8, device=DEV)
        st = torch.empty((cols, rows // 32), dtype=torch.uint8, device=DEV)
    elif dual:
        ct = torch.empty((cols, rows // 2), dtype=torch.uint8, device=DEV)
        st = torch.empty((cols // 32, rows // 32), dtype=torch.uint8, device=DEV)
    ops.fourtune_quantize(mode, x, rows, cols, ld, c, s, ct, st)
    torch.cuda.synchronize()
    return u8(c), u8(s), (u8(ct) if ct is not None else None), (u8(st) if st is not None else None)


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("shape,ld", [((37, 96), None), ((5, 32), 40), ((256, 4096), None),
                                      ((1, 12288), None), ((300, 288), 296)])
def test_row32_random(shape, ld):
    rng = np.random.default_rng(sum(shape))
    x = synth.to_bf16_bits(rng.standard_t(3, size=shape) * np.exp2(rng.integers(-30, 30, (shape[0], 1))))
    say("row32", shape, ld)
    c, s, _, _ = _run(ops.FT_Q_ROW32, x, ld)
    ec, es = OQ.quantize_row32(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)


def test_row32_adversarial_blocks():
    blocks = synth.adversarial_blocks(1, 6000)             # [6000, 32]
    x = blocks.reshape(600, 320)
    say("row32 adversarial")
    c, s, _, _ = _run(ops.FT_Q_ROW32, x)
    ec, es = OQ.quantize_row32(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)


def test_row32_every_bf16_value_at_every_scale_regime():
    # each block: one scale-setting amax and 31 consecutive bf16 bit patterns,
    # sweeping all finite non-negative and negative patterns
    pats = np.concatenate([np.arange(0, 0x7F80), np.arange(0x8000, 0xFF80)]).astype(np.uint16)
    n = (pats.size + 30) // 31
    pats = np.resize(pats, n * 31).reshape(n, 31)
    rng = np.random.default_rng(2)
    lead = (rng.integers(0, 0x7F80, n)).astype(np.uint16)
    x = np.concatenate([lead[:, None], pats], axis=1)
    x = x[: (n // 10) * 10].reshape(-1, 320)
    say("row32 all bf16 patterns", x.shape)
    c, s, _, _ = _run(ops.FT_Q_ROW32, x)
    ec, es = OQ.quantize_row32(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)


@pytest.mark.parametrize("dual", [False, True])
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (64, 416), (128, 4096), (320, 544)])
def test_tile32(shape, dual):
    rng = np.random.default_rng(shape[1])
    w = synth.to_bf16_bits(rng.standard_normal(shape) * 0.02 *
                           np.exp2(rng.integers(-10, 10, (shape[0] // 32, 1, shape[1] // 32, 1)))
                           .repeat(32, 1).repeat(32, 3).reshape(shape))
    w[:32, :32] = 0            # an all-zero tile
    say("tile32", shape, "dual" if dual else "")
    c, s, ct, st = _run(ops.FT_Q_TILE32, w, dual=dual)
    ec, es = OQ.quantize_tile32(w)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)
    if dual:
        # a 32x32 tile's scale does not depend on the orientation, so the
        # transposed codes are the tile quantization of the transpose
        ect, est = OQ.quantize_tile32(np.ascontiguousarray(w.T))
        np.testing.assert_array_equal(st, est)
        np.testing.assert_array_equal(ct, ect)


def test_tile32_adversarial():
    x = synth.adversarial_blocks(3, 96 * 12).reshape(96, 384)
    say("tile32 adversarial")
    c, s, _, _ = _run(ops.FT_Q_TILE32, x)
    ec, es = OQ.quantize_tile32(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)


@pytest.mark.parametrize("shape", [(32, 32), (64, 64), (96, 160), (160, 96), (544, 288), (512, 512),
                                   (800, 1056)])
def test_row32_t(shape):
    x = synth.stress_activation(seed=shape[0], rows=shape[0], cols=shape[1], zero_tile_frac=0.1)
    say("row32_t", shape)
    c, s, ct, st = _run(ops.FT_Q_ROW32_T, x)
    ec, es = OQ.quantize_row32(x)
    ect, est = OQ.quantize_row32_t(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)
    np.testing.assert_array_equal(st, est)
    np.testing.assert_array_equal(ct, ect)


def test_row32_t_adversarial():
    x = synth.adversarial_blocks(4, 64 * 10).reshape(64, 320)
    say("row32_t adversarial")
    c, s, ct, st = _run(ops.FT_Q_ROW32_T, x)
    ec, es = OQ.quantize_row32(x)
    ect, est = OQ.quantize_row32_t(x)
    np.testing.assert_array_equal(s, es)
    np.testing.assert_array_equal(c, ec)
    np.testing.assert_array_equal(st, est)
    np.testing.assert_array_equal(ct, ect)


def _sample_blocks(rng, rows, cols, n):
    r = rng.integers(0, rows, n)
    b = rng.integers(0, cols // 32, n)
    return r, b


def test_stress_full_size_row32_t_sampled():
    """Quantizer stress workload at its full size (bf16 16384 x 12288), dual output,
    in the launch configuration the benchmark times; sampled blocks vs the oracle,
    plus the all-zero-block property everywhere."""
    T = synth.stress_activation()
    rows, cols = T.shape
    say("stress row32_t full", T.shape)
    c, s, ct, st = _run(ops.FT_Q_ROW32_T, T)
    rng = np.random.default_rng(0)
    r, b = _sample_blocks(rng, rows, cols, 4096)
    blocks = OQ.bf16_bits_to_f64(T[r[:, None], 32 * b[:, None] + np.arange(32)])
    ec, es = OQ.quantize_blocks(blocks)
    np.testing.assert_array_equal(s[r, b], es)
    np.testing.assert_array_equal(OQ.unpack_nibbles(c[r[:, None], 16 * b[:, None] + np.arange(16)]), ec)
    cc, rb = _sample_blocks(rng, cols, rows, 4096)
    blocks = OQ.bf16_bits_to_f64(T[32 * rb[:, None] + np.arange(32), cc[:, None]])
    ec, es = OQ.quantize_blocks(blocks)
    np.testing.assert_array_equal(st[cc, rb], es)
    np.testing.assert_array_equal(OQ.unpack_nibbles(ct[cc[:, None], 16 * rb[:, None] + np.arange(16)]), ec)
    # zero tiles: every 32x32 all-zero tile gives zero scales and codes in both layouts
    Tz = np.all(T.reshape(rows // 32, 32, cols // 32, 32) == 0, axis=(1, 3))
    zi, zj = np.nonzero(Tz)
    assert zi.size > 1000
    assert np.all(s[32 * zi, zj] == 0) and np.all(st[32 * zj, zi] == 0)


def test_stress_full_size_tile32_sampled():
    W = synth.stress_weight()
    n = W.shape[0]
    say("stress tile32 full", W.shape)
    c, s, _, _ = _run(ops.FT_Q_TILE32, W)
    rng = np.random.default_rng(1)
    ti = rng.integers(0, n // 32, 256)
    tj = rng.integers(0, n // 32, 256)
    for i, j in zip(ti, tj):
        blk = W[32 * i:32 * i + 32, 32 * j:32 * j + 32]
        ec, es = OQ.quantize_tile32(blk)
        assert s[i, j] == es[0, 0]
        np.testing.assert_array_equal(c[32 * i:32 * i + 32, 16 * j:16 * j + 16], ec)


def _dequant(codes, scales):
    rows, cols = codes.shape[0], codes.shape[1] * 2
    c = torch.from_numpy(np.ascontiguousarray(codes)).to(DEV)
    s = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    out = torch.empty((rows, cols), dtype=torch.int16, device=DEV)
    ops.fourtune_dequantize(ops.FT_Q_TILE32, c, s, rows, cols, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (320, 544), (1024, 4096)])
def test_dequant_tile32_every_code_and_scale(shape):
    """Arbitrary code bytes (every nibble, both signs of zero) under scale bytes
    0..252 (the whole range a finite input is quantized to: bf16 subnormal
    results included) against the oracle's exact values rounded to bf16."""
    rng = np.random.default_rng(shape[1])
    rows, cols = shape
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 253, size=(rows // 32, cols // 32), dtype=np.uint8)
    scales.flat[:3] = (0, 1, 252)
    say("dequant tile32", shape)
    got = _dequant(codes, scales)
    np.testing.assert_array_equal(got, OQ.f64_to_bf16_bits(OQ.dequantize_tile32(codes, scales)))


def test_dequant_tile32_of_quantized_weight():
    """Dequantizing Qtile(W) (plain and transposed copies) gives the oracle's
    deq(Qtile(W)) and deq(Qtile(W))^T bit for bit."""
    rng = np.random.default_rng(9)
    w = synth.to_bf16_bits(rng.standard_normal((288, 640)) * 0.02 *
                           np.exp2(rng.integers(-20, 20, (9, 1, 20, 1))).repeat(32, 1).repeat(32, 3)
                           .reshape(288, 640))
    say("dequant of a quantized weight")
    c, s, ct, st = _run(ops.FT_Q_TILE32, w, dual=True)
    ref = OQ.f64_to_bf16_bits(OQ.dequantize_tile32(*OQ.quantize_tile32(w)))
    np.testing.assert_array_equal(_dequant(c, s), ref)
    np.testing.assert_array_equal(_dequant(ct, st), np.ascontiguousarray(ref.T))
