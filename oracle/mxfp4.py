"""Plain CPU oracle for the MXFP4 codec used by FourTune's W4A4G4 linear.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the CPU-baseline
leg of the benchmark do.  It shares no code with the HIP path.

What is computed (FourTune, arXiv 2607.05711, "2.3 Model Quantization":
quantization maps a tensor to low-bit codes via Round(W / s) with a
group scale s, citing MXFP4 as one such format; "3.2 4-Bit Backward Pass via
Block-Quantization": block-wise scales that stay local to a tile).  The
format details come from the OCP Microscaling (MX) v1.0 specification that
the page cites for MXFP4:

* element: E2M1, magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign bit 3;
* scale:   E8M0, value 2**(code - 127), one byte per block;
* scale choice: exponent floor(log2(amax)) - emax_elem, emax_elem = 2;
* element rounding: round-to-nearest, ties to the even code, saturating
  at 6.

Readings taken where the pages are silent (each one is listed in the design
notes):

* blocks are 1x32 along the last (reduction) axis for activations and
  gradients, and 32x32 square tiles for the frozen residual weight;
* the scale code is clamped to [0, 254]; an all-zero block gets code 0;
* the sign bit is the IEEE sign of the input, so -0.0 and small negative
  values that round to zero encode as 0x8;
* packing: byte i of a row holds element 2i in the low nibble and element
  2i+1 in the high nibble; scale bytes are row-major.

Everything here works on bf16 bit patterns (uint16), widened exactly to
float64.  The code favours being checkable by eye over speed.
"""
from __future__ import annotations

import numpy as np

# E2M1 magnitudes indexed by the 3-bit magnitude code (OCP MX v1.0, FP4 E2M1).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_EMAX = 2          # exponent of the largest normal E2M1 value (6 = 1.5 * 2**2)
E8M0_BIAS = 127
E8M0_MAX_FINITE = 254  # 0xFF is NaN in E8M0
BLOCK = 32


# --------------------------------------------------------------------------
# bf16 <-> float64
# --------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: bf16 is the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (round to nearest, ties to even), as bits.

    bf16 has 8 significant bits (1 implicit + 7 stored) and fp32's exponent
    range, so a value in [2**(e-1), 2**e) is a multiple of 2**(e-8), and
    subnormals are multiples of 2**-133.  np.rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("non-finite value")
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.rint(x / quantum) * quantum       # exact: division by a power of two
    if np.any(np.abs(r) >= 2.0 ** 128):
        raise OverflowError("value overflows bf16")
    f32 = r.astype(np.float32)               # exact: r has <= 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """Round float64 to float32 (numpy's cast rounds to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------
# E2M1 element codec
# --------------------------------------------------------------------------
def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    """Value of 4-bit E2M1 codes (bit 3 = sign, bits 0-2 index the magnitude)."""
    c = np.asarray(codes, dtype=np.uint8)
    mag = E2M1_MAGNITUDES[c & 0x7]
    return np.where((c & 0x8) != 0, -mag, mag)


def e2m1_encode(t: np.ndarray) -> np.ndarray:
    """Encode already-scaled values t onto E2M1.

    Nearest representable magnitude; on an exact tie between two neighbours
    the one with the even code wins (round half to even on the code, which
    is the IEEE rule for a 1-bit mantissa).  Magnitudes above 6 saturate to
    6 because 6 is then the nearest point.  The sign bit is the IEEE sign
    of t (so -0.0 gives 0x8).
    """
    t = np.asarray(t, dtype=np.float64)
    # Every |t| >= 7 has 6 as its nearest point; clipping at 8 keeps that
    # while keeping the distances below exact in float64 for huge inputs.
    a = np.minimum(np.abs(t), 8.0).reshape(-1)
    dist = np.abs(a[:, None] - E2M1_MAGNITUDES[None, :])       # [n, 8]
    best = np.argmin(dist, axis=1)                              # lowest index on ties
    dmin = dist[np.arange(a.size), best]
    nxt = np.minimum(best + 1, 7)
    tie = (best < 7) & (dist[np.arange(a.size), nxt] == dmin)
    # two nearest points are adjacent codes, exactly one of them is even
    best = np.where(tie & (best % 2 == 1), nxt, best)
    sign = np.signbit(t).reshape(-1).astype(np.uint8) << 3
    return (best.astype(np.uint8) | sign).reshape(t.shape)


# --------------------------------------------------------------------------
# E8M0 block scale
# --------------------------------------------------------------------------
def e8m0_decode(code: np.ndarray) -> np.ndarray:
    """2**(code - 127) for finite codes 0..254."""
    c = np.asarray(code, dtype=np.int64)
    if np.any((c < 0) | (c > E8M0_MAX_FINITE)):
        raise ValueError("E8M0 code out of the finite range")
    return np.ldexp(1.0, c - E8M0_BIAS)


def e8m0_from_amax(amax: np.ndarray) -> np.ndarray:
    """Shared block exponent: floor(log2(amax)) - 2, biased by 127, clamped.

    amax == 0 (an all-zero block) gives code 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    if not np.all(np.isfinite(a)) or np.any(a < 0):
        raise ValueError("amax must be finite and >= 0")
    _, e = np.frexp(a)                 # a = m * 2**e, m in [0.5, 1)  =>  floor(log2 a) = e - 1
    code = (e - 1) - E2M1_EMAX + E8M0_BIAS
    code = np.where(a == 0.0, 0, code)
    return np.clip(code, 0, E8M0_MAX_FINITE).astype(np.uint8)


# --------------------------------------------------------------------------
# block quantization
# --------------------------------------------------------------------------
def quantize_blocks(v: np.ndarray):
    """Quantize blocks given as rows of v [nblocks, block_len] (float64).

    Returns (codes uint8 [nblocks, block_len], scale codes uint8 [nblocks]).
    Each element is divided by its block's power-of-two scale (exact) and
    then encoded.
    """
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input")
    amax = np.max(np.abs(v), axis=1)
    s = e8m0_from_amax(amax)
    t = v / e8m0_decode(s)[:, None]
    return e2m1_encode(t), s


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """[..., 2n] 4-bit codes -> [..., n] bytes, element 2i in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def quantize_row32(x_bits: np.ndarray):
    """1x32 blocks along the last axis of a bf16 matrix [rows, cols].

    Returns packed codes uint8 [rows, cols/2] and scales uint8 [rows, cols/32].
    """
    x = bf16_bits_to_f64(x_bits)
    rows, cols = x.shape
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    codes, s = quantize_blocks(x.reshape(rows * cols // BLOCK, BLOCK))
    return pack_nibbles(codes.reshape(rows, cols)), s.reshape(rows, cols // BLOCK)


def quantize_row32_t(x_bits: np.ndarray):
    """1x32 blocks of the transpose: quantize_row32(x.T).

    Returns codes [cols, rows/2] and scales [cols, rows/32].
    """
    return quantize_row32(np.ascontiguousarray(np.asarray(x_bits, dtype=np.uint16).T))


def quantize_tile32(w_bits: np.ndarray):
    """32x32 square tiles sharing one scale (the weight format).

    Returns packed codes uint8 [rows, cols/2] (row-major, same element order
    as the input) and tile scales uint8 [rows/32, cols/32].
    """
    w = bf16_bits_to_f64(w_bits)
    rows, cols = w.shape
    if rows % BLOCK or cols % BLOCK:
        raise ValueError("rows and cols must be multiples of 32")
    tr, tc = rows // BLOCK, cols // BLOCK
    tiles = w.reshape(tr, BLOCK, tc, BLOCK).transpose(0, 2, 1, 3).reshape(tr * tc, BLOCK * BLOCK)
    codes, s = quantize_blocks(tiles)
    codes = codes.reshape(tr, tc, BLOCK, BLOCK).transpose(0, 2, 1, 3).reshape(rows, cols)
    return pack_nibbles(codes), s.reshape(tr, tc)


def dequantize_row32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of 1x32-block MXFP4 data."""
    vals = e2m1_decode(unpack_nibbles(codes))
    rows, cols = vals.shape
    sc = e8m0_decode(np.asarray(scales))
    return vals * np.repeat(sc, BLOCK, axis=1).reshape(rows, cols)


def dequantize_tile32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact float64 values of 32x32-tile MXFP4 data."""
    vals = e2m1_decode(unpack_nibbles(codes))
    sc = e8m0_decode(np.asarray(scales))
    return vals * np.repeat(np.repeat(sc, BLOCK, axis=0), BLOCK, axis=1)
