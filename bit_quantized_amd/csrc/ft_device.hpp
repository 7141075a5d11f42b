// Device-side building blocks shared by the HIP kernels of libfourtune:
// vector types, bf16 rounding, the MXFP4 block-scale rule and wrappers of
// the gfx950 matrix-core and conversion instructions.
//
// MXFP4 (OCP Microscaling v1.0, the format FourTune's "2.3 Model
// Quantization" cites): a block of 32 (or a 32x32 tile) shares one E8M0
// scale 2^(s-127) with s = floor(log2(amax)) - 2 + 127, clamped to >= 0;
// elements are E2M1, rounded to nearest with ties to even and saturated at
// 6.  On gfx950, v_cvt_scalef32_pk_fp4_bf16 divides two bf16 values by a
// power-of-two fp32 scale and encodes them that way (round to nearest even,
// saturating, sign of zero kept), including the fp32-denormal scale 2^-127.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ft {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

#define FT_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round a finite fp32 to bf16, nearest with ties to even.
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_rne(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_rne(hi)) << 16);
}

// ---------------------------------------------------------------- MXFP4 scale
// Magnitude bits of two packed bf16 (sign bits cleared).
__device__ __forceinline__ uint32_t abs_bf16x2(uint32_t w) { return w & 0x7FFF7FFFu; }

// Lane-wise max of two packed u16 pairs (v_pk_max_u16).
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  u16x2 x = __builtin_bit_cast(u16x2, a);
  u16x2 y = __builtin_bit_cast(u16x2, b);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Largest magnitude (as bf16 magnitude bits) in a packed-max accumulator.
__device__ __forceinline__ uint32_t hmax_u16x2(uint32_t m) {
  uint32_t lo = m & 0xFFFFu, hi = m >> 16;
  return lo > hi ? lo : hi;
}

// E8M0 scale byte from the bf16 magnitude bits of the block amax:
// floor(log2(amax)) is the unbiased exponent for normals; bf16 subnormals
// and zero have exponent field 0 and give 0 after the clamp.
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits) {
  int e = static_cast<int>(amax_bits >> 7) - 2;
  e = e < 0 ? 0 : e;
  return static_cast<uint32_t>(e > 254 ? 254 : e);
}

// The scale 2^(s-127) as an fp32 value; s == 0 is the denormal 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s ? (s << 23) : 0x00400000u);
}

// Encode 8 bf16 (4 packed words) to 8 E2M1 codes (one u32, element i in
// nibble i) with scale `sc`.
__device__ __forceinline__ uint32_t encode8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3,
                                            float sc) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w0), sc, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w1), sc, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w2), sc, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, __builtin_bit_cast(bf16x2, w3), sc, 3);
  return r;
}

// ---------------------------------------------------------------- scheduling
// Workgroup i of n -> logical index, so that the workgroups the hardware
// sends to one XCD (i % 8; each XCD has its own L2) get consecutive logical
// indices.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t x = i & 7, j = i >> 3, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + j;
}

// ---------------------------------------------------------------- matrix cores
// 32x32x64 MXFP4 x MXFP4 -> fp32.  Lane l supplies 32 E2M1 codes (16 bytes)
// of row/column l%32 for reduction block l/32, and the E8M0 scale of that
// block in byte OPSEL of its scale word.
template <int OPA, int OPB>
__device__ __forceinline__ f32x16 mfma_fp4_32x32x64(u32x4 a, u32x4 b, f32x16 c, uint32_t sa,
                                                    uint32_t sb) {
  i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, OPA, (int)sa, OPB,
                                                         (int)sb);
}

// 32x32x16 bf16 -> fp32 (same accumulator layout as the fp4 instruction).
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x32 bf16 -> fp32.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x16 bf16 -> fp32: lane l supplies 4 reduction values of row (A) or
// column (B) l % 16, reduction indices 4 (l / 16) .. +3.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x16(i32x2 a, u32x2 b, f32x4 c) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// 64-bit LDS read with a 16x16 transpose of 4-bit elements across each
// group of 16 lanes: lane q of a group receives nibble q of the 8 bytes
// addressed by each of the 16 lanes, in lane order.  `p` must point into
// __shared__ memory.
__device__ __forceinline__ u32x2 lds_read_tr4(const void* p) {
  i32x2 r = __builtin_amdgcn_ds_read_tr4_b64_v2i32((FT_LDS i32x2*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// 64-bit LDS read with a transpose of 16-bit elements across each group of
// 16 lanes: lane q receives element q % 4 of the 8-byte chunks addressed by
// lanes q/4, q/4 + 4, q/4 + 8 and q/4 + 12, in that order (layout probed
// on the target).  With lane j of a group addressing row k0 + j/4, columns
// c0 + 4 (j % 4) .. +3 of a row-major bf16 tile, lane q receives rows
// k0 .. k0+3 of column c0 + q: four consecutive reduction indices of one
// MFMA operand column.  `p` must point into __shared__ memory.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FT_LDS s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// 128-bit read from __shared__ memory.
__device__ __forceinline__ u32x4 lds_read_b128(const void* p) {
  return *(const FT_LDS u32x4*)(p);
}

// ---------------------------------------------------------------- activation
// tanh-form GELU between the two linears of an MLP block (FourTune, "3.3
// Kernel Fusion for Efficiency / MLP Fusion" names GeLU on the wide
// intermediate):  gelu(h) = h * (1 + tanh(u)) / 2,  u = sqrt(2/pi) (h + 0.044715 h^3).
// With z = 2u and e = exp(-|z|) <= 1:
//   (1 + tanh(u)) / 2 = sigmoid(z) = s,   s = 1/(1+e) (z >= 0) or e/(1+e) (z < 0),
//   1 - s = e/(1+e) (z >= 0) or 1/(1+e) (z < 0),
//   gelu'(h) = s + h s (1 - s) dz/dh,     dz/dh = 2 sqrt(2/pi) (1 + 3 * 0.044715 h^2),
// so neither tail overflows.  The hardware exp2 flushes results below
// 2^-126, so it computes E = e * 2^64 (at most 2^64) and the scale comes out
// in the last multiplication of the z < 0 branch.  1/(1+e) is the hardware
// reciprocal (1 ulp).  In gelu' the polynomial uses h clamped to [-16, 16]:
// beyond that the second term is below 2^-100 of the first (z >= 0) or the
// whole value underflows (z < 0), and the clamp keeps 0 * inf out.  fp32
// throughout, every operation written out (no contraction), so that every
// kernel that calls these gets the same bits; the caller rounds to bf16 once.
constexpr float kGeluC2 = 1.5957691216057308f;      // 2 sqrt(2/pi)
constexpr float kGeluC2A = 0.07135481627260025f;    // 2 sqrt(2/pi) * 0.044715
constexpr float kGeluC6A = 0.21406444881780076f;    // 6 sqrt(2/pi) * 0.044715
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kTwo64 = 18446744073709551616.0f;   // 2^64
constexpr float kTwoM64 = 5.421010862427522e-20f;   // 2^-64

// gelu(h) = h s
__device__ __forceinline__ float gelu_tanh_f32(float h) {
#pragma clang fp contract(off)
  const float z = h * __builtin_fmaf(kGeluC2A, h * h, kGeluC2);
  const float E = __builtin_amdgcn_exp2f(__builtin_fmaf(-__builtin_fabsf(z), kLog2e, 64.0f));
  const float inv = __builtin_amdgcn_rcpf(__builtin_fmaf(E, kTwoM64, 1.0f));
  const float pos = h * inv;
  const float neg = ((h * E) * inv) * kTwoM64;
  return z >= 0.0f ? pos : neg;
}

// g gelu'(h) = g s (1 + h (1 - s) dz/dh)      (s (1 - s) = e inv^2)
__device__ __forceinline__ float gelu_tanh_grad_f32(float h, float g) {
#pragma clang fp contract(off)
  const float z = h * __builtin_fmaf(kGeluC2A, h * h, kGeluC2);
  const float E = __builtin_amdgcn_exp2f(__builtin_fmaf(-__builtin_fabsf(z), kLog2e, 64.0f));
  const float e = E * kTwoM64;
  const float inv = __builtin_amdgcn_rcpf(__builtin_fmaf(E, kTwoM64, 1.0f));
  const float hc = __builtin_amdgcn_fmed3f(h, -16.0f, 16.0f);
  const float dz = __builtin_fmaf(kGeluC6A, hc * hc, kGeluC2);
  // z >= 0: s = inv, 1 - s = e inv
  const float pos = (g * inv) * __builtin_fmaf(hc * (e * inv), dz, 1.0f);
  // z < 0: s = e inv, 1 - s = inv
  const float neg = (((g * E) * inv) * __builtin_fmaf(hc * inv, dz, 1.0f)) * kTwoM64;
  return z >= 0.0f ? pos : neg;
}

// Activation modes of a bf16 input stream (FT_ACT_* of the C ABI):
// ACT 0: x as is; ACT 1: gelu(x); ACT 2: x * gelu'(h) with h a second stream.
// Applied to two packed bf16, rounded to bf16 (nearest even).
// Two fp32 to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2 x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

template <int ACT>
__device__ __forceinline__ uint32_t act_bf16x2(uint32_t x, uint32_t h) {
  if constexpr (ACT == 1) {
    return cvt_pk_bf16(gelu_tanh_f32(bf16lo_to_f32(x)), gelu_tanh_f32(bf16hi_to_f32(x)));
  } else if constexpr (ACT == 2) {
    return cvt_pk_bf16(gelu_tanh_grad_f32(bf16lo_to_f32(h), bf16lo_to_f32(x)),
                       gelu_tanh_grad_f32(bf16hi_to_f32(h), bf16hi_to_f32(x)));
  } else {
    (void)h;
    return x;
  }
}
template <int ACT>
__device__ __forceinline__ u32x4 act_bf16x8(u32x4 x, u32x4 h) {
  if constexpr (ACT == 0) {
    (void)h;
    return x;
  } else {
    return u32x4{act_bf16x2<ACT>(x[0], h[0]), act_bf16x2<ACT>(x[1], h[1]),
                 act_bf16x2<ACT>(x[2], h[2]), act_bf16x2<ACT>(x[3], h[3])};
  }
}

// Buffer resource for raw buffer loads: offsets at or past `bytes` read as 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes > 0x7FFFFFFFu ? 0x7FFFFFFFu : bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 buf_load128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// The same with the non-temporal (streaming) cache policy, for data read once.
__device__ __forceinline__ u32x4 buf_load128_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ uint32_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
constexpr uint32_t BUF_OOB = 0x80000000u;   // a buffer offset past every tensor
// Raw buffer stores: offsets at or past the buffer size are dropped.  They
// let edge masking be an offset instead of a branch, so every store is issued
// unconditionally and the compiler can count outstanding memory operations
// exactly (a store under a branch makes later waits conservative).
__device__ __forceinline__ void buf_store32(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(v), r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store128(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}


}  // namespace ft
