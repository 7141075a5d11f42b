// Adapter (LoRA) weight gradients.
//
// FourTune (arXiv 2607.05711), "3.2 4-Bit Backward Pass via
// Block-Quantization": weight gradients are computed for the adapter only,
//   dL/dB = (X A)^T G,    dL/dA = X^T (G B^T),
// with X and G unquantized.  Here (X A) is the adapter part of the saved
// down-projection U = bf16(X [L1|A]) and (G B^T) the adapter part of
// P = bf16(G [L2;B]^T).  Both gradients have the form
//   out[r][i] = sum_m small[m][r0 + r] * big[m][i]
// with big = X (dA) or dY (dB) and small = P or U, stored like the factors,
// rank-major (dA^T [r, K] and dB [r, N]).  One launch computes both: the
// first workgroup columns cover dA, the rest dB.
//
// 16x16x32 bf16 MFMAs with A = small^T (ranks x tokens) and B = big (tokens
// x columns), fp32 accumulation.  The reduction runs over tokens, the row
// index of both operands in memory, so both are staged in LDS row-major as
// loaded (16-byte stores, no transposition) and the operands are read with
// ds_read_b64_tr_b16, which hands each lane four consecutive tokens of its
// column.  The MFMA's 32 reduction slots of lane group g take tokens
// 4g .. 4g+3 and 16+4g .. 16+4g+3 of a 32-token half step, the same for both
// operands, which keeps each read conflict-free (8 rows per half wave,
// pitches chosen so 8 consecutive rows start in distinct 8-bank groups).
// A workgroup covers 64 columns x 512 tokens; all of its global loads go out
// up front.  Each 512-token chunk writes fp32 partials; k_lora_reduce, the
// next kernel on the stream, adds them in chunk order (deterministic) and
// rounds once.  HBM bound: big is read once.
//
// Around a GELU ("3.3 ... MLP Fusion"): the second linear of an MLP takes
// gelu(h) as its input, so its dA recomputes gelu on the saved h as big is
// loaded; the first linear's incoming gradient is dY * gelu'(h), which its
// dB recomputes from dY and h the same way.
#include "ft_device.hpp"
#include "ft_kernels.h"
#include "lora_block.hpp"

namespace ft {

namespace {

using lora_dev::IB;
using lora_dev::MC;
using lora_dev::MS;
using lora_dev::PB;
using lora_dev::lora_block;
using lora_dev::lora_reduce_quad;
using lora_dev::small_pitch;

template <int RG, int ACTA, int ACTB>
__global__ __launch_bounds__(256) void k_lora_grads(const LoraGradArgs pa, const LoraGradArgs pb,
                                                    uint32_t nib_a) {
  __shared__ __attribute__((aligned(16))) uint16_t bigL[2][MS * PB];
  __shared__ __attribute__((aligned(16))) uint16_t smL[MC * small_pitch<RG>()];
  if (blockIdx.x < nib_a) lora_block<RG, ACTA>(pa, blockIdx.x, blockIdx.y, bigL, smL);
  else lora_block<RG, ACTB>(pb, blockIdx.x - nib_a, blockIdx.y, bigL, smL);
}

// out[r][i .. i+3] = sum over chunks y < nchunk (in order) of part[y][r][i .. i+3];
// consecutive threads take consecutive column quads of a rank row.  Blocks
// [0, nblk_a) serve dA.
template <int RG>
__global__ __launch_bounds__(256) void k_lora_reduce(const LoraGradArgs pa, const LoraGradArgs pb,
                                                     uint32_t nblk_a) {
  const bool is_a = blockIdx.x < nblk_a;
  const LoraGradArgs& a = is_a ? pa : pb;
  const uint64_t idx = static_cast<uint64_t>(is_a ? blockIdx.x : blockIdx.x - nblk_a) * 256 + threadIdx.x;
  if (idx >= static_cast<uint64_t>(a.rl) * (a.I / 4)) return;
  lora_reduce_quad(a, RG * 16, idx);
}

}  // namespace

size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl) {
  const int64_t nmc = (M + MC - 1) / MC;
  const int RP = ((rl < 64 ? rl : 64) + 15) / 16 * 16;     // ranks of one pass
  return static_cast<size_t>(nmc) * I * RP * sizeof(float);
}

uint32_t lora_chunks(int64_t M) { return static_cast<uint32_t>((M + MC - 1) / MC); }
uint32_t lora_col_blocks(int64_t I) { return static_cast<uint32_t>((I + IB - 1) / IB); }

// The sums of a pass: dA's partials (dA.nchunk chunks), then dB's.
static hipError_t reduce_pass(const LoraGradArgs& dA, const LoraGradArgs& dB, int rg,
                              hipStream_t st) {
  // rl * I / 4 threads per problem
  const uint32_t nblk_a = static_cast<uint32_t>((dA.rl * (dA.I / 4) + 255) / 256);
  const uint32_t nblk_b = static_cast<uint32_t>((dB.rl * (dB.I / 4) + 255) / 256);
#define FT_LR(RG) \
  hipLaunchKernelGGL(k_lora_reduce<RG>, dim3(nblk_a + nblk_b), dim3(256), 0, st, dA, dB, nblk_a)
  switch (rg) {
    case 1: FT_LR(1); break;
    case 2: FT_LR(2); break;
    case 3: FT_LR(3); break;
    default: FT_LR(4); break;
  }
#undef FT_LR
  return hipGetLastError();
}

// One pass over at most 64 ranks (4 groups of 16: the rank operand of a
// 512-token chunk fills most of the LDS at 64).
static hipError_t lora_grads_pass(const LoraGradArgs& dA_in, const LoraGradArgs& dB_in, bool dB_done,
                                  hipStream_t st) {
  LoraGradArgs dA = dA_in, dB = dB_in;
  const uint32_t nib_a = static_cast<uint32_t>((dA.I + IB - 1) / IB);
  const uint32_t nib_b = dB_done ? 0u : static_cast<uint32_t>((dB.I + IB - 1) / IB);
  const uint32_t nmc = static_cast<uint32_t>((dA.M + MC - 1) / MC);
  dA.nchunk = static_cast<int>(nmc);
  if (!dB_done) dB.nchunk = static_cast<int>(nmc);
  dim3 grid(nib_a + nib_b, nmc);
  const int rg = (dA.rl + 15) / 16;
#define FT_LA(RG, A, B) hipLaunchKernelGGL((k_lora_grads<RG, A, B>), grid, dim3(256), 0, st, dA, dB, nib_a)
#define FT_L(RG)                                                                              \
  do {                                                                                        \
    if (dA.act == 1) { if (dB.act == 2) FT_LA(RG, 1, 2); else FT_LA(RG, 1, 0); }              \
    else { if (dB.act == 2) FT_LA(RG, 0, 2); else FT_LA(RG, 0, 0); }                          \
  } while (0)
  switch (rg) {
    case 1: FT_L(1); break;
    case 2: FT_L(2); break;
    case 3: FT_L(3); break;
    default: FT_L(4); break;
  }
#undef FT_L
#undef FT_LA
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  return reduce_pass(dA, dB, rg, st);
}

hipError_t launch_lora_grads(const LoraGradArgs& dA, const LoraGradArgs& dB, bool dB_done,
                             hipStream_t st) {
  if (dA.rl <= 64) return lora_grads_pass(dA, dB, dB_done, st);
  // more than 64 ranks (never with dB_done: the quantizer fuses dB only up
  // to 64): ranks 0 .. 63, then the rest, one after the other on the stream,
  // so the second pass reuses the partial buffers
  if (dB_done) return hipErrorInvalidValue;
  const size_t es = dA.out_f32 ? 4 : 2;
  LoraGradArgs a0 = dA, b0 = dB, a1 = dA, b1 = dB;
  a0.rl = b0.rl = 64;
  a1.rl = b1.rl = dA.rl - 64;
  a1.r0 += 64;
  b1.r0 += 64;
  a1.out = static_cast<char*>(dA.out) + 64 * dA.I * es;
  b1.out = static_cast<char*>(dB.out) + 64 * dB.I * (dB.out_f32 ? 4 : 2);
  if (hipError_t e = lora_grads_pass(a0, b0, false, st); e != hipSuccess) return e;
  return lora_grads_pass(a1, b1, false, st);
}

}  // namespace ft
