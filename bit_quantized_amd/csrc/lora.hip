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

namespace ft {

namespace {

constexpr int IB = 64;      // columns of big per workgroup
constexpr int MS = 64;      // tokens per step
constexpr int NSTEP = 8;    // steps per workgroup
constexpr int MC = MS * NSTEP;
constexpr int PB = 80;      // LDS pitch (bf16) of a big row: 40 dwords
// LDS pitch (bf16) of a small row: 8 (2 RG - 1) dwords, an odd multiple of 8
template <int RG> constexpr int small_pitch() { return 16 * (2 * RG - 1); }

// One workgroup: 64 columns of big (column block cb) x 512 tokens.  ACT is
// the activation applied to big as it is loaded (rounded to bf16).
template <int RG, int ACT>
__device__ __forceinline__ void lora_block(const LoraGradArgs& a, uint32_t cb,
                                           uint16_t (*bigL)[MS * PB], uint16_t* smL) {
  constexpr int RP = RG * 16;
  constexpr int PS = small_pitch<RG>();
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int64_t M = a.M, I = a.I;
  const int64_t i0 = static_cast<int64_t>(cb) * IB;
  const int64_t mbeg = static_cast<int64_t>(blockIdx.y) * MC;
  const int64_t mend = M < mbeg + MC ? M : mbeg + MC;

  // ---- big loads of every step: thread t covers rows t/8 and 32 + t/8 of
  // the step, columns 8 (t % 8) .. +8 (each row's 128 bytes in 8 lanes)
  const auto rbig = make_rsrc(a.big, static_cast<uint64_t>(M) * I * 2);
  const auto rbig2 = make_rsrc(a.big2, ACT == 2 ? static_cast<uint64_t>(M) * I * 2 : 0);
  const int lr = t >> 3, cc = (t & 7) * 8;
  const bool col_ok = i0 + cc < I;
  u32x4 va[NSTEP], vb[NSTEP], ha[NSTEP], hb[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int64_t ma = mbeg + s * MS + lr, mb = ma + 32;
    const uint32_t oa = col_ok && ma < mend ? static_cast<uint32_t>((ma * I + i0 + cc) * 2) : BUF_OOB;
    const uint32_t ob = col_ok && mb < mend ? static_cast<uint32_t>((mb * I + i0 + cc) * 2) : BUF_OOB;
    va[s] = buf_load128(rbig, oa);
    vb[s] = buf_load128(rbig, ob);
    if constexpr (ACT == 2) {
      ha[s] = buf_load128(rbig2, oa);
      hb[s] = buf_load128(rbig2, ob);
    }
  }

  // ---- small[m][r0 + r] of the chunk, row-major: smL[m][r], ranks >= rl zero
  const int rl = a.rl;
  if ((a.r0 & 7) == 0 && (a.ld_small & 7) == 0 && (rl & 7) == 0) {
    const auto rs = make_rsrc(a.small, static_cast<uint64_t>(M) * a.ld_small * 2);
    constexpr int CPR = RP / 8;                      // 16-byte chunks per token
    constexpr int PER = MC * CPR / 256;
    u32x4 w[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;
      const int m = c / CPR, rc = c % CPR;
      const int64_t gm = mbeg + m;
      w[e] = buf_load128(rs, (8 * rc < rl && gm < mend)
                                 ? static_cast<uint32_t>((gm * a.ld_small + a.r0 + 8 * rc) * 2) : BUF_OOB);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;
      *reinterpret_cast<u32x4*>(&smL[(c / CPR) * PS + (c % CPR) * 8]) = w[e];
    }
  } else {
    for (int idx = t; idx < MC * RP; idx += 256) {
      const int m = idx / RP, r = idx % RP;
      const int64_t gm = mbeg + m;
      smL[m * PS + r] = (gm < mend && r < rl) ? a.small[gm * a.ld_small + a.r0 + r] : uint16_t(0);
    }
  }

  f32x4 acc[RG];
#pragma unroll
  for (int c = 0; c < RG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    uint16_t* bl = bigL[s & 1];
    *reinterpret_cast<u32x4*>(&bl[lr * PB + cc]) = act_bf16x8<ACT>(va[s], ACT == 2 ? ha[s] : va[s]);
    *reinterpret_cast<u32x4*>(&bl[(32 + lr) * PB + cc]) = act_bf16x8<ACT>(vb[s], ACT == 2 ? hb[s] : vb[s]);
    __syncthreads();
    // wave w: columns 16w .. 16w+15 of the block; lane q of group g addresses
    // row 4g + q/4 (+16) of the half step, columns c0 + 4 (q % 4)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const uint16_t* bp = bl + (kk * 32 + 4 * g + (q >> 2)) * PB + 16 * wave + 4 * (q & 3);
      const u32x2 b0 = lds_read_tr16(bp), b1 = lds_read_tr16(bp + 16 * PB);
      const u32x4 bf = {b0[0], b0[1], b1[0], b1[1]};
#pragma unroll
      for (int c = 0; c < RG; ++c) {
        const uint16_t* sp = smL + (s * MS + kk * 32 + 4 * g + (q >> 2)) * PS + 16 * c + 4 * (q & 3);
        const u32x2 a0 = lds_read_tr16(sp), a1 = lds_read_tr16(sp + 16 * PS);
        acc[c] = mfma_bf16_16x16x32(u32x4{a0[0], a0[1], a1[0], a1[1]}, bf, acc[c]);
      }
    }
  }

  // acc[c][j]: rank r = 16c + 4g + j, column i = i0 + 16 wave + q;
  // partials part[chunk][r][I], rank-major
  const int64_t i = i0 + 16 * wave + q;
  if (i < I) {
    float* mypart = a.part + static_cast<int64_t>(blockIdx.y) * RP * I;
#pragma unroll
    for (int c = 0; c < RG; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) mypart[(16 * c + 4 * g + j) * I + i] = acc[c][j];
  }
}

template <int RG, int ACTA, int ACTB>
__global__ __launch_bounds__(256) void k_lora_grads(const LoraGradArgs pa, const LoraGradArgs pb,
                                                    uint32_t nib_a) {
  __shared__ __attribute__((aligned(16))) uint16_t bigL[2][MS * PB];
  __shared__ __attribute__((aligned(16))) uint16_t smL[MC * small_pitch<RG>()];
  if (blockIdx.x < nib_a) lora_block<RG, ACTA>(pa, blockIdx.x, bigL, smL);
  else lora_block<RG, ACTB>(pb, blockIdx.x - nib_a, bigL, smL);
}

// out[r][i .. i+3] = sum over chunks y < nchunk (in order) of part[y][r][i .. i+3];
// consecutive threads take consecutive column quads of a rank row.  Blocks
// [0, nblk_a) serve dA.
template <int RG>
__global__ __launch_bounds__(256) void k_lora_reduce(const LoraGradArgs pa, const LoraGradArgs pb,
                                                     uint32_t nblk_a) {
  constexpr int RP = RG * 16;
  const bool is_a = blockIdx.x < nblk_a;
  const LoraGradArgs& a = is_a ? pa : pb;
  const uint64_t idx = static_cast<uint64_t>(is_a ? blockIdx.x : blockIdx.x - nblk_a) * 256 + threadIdx.x;
  const int64_t I = a.I, I4 = I / 4;
  if (idx >= static_cast<uint64_t>(a.rl) * I4) return;
  const int64_t r = static_cast<int64_t>(idx / I4);
  const int64_t i = 4 * static_cast<int64_t>(idx % I4);
  const uint64_t stride = static_cast<uint64_t>(RP) * I;
  const uint32_t nmc = static_cast<uint32_t>(a.nchunk);
  // 16 chunks' loads at once, as buffer loads (past the last chunk: zero),
  // so that a batch costs one memory latency; added in chunk order
  const auto rpart = make_rsrc(a.part, stride * nmc * 4);
  const uint32_t base = static_cast<uint32_t>((r * I + i) * 4);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (uint32_t y0 = 0; y0 < nmc; y0 += 16) {
    f32x4 v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t off = y0 + k < nmc ? base + static_cast<uint32_t>((y0 + k) * stride * 4) : BUF_OOB;
      v[k] = __builtin_bit_cast(f32x4, buf_load128(rpart, off));
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) s += v[k];
  }
  const int64_t o = r * I + i;
  if (a.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = s;
  } else {
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) =
        u32x2{cvt_pk_bf16(s[0], s[1]), cvt_pk_bf16(s[2], s[3])};
  }
}

}  // namespace

size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl) {
  const int64_t nmc = (M + MC - 1) / MC;
  const int RP = ((rl < 64 ? rl : 64) + 15) / 16 * 16;     // ranks of one pass
  return static_cast<size_t>(nmc) * I * RP * sizeof(float);
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
  // reduction: rl * I / 4 threads per problem
  const uint32_t nblk_a = static_cast<uint32_t>((dA.rl * (dA.I / 4) + 255) / 256);
  const uint32_t nblk_b = static_cast<uint32_t>((dB.rl * (dB.I / 4) + 255) / 256);
#define FT_LA(RG, A, B) hipLaunchKernelGGL((k_lora_grads<RG, A, B>), grid, dim3(256), 0, st, dA, dB, nib_a)
#define FT_L(RG)                                                                              \
  do {                                                                                        \
    if (dA.act == 1) { if (dB.act == 2) FT_LA(RG, 1, 2); else FT_LA(RG, 1, 0); }              \
    else { if (dB.act == 2) FT_LA(RG, 0, 2); else FT_LA(RG, 0, 0); }                          \
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;                        \
    hipLaunchKernelGGL(k_lora_reduce<RG>, dim3(nblk_a + nblk_b), dim3(256), 0, st, dA, dB,    \
                       nblk_a);                                                               \
  } while (0)
  switch (rg) {
    case 1: FT_L(1); break;
    case 2: FT_L(2); break;
    case 3: FT_L(3); break;
    default: FT_L(4); break;
  }
#undef FT_L
#undef FT_LA
  return hipGetLastError();
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
