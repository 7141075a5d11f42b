// Adapter (LoRA) weight gradients.
//
// FourTune (arXiv 2607.05711), "3.2 4-Bit Backward Pass via
// Block-Quantization": weight gradients are computed for the adapter only,
//   dL/dB = (X A)^T G,    dL/dA = X^T (G B^T),
// with X and G unquantized.  Here (X A) is the adapter part of the saved
// down-projection U = bf16(X [L1|A]) and (G B^T) the adapter part of
// P = bf16(G [L2;B]^T).  Both gradients have the form
//   g(i, r) = sum_m big[m][i] * small[m][r0 + r]
// with big = X (dA) or dY (dB) and small = P or U, and are stored like the
// factors, rank-major: out[r][i] (dA^T [r, K] and dB [r, N]).  One launch computes
// both: the first workgroup columns cover dA, the rest dB.
//
// The reduction runs over tokens m, which is the row index of both
// operands, so each 64-token step of big is written to LDS transposed
// (token index contiguous) and consumed by 16x16x32 bf16 MFMAs with fp32
// accumulation; the small operand of the workgroup's 512 tokens is staged
// transposed once.  All global loads of a workgroup are issued up front.
// Each 512-token chunk writes fp32 partials; k_lora_reduce, the next kernel
// on the stream, adds them in chunk order (deterministic) and rounds once.
// HBM bound: big is read once.
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
constexpr int MS = 64;      // tokens per LDS step
constexpr int NSTEP = 8;    // steps per workgroup
constexpr int MC = MS * NSTEP;
constexpr int PM = MS + 8;  // LDS pitch (bf16) of a transposed big step
constexpr int PS = MC + 8;  // LDS pitch (bf16) of the transposed small operand

// One workgroup: 64 columns of big (column block cb) x 512 tokens.  ACT is
// the activation applied to big as it is loaded (rounded to bf16).
template <int RG, int ACT>
__device__ __forceinline__ void lora_block(const LoraGradArgs& a, uint32_t cb, uint16_t (*bigT)[IB * PM],
                                           uint16_t* smT) {
  constexpr int RP = RG * 16;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = a.M, I = a.I;
  const int64_t i0 = static_cast<int64_t>(cb) * IB;
  const int64_t mbeg = static_cast<int64_t>(blockIdx.y) * MC;
  const int64_t mend = M < mbeg + MC ? M : mbeg + MC;

  // ---- issue the big loads of every step: thread t covers row pair p = t/8
  // (tokens 2p, 2p+1 of the step) and columns 8*(t%8) .. +8
  const auto rbig = make_rsrc(a.big, static_cast<uint64_t>(M) * I * 2);
  const auto rbig2 = make_rsrc(a.big2, ACT == 2 ? static_cast<uint64_t>(M) * I * 2 : 0);
  const int pp = t >> 3, cc = (t & 7) * 8;
  const bool col_ok = i0 + cc < I;
  u32x4 va[NSTEP], vb[NSTEP], ha[NSTEP], hb[NSTEP];
#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    const int64_t ma = mbeg + s * MS + 2 * pp, mb = ma + 1;
    const uint32_t oa = col_ok && ma < mend ? static_cast<uint32_t>((ma * I + i0 + cc) * 2) : BUF_OOB;
    const uint32_t ob = col_ok && mb < mend ? static_cast<uint32_t>((mb * I + i0 + cc) * 2) : BUF_OOB;
    va[s] = buf_load128(rbig, oa);
    vb[s] = buf_load128(rbig, ob);
    if constexpr (ACT == 2) {
      ha[s] = buf_load128(rbig2, oa);
      hb[s] = buf_load128(rbig2, ob);
    }
  }

  // ---- stage small[m][r0 + r] of the chunk transposed: smT[r][m - mbeg]
  const int rl = a.rl;
  if ((a.r0 & 7) == 0 && (a.ld_small & 7) == 0 && (rl & 7) == 0) {
    const auto rs = make_rsrc(a.small, static_cast<uint64_t>(M) * a.ld_small * 2);
    constexpr int PER = MC * RP / 8 / 256;          // 16-byte chunks per thread (upper bound)
    u32x4 w[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;                    // chunk = 8 ranks of token m
      const int m = c % MC, rc = c / MC;
      const int64_t gm = mbeg + m;
      w[e] = buf_load128(rs, (8 * rc < rl && gm < mend)
                                 ? static_cast<uint32_t>((gm * a.ld_small + a.r0 + 8 * rc) * 2) : BUF_OOB);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;
      const int m = c % MC, rc = c / MC;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        smT[(8 * rc + 2 * k) * PS + m] = static_cast<uint16_t>(w[e][k]);
        smT[(8 * rc + 2 * k + 1) * PS + m] = static_cast<uint16_t>(w[e][k] >> 16);
      }
    }
  } else {
    for (int idx = t; idx < MC * RP; idx += 256) {
      const int m = idx % MC, r = idx / MC;
      const int64_t gm = mbeg + m;
      smT[r * PS + m] = (gm < mend && r < rl) ? a.small[gm * a.ld_small + a.r0 + r] : uint16_t(0);
    }
  }

  f32x4 acc[RG];
#pragma unroll
  for (int c = 0; c < RG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < NSTEP; ++s) {
    uint16_t* bt = bigT[s & 1];
    const u32x4 xa = act_bf16x8<ACT>(va[s], ACT == 2 ? ha[s] : va[s]);
    const u32x4 xb = act_bf16x8<ACT>(vb[s], ACT == 2 ? hb[s] : vb[s]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (xa[j] & 0xFFFFu) | (xb[j] << 16);        // column cc+2j
      const uint32_t hi = (xa[j] >> 16) | (xb[j] & 0xFFFF0000u);    // column cc+2j+1
      *reinterpret_cast<uint32_t*>(&bt[(cc + 2 * j) * PM + 2 * pp]) = lo;
      *reinterpret_cast<uint32_t*>(&bt[(cc + 2 * j + 1) * PM + 2 * pp]) = hi;
    }
    __syncthreads();
    // wave w owns columns 16w .. 16w+15 of the block; lane (row l16, group g)
    // covers tokens 8g .. 8g+7 of each 32-token half of the step
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 af = *reinterpret_cast<const u32x4*>(&bt[(16 * wave + l16) * PM + 32 * h + 8 * g]);
#pragma unroll
      for (int c = 0; c < RG; ++c) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(&smT[(16 * c + l16) * PS + s * MS + 32 * h + 8 * g]);
        acc[c] = mfma_bf16_16x16x32(af, bf, acc[c]);
      }
    }
  }

  // acc[c][j]: column i = i0 + 16*wave + 4*g + j, rank r = 16*c + l16;
  // partials part[chunk][i][RP]
  float* mypart = a.part + static_cast<int64_t>(blockIdx.y) * I * RP;
#pragma unroll
  for (int c = 0; c < RG; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + 16 * wave + 4 * g + j;
      if (i < I) mypart[i * RP + 16 * c + l16] = acc[c][j];
    }
}

template <int RG, int ACTA, int ACTB>
__global__ __launch_bounds__(256) void k_lora_grads(const LoraGradArgs pa, const LoraGradArgs pb,
                                                    uint32_t nib_a) {
  constexpr int RP = RG * 16;
  __shared__ __attribute__((aligned(16))) uint16_t bigT[2][IB * PM];
  __shared__ __attribute__((aligned(16))) uint16_t smT[RP * PS];
  if (blockIdx.x < nib_a) lora_block<RG, ACTA>(pa, blockIdx.x, bigT, smT);
  else lora_block<RG, ACTB>(pb, blockIdx.x - nib_a, bigT, smT);
}

// out[r][i] = sum over chunks y (in order) of part[y][i][r]; a thread owns
// column i and 4 consecutive ranks, so consecutive threads store
// consecutive columns of a rank row.  Blocks [0, nblk_a) serve dA.
template <int RG>
__global__ __launch_bounds__(256) void k_lora_reduce(const LoraGradArgs pa, const LoraGradArgs pb,
                                                     uint32_t nblk_a, uint32_t nmc) {
  constexpr int RP = RG * 16;
  const bool is_a = blockIdx.x < nblk_a;
  const LoraGradArgs& a = is_a ? pa : pb;
  const uint64_t idx = static_cast<uint64_t>(is_a ? blockIdx.x : blockIdx.x - nblk_a) * 256 + threadIdx.x;
  const int64_t I = a.I;
  if (idx >= static_cast<uint64_t>(I) * (RP / 4)) return;
  const int64_t i = static_cast<int64_t>(idx % static_cast<uint64_t>(I));
  const int r = static_cast<int>(idx / static_cast<uint64_t>(I)) * 4;
  if (r >= a.rl) return;
  const float* p = a.part + i * RP + r;
  const uint64_t stride = static_cast<uint64_t>(I) * RP;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (uint32_t y0 = 0; y0 < nmc; y0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = (y0 + k < nmc) ? *reinterpret_cast<const f32x4*>(p + (y0 + k) * stride)
                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (r + k >= a.rl) break;
    const int64_t o = static_cast<int64_t>(r + k) * I + i;
    if (a.out_f32) static_cast<float*>(a.out)[o] = s[k];
    else static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_rne(s[k]);
  }
}

}  // namespace

size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl) {
  const int64_t nmc = (M + MC - 1) / MC;
  const int RP = ((rl + 15) / 16) * 16;
  return static_cast<size_t>(nmc) * I * RP * sizeof(float);
}

hipError_t launch_lora_grads(const LoraGradArgs& dA, const LoraGradArgs& dB, hipStream_t st) {
  const uint32_t nib_a = static_cast<uint32_t>((dA.I + IB - 1) / IB);
  const uint32_t nib_b = static_cast<uint32_t>((dB.I + IB - 1) / IB);
  const uint32_t nmc = static_cast<uint32_t>((dA.M + MC - 1) / MC);
  dim3 grid(nib_a + nib_b, nmc);
  const int rg = (dA.rl + 15) / 16;
  // reduction: I * RP/4 threads per problem
  const uint32_t nblk_a = static_cast<uint32_t>((dA.I * rg * 4 + 255) / 256);
  const uint32_t nblk_b = static_cast<uint32_t>((dB.I * rg * 4 + 255) / 256);
#define FT_LA(RG, A, B) hipLaunchKernelGGL((k_lora_grads<RG, A, B>), grid, dim3(256), 0, st, dA, dB, nib_a)
#define FT_L(RG)                                                                              \
  do {                                                                                        \
    if (dA.act == 1) { if (dB.act == 2) FT_LA(RG, 1, 2); else FT_LA(RG, 1, 0); }              \
    else { if (dB.act == 2) FT_LA(RG, 0, 2); else FT_LA(RG, 0, 0); }                          \
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;                        \
    hipLaunchKernelGGL(k_lora_reduce<RG>, dim3(nblk_a + nblk_b), dim3(256), 0, st, dA, dB,    \
                       nblk_a, nmc);                                                          \
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

}  // namespace ft
