// The work item of the adapter-gradient partials (64 columns of big x 512
// tokens), shared by the adapter-gradient kernel (lora.hip) and the
// products that compute dA on CUs their tiles leave free (gemm_pipe.hpp).
// The method and the MFMA layout are described at the top of lora.hip.
#pragma once

#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {
namespace lora_dev {

constexpr int IB = 64;      // columns of big per workgroup
constexpr int MS = 64;      // tokens per step
constexpr int NSTEP = 8;    // steps per workgroup
constexpr int MC = MS * NSTEP;
constexpr int PB = 80;      // LDS pitch (bf16) of a big row: 40 dwords
// LDS pitch (bf16) of a small row: 8 (2 RG - 1) dwords, an odd multiple of 8
template <int RG> constexpr int small_pitch() { return 16 * (2 * RG - 1); }

// One work item: 64 columns of big (column block cb) x 512 tokens (chunk),
// its MFMA sums set into acc (rank r = 16 c + 4 g + j at acc[c][j], column
// i0 + 16 wave + q).  ACT is the activation applied to big as it is loaded
// (rounded to bf16).  The caller's 256 threads all take part (barriers
// inside; the caller orders the LDS between items).
template <int RG, int ACT>
__device__ __forceinline__ void lora_item_sums(const LoraGradArgs& a, uint32_t cb, uint32_t chunk,
                                               uint16_t (*bigL)[MS * PB], uint16_t* smL,
                                               f32x4 (&acc)[RG]) {
  constexpr int RP = RG * 16;
  constexpr int PS = small_pitch<RG>();
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int64_t M = a.M, I = a.I;
  const int64_t i0 = static_cast<int64_t>(cb) * IB;
  const int64_t mbeg = static_cast<int64_t>(chunk) * MC;
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

}

// One work item's fp32 partials: part[chunk][r][I], rank-major.
template <int RG, int ACT>
__device__ __forceinline__ void lora_block(const LoraGradArgs& a, uint32_t cb, uint32_t chunk,
                                           uint16_t (*bigL)[MS * PB], uint16_t* smL) {
  constexpr int RP = RG * 16;
  f32x4 acc[RG];
  lora_item_sums<RG, ACT>(a, cb, chunk, bigL, smL, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int64_t I = a.I;
  const int64_t i = static_cast<int64_t>(cb) * IB + 16 * wave + q;
  if (i < I) {
    float* mypart = a.part + static_cast<int64_t>(chunk) * RP * I;
#pragma unroll
    for (int c = 0; c < RG; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) mypart[(16 * c + 4 * g + j) * I + i] = acc[c][j];
  }
}

// out[r][i] (r < rl) written from an fp32 sum: bf16 (round to nearest even)
// or fp32, as the reduction kernel writes it.
__device__ __forceinline__ void lora_out1(const LoraGradArgs& a, int64_t o, float v) {
  if (a.out_f32) static_cast<float*>(a.out)[o] = v;
  else static_cast<uint16_t*>(a.out)[o] = static_cast<uint16_t>(cvt_pk_bf16(v, v) & 0xFFFFu);
}

// A whole column block of out over every 512-token chunk, without
// partials: each chunk's sums start from zero and are added to the total
// in chunk order, the order in which the reduction kernel adds the
// partials, so the result is the same bits; rounded once into out.
template <int RG, int ACT>
__device__ __forceinline__ void lora_column_block(const LoraGradArgs& a, uint32_t cb,
                                                  uint16_t (*bigL)[MS * PB], uint16_t* smL) {
  f32x4 tot[RG];
#pragma unroll
  for (int c = 0; c < RG; ++c) tot[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t nmc = static_cast<uint32_t>((a.M + MC - 1) / MC);
  for (uint32_t ch = 0; ch < nmc; ++ch) {
    // the previous chunk's LDS reads are done before this one's stores
    __syncthreads();
    f32x4 acc[RG];
    lora_item_sums<RG, ACT>(a, cb, ch, bigL, smL, acc);
#pragma unroll
    for (int c = 0; c < RG; ++c) tot[c] += acc[c];
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, q = lane & 15;
  const int64_t I = a.I;
  const int64_t i = static_cast<int64_t>(cb) * IB + 16 * wave + q;
  if (i < I) {
#pragma unroll
    for (int c = 0; c < RG; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * c + 4 * g + j;
        if (r < a.rl) lora_out1(a, static_cast<int64_t>(r) * I + i, tot[c][j]);
      }
  }
}

// Quad idx (rank idx / (I/4), columns 4 (idx % (I/4)) .. +3) of out as the
// sum over a.nchunk partials [chunk][RP][I] in chunk order, 16 chunks' loads
// at a time (past the last chunk: zero), rounded once.  idx < rl * I / 4.
__device__ __forceinline__ void lora_reduce_quad(const LoraGradArgs& a, int RP, uint64_t idx) {
  const int64_t I = a.I, I4 = I / 4;
  const int64_t r = static_cast<int64_t>(idx / I4);
  const int64_t i = 4 * static_cast<int64_t>(idx % I4);
  const uint64_t stride = static_cast<uint64_t>(RP) * I;
  const uint32_t nmc = static_cast<uint32_t>(a.nchunk);
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

}  // namespace lora_dev
}  // namespace ft
