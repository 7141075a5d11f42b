// Adapter (LoRA) weight gradients.
//
// FourTune (arXiv 2607.05711), "3.2 4-Bit Backward Pass via
// Block-Quantization": weight gradients are computed for the adapter only,
//   dL/dB = (X A)^T G,    dL/dA = X^T (G B^T),
// with X and G unquantized.  Here (X A) is the adapter part of the saved
// down-projection U = bf16(X [L1|A]) and (G B^T) the adapter part of
// P = bf16(G [L2;B]^T), so both gradients have the form
//   out(i, r) = sum_m big[m][i] * small[m][r0 + r]
// with big = X (dA) or dY (dB) and small = P or U.
//
// The reduction runs over tokens m, which is the row index of both
// operands, so each 64-row step is staged in LDS transposed (token index
// contiguous) and consumed by 16x16x32 bf16 MFMAs with fp32 accumulation.
// Workgroups split the tokens into chunks; the last workgroup to finish
// a column block adds the chunk partials in chunk order (deterministic)
// and writes the result.  HBM bound: each element of big is read once.
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

namespace {

constexpr int IB = 64;      // columns of big per workgroup
constexpr int MS = 64;      // tokens per LDS step
constexpr int MC = 512;     // tokens per workgroup
constexpr int PM = MS + 8;  // LDS pitch (bf16) of the transposed tiles

template <int RG>
__global__ __launch_bounds__(256) void k_lora_grad(const LoraGradArgs a) {
  constexpr int RP = RG * 16;
  __shared__ __attribute__((aligned(16))) uint16_t bigT[IB * PM];
  __shared__ __attribute__((aligned(16))) uint16_t smT[RP * PM];
  __shared__ int s_last;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t M = a.M, I = a.I;
  const int64_t i0 = static_cast<int64_t>(blockIdx.x) * IB;
  const int64_t mbeg = static_cast<int64_t>(blockIdx.y) * MC;
  const int64_t mend = min(M, mbeg + MC);

  f32x4 acc[RG];
#pragma unroll
  for (int c = 0; c < RG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int64_t ms = mbeg; ms < mend; ms += MS) {
    __syncthreads();
    {
      // thread t: row pair p = t/8 (rows ms+2p, ms+2p+1), columns 8*(t%8) .. +8
      const int p = t >> 3, cc = (t & 7) * 8;
      const int64_t ma = ms + 2 * p, mb = ma + 1, col = i0 + cc;
      u32x4 va = {0, 0, 0, 0}, vb = {0, 0, 0, 0};
      if (col < I) {
        if (ma < mend) va = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.big + ma * I + col));
        if (mb < mend) vb = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.big + mb * I + col));
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (va[j] & 0xFFFFu) | (vb[j] << 16);           // column cc+2j
        const uint32_t hi = (va[j] >> 16) | (vb[j] & 0xFFFF0000u);       // column cc+2j+1
        *reinterpret_cast<uint32_t*>(&bigT[(cc + 2 * j) * PM + 2 * p]) = lo;
        *reinterpret_cast<uint32_t*>(&bigT[(cc + 2 * j + 1) * PM + 2 * p]) = hi;
      }
    }
    for (int idx = t; idx < MS * RP; idx += 256) {
      const int mm = idx / RP, r = idx % RP;
      const int64_t m = ms + mm;
      uint16_t v = 0;
      if (m < mend && r < a.rl) v = a.small[m * a.ld_small + a.r0 + r];
      smT[r * PM + mm] = v;
    }
    __syncthreads();
    // wave w owns columns 16w .. 16w+15 of the block; lane (row l16, group g)
    // covers tokens 8g .. 8g+7 of each 32-token half.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 af = *reinterpret_cast<const u32x4*>(&bigT[(16 * wave + l16) * PM + 32 * h + 8 * g]);
#pragma unroll
      for (int c = 0; c < RG; ++c) {
        const u32x4 bf = *reinterpret_cast<const u32x4*>(&smT[(16 * c + l16) * PM + 32 * h + 8 * g]);
        acc[c] = mfma_bf16_16x16x32(af, bf, acc[c]);
      }
    }
  }

  // acc[c][j]: column i = i0 + 16*wave + 4*g + j, rank r = 16*c + l16
  float* mypart = a.part + static_cast<int64_t>(blockIdx.y) * I * RP;
#pragma unroll
  for (int c = 0; c < RG; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t i = i0 + 16 * wave + 4 * g + j;
      if (i < I) mypart[i * RP + 16 * c + l16] = acc[c][j];
    }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t old = atomicAdd(&a.cnt[blockIdx.x], 1u);
    s_last = (old == gridDim.y - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  for (int idx = t; idx < IB * RP; idx += 256) {
    const int64_t i = i0 + idx / RP;
    const int r = idx % RP;
    if (i >= I || r >= a.rl) continue;
    float s = 0.f;
    for (uint32_t y = 0; y < gridDim.y; ++y)
      s += __hip_atomic_load(a.part + (static_cast<int64_t>(y) * I + i) * RP + r, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    const int64_t o = a.transpose_out ? static_cast<int64_t>(r) * I + i : i * a.rl + r;
    if (a.out_f32)
      static_cast<float*>(a.out)[o] = s;
    else
      static_cast<uint16_t*>(a.out)[o] = f32_to_bf16_rne(s);
  }
  if (t == 0) a.cnt[blockIdx.x] = 0;
}

__global__ void k_zero_u32(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

}  // namespace

size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl) {
  const int64_t nmc = (M + MC - 1) / MC;
  const int RP = ((rl + 15) / 16) * 16;
  return static_cast<size_t>(nmc) * I * RP * sizeof(float);
}

size_t lora_grad_cnt_bytes(int64_t I) { return static_cast<size_t>((I + IB - 1) / IB) * 4; }

hipError_t launch_lora_grad(const LoraGradArgs& a, hipStream_t st) {
  const uint32_t nib = static_cast<uint32_t>((a.I + IB - 1) / IB);
  const uint32_t nmc = static_cast<uint32_t>((a.M + MC - 1) / MC);
  hipLaunchKernelGGL(k_zero_u32, dim3((nib + 255) / 256), dim3(256), 0, st, a.cnt, nib);
  dim3 grid(nib, nmc);
#define FT_L(RG) hipLaunchKernelGGL(k_lora_grad<RG>, grid, dim3(256), 0, st, a)
  switch ((a.rl + 15) / 16) {
    case 1: FT_L(1); break;
    case 2: FT_L(2); break;
    case 3: FT_L(3); break;
    default: FT_L(4); break;
  }
#undef FT_L
  return hipGetLastError();
}

}  // namespace ft
