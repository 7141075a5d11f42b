// MXFP4 quantizers for gfx950.
//
// FourTune (arXiv 2607.05711): "2.3 Model Quantization" (Round(W/s) with a
// group scale; MXFP4), "3.1" (Q applied offline to the residual weight and
// dynamically to activations), "3.2" (dynamic Q of the incoming gradient;
// square weight blocks whose scales stay local so the same codes serve the
// transposed product), "3.3 Kernel Fusion / LoRA Fusion" (the quantization
// and every low-rank down-projection share one read of the input).
//
// Kernels
//   k_quant_row32     1x32 blocks along rows                       (HBM bound)
//   k_quant_tile32    32x32 tiles, one scale per tile               (HBM bound)
//   k_quant_row32_t   1x32 blocks of the input and of its transpose,
//                     one read of the input                          (HBM bound)
//   k_quant_down      1x32 blocks along rows fused with the rank-R
//                     down-projection (bf16 MFMA, fp32 accumulation),
//                     split over columns with a deterministic
//                     last-arriving-workgroup reduction             (HBM bound)
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

// ---------------------------------------------------------------------------
// 1x32 row blocks: each lane owns one block (64 B in, 16 B codes, 1 B scale).
__global__ __launch_bounds__(256) void k_quant_row32(const uint16_t* __restrict__ in,
                                                     uint32_t rows, uint32_t cols, int64_t ld,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const uint32_t bpr = cols >> 5;
  const uint64_t nblk = static_cast<uint64_t>(rows) * bpr;
  for (uint64_t b = static_cast<uint64_t>(blockIdx.x) * 256 + threadIdx.x; b < nblk;
       b += static_cast<uint64_t>(gridDim.x) * 256) {
    const uint32_t r = static_cast<uint32_t>(b / bpr);
    const uint32_t cb = static_cast<uint32_t>(b - static_cast<uint64_t>(r) * bpr);
    const u32x4* src = reinterpret_cast<const u32x4*>(in + r * ld + cb * 32);
    u32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(src + i);
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) m = max_u16x2(m, abs_bf16x2(v[i][j]));
    const uint32_t s = e8m0_from_amax_bits(hmax_u16x2(m));
    const float sc = e8m0_to_f32(s);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = encode8(v[i][0], v[i][1], v[i][2], v[i][3], sc);
    *reinterpret_cast<u32x4*>(codes + static_cast<uint64_t>(r) * (cols >> 1) + cb * 16) = o;
    scales[b] = static_cast<uint8_t>(s);
  }
}

// ---------------------------------------------------------------------------
// 32x32 tiles.  A workgroup covers 32 rows x 128 columns (4 tiles); thread
// t reads 16 consecutive elements of row t/8 (columns 16*(t%8) ...).
__global__ __launch_bounds__(256) void k_quant_tile32(const uint16_t* __restrict__ in,
                                                      uint32_t rows, uint32_t cols, int64_t ld,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  __shared__ uint32_t red[4][4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t row = blockIdx.y * 32 + (t >> 3);
  const uint32_t col = blockIdx.x * 128 + (t & 7) * 16;
  const bool ok = col < cols;  // rows is a multiple of 32, so row < rows
  u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
  if (ok) {
    const u32x4* src = reinterpret_cast<const u32x4*>(in + row * ld + col);
    v0 = __builtin_nontemporal_load(src);
    v1 = __builtin_nontemporal_load(src + 1);
  }
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max_u16x2(m, max_u16x2(abs_bf16x2(v0[j]), abs_bf16x2(v1[j])));
  uint32_t a = hmax_u16x2(m);
  // reduce over the 16 lanes of this wave that hold the same tile:
  // lane bit 0 (half of the tile row) and bits 3-5 (row within the wave)
  a = max(a, (uint32_t)__shfl_xor((int)a, 1));
  a = max(a, (uint32_t)__shfl_xor((int)a, 8));
  a = max(a, (uint32_t)__shfl_xor((int)a, 16));
  a = max(a, (uint32_t)__shfl_xor((int)a, 32));
  const int tile = (t & 7) >> 1;
  if ((lane & 0x39) == 0) red[wave][tile] = a;  // lanes 0,2,4,6 of the wave
  __syncthreads();
  a = max(max(red[0][tile], red[1][tile]), max(red[2][tile], red[3][tile]));
  const uint32_t s = e8m0_from_amax_bits(a);
  const float sc = e8m0_to_f32(s);
  if (ok) {
    u32x2 o;
    o[0] = encode8(v0[0], v0[1], v0[2], v0[3], sc);
    o[1] = encode8(v1[0], v1[1], v1[2], v1[3], sc);
    *reinterpret_cast<u32x2*>(codes + static_cast<uint64_t>(row) * (cols >> 1) + (col >> 1)) = o;
    if ((t >> 3) == 0 && (t & 1) == 0)
      scales[static_cast<uint64_t>(blockIdx.y) * (cols >> 5) + (col >> 5)] =
          static_cast<uint8_t>(s);
  }
}

// ---------------------------------------------------------------------------
// Dual output: 1x32 blocks along rows and along columns, from one read.
// A workgroup covers a 64x64 tile.  Row pass: thread t holds 16 elements
// of row t/4.  Column pass (through LDS): thread t holds 16 elements of
// column t/4.
__global__ __launch_bounds__(256) void k_quant_row32_t(const uint16_t* __restrict__ in,
                                                       uint32_t rows, uint32_t cols, int64_t ld,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       uint8_t* __restrict__ codes_t,
                                                       uint8_t* __restrict__ scales_t) {
  constexpr int P = 66;  // LDS row pitch in bf16 (odd number of dwords)
  __shared__ uint16_t tile[64 * P];
  const int t = threadIdx.x;
  const uint32_t r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  {
    const int lr = t >> 2, lc = (t & 3) * 16;
    const uint32_t row = r0 + lr, col = c0 + lc;
    const bool ok = row < rows && col < cols;
    u32x4 v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
    if (ok) {
      const u32x4* src = reinterpret_cast<const u32x4*>(in + row * ld + col);
      v0 = __builtin_nontemporal_load(src);
      v1 = __builtin_nontemporal_load(src + 1);
    }
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max_u16x2(m, max_u16x2(abs_bf16x2(v0[j]), abs_bf16x2(v1[j])));
    uint32_t a = hmax_u16x2(m);
    a = max(a, (uint32_t)__shfl_xor((int)a, 1));
    const uint32_t s = e8m0_from_amax_bits(a);
    const float sc = e8m0_to_f32(s);
    if (ok) {
      u32x2 o;
      o[0] = encode8(v0[0], v0[1], v0[2], v0[3], sc);
      o[1] = encode8(v1[0], v1[1], v1[2], v1[3], sc);
      *reinterpret_cast<u32x2*>(codes + static_cast<uint64_t>(row) * (cols >> 1) + (col >> 1)) = o;
      if ((t & 1) == 0)
        scales[static_cast<uint64_t>(row) * (cols >> 5) + (col >> 5)] = static_cast<uint8_t>(s);
    }
    uint16_t* dst = tile + lr * P + lc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dst[2 * j] = static_cast<uint16_t>(v0[j]);
      dst[2 * j + 1] = static_cast<uint16_t>(v0[j] >> 16);
      dst[8 + 2 * j] = static_cast<uint16_t>(v1[j]);
      dst[8 + 2 * j + 1] = static_cast<uint16_t>(v1[j] >> 16);
    }
  }
  __syncthreads();
  {
    const int lc = t >> 2, lr = (t & 3) * 16;
    const uint32_t col = c0 + lc, row = r0 + lr;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j] = static_cast<uint32_t>(tile[(lr + 2 * j) * P + lc]) |
             (static_cast<uint32_t>(tile[(lr + 2 * j + 1) * P + lc]) << 16);
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = max_u16x2(m, abs_bf16x2(w[j]));
    uint32_t a = hmax_u16x2(m);
    a = max(a, (uint32_t)__shfl_xor((int)a, 1));
    const uint32_t s = e8m0_from_amax_bits(a);
    const float sc = e8m0_to_f32(s);
    if (col < cols && row < rows) {
      u32x2 o;
      o[0] = encode8(w[0], w[1], w[2], w[3], sc);
      o[1] = encode8(w[4], w[5], w[6], w[7], sc);
      *reinterpret_cast<u32x2*>(codes_t + static_cast<uint64_t>(col) * (rows >> 1) + (row >> 1)) =
          o;
      if ((t & 1) == 0)
        scales_t[static_cast<uint64_t>(col) * (rows >> 5) + (row >> 5)] = static_cast<uint8_t>(s);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused 1x32 row quantization + rank-R down-projection.
//
// out_lr[row][r] = bf16( sum_c in[row][c] * proj(c, r) ),  r < R,
// proj(c, r) = r < r0 ? p0[c*s0c + r*s0r] : p1[c*s1c + (r-r0)*s1r].
//
// Workgroup: 4 waves x 16 rows = 64 rows; blockIdx.y selects a column range
// of `kc` columns (multiple of 128).  Per 128-column step a lane owns one
// 1x32 block of its row (row = l%16, block = l/16): it quantizes the block
// and feeds the same 32 values to four 16x16x32 bf16 MFMAs, in the
// reduction order (block, 8-element group, element); the projection slice
// is staged in LDS transposed and read with the same order.
template <int NRG>
__global__ __launch_bounds__(256) void k_quant_down(
    const uint16_t* __restrict__ in, uint32_t rows, uint32_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const uint16_t* __restrict__ p0,
    int64_t s0c, int64_t s0r, int r0, const uint16_t* __restrict__ p1, int64_t s1c, int64_t s1r,
    int R, uint16_t* __restrict__ out_lr, float* __restrict__ part, uint32_t* __restrict__ cnt,
    uint32_t kc) {
  constexpr int RP = NRG * 16;      // padded rank
  constexpr int PT = 128 + 8;       // LDS pitch (bf16) of the staged projection
  __shared__ __attribute__((aligned(16))) uint16_t pt[RP * PT];
  __shared__ int s_last;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int g = lane >> 4, lr = lane & 15;
  const uint32_t m0 = blockIdx.x * 64;
  const uint32_t row = m0 + wave * 16 + lr;
  const uint32_t cbeg = blockIdx.y * kc;
  const uint32_t cend = min(cols, cbeg + kc);
  f32x4 acc[NRG];
#pragma unroll
  for (int c = 0; c < NRG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (uint32_t c0 = cbeg; c0 < cend; c0 += 128) {
    __syncthreads();
    for (int idx = t; idx < RP * 128; idx += 256) {
      const int r = idx >> 7, cc = idx & 127;
      const uint32_t c = c0 + cc;
      uint16_t v = 0;
      if (c < cend && r < R)
        v = r < r0 ? p0[c * s0c + r * s0r] : p1[c * s1c + (r - r0) * s1r];
      pt[r * PT + cc] = v;
    }
    __syncthreads();
    const uint32_t cb = c0 + 32 * g;
    u32x4 v[4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
    if (row < rows && cb < cend) {
      const u32x4* src = reinterpret_cast<const u32x4*>(in + row * ld + cb);
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = __builtin_nontemporal_load(src + i);
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = max_u16x2(m, abs_bf16x2(v[i][j]));
      const uint32_t s = e8m0_from_amax_bits(hmax_u16x2(m));
      const float sc = e8m0_to_f32(s);
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = encode8(v[i][0], v[i][1], v[i][2], v[i][3], sc);
      *reinterpret_cast<u32x4*>(codes + static_cast<uint64_t>(row) * (cols >> 1) + (cb >> 1)) = o;
      scales[static_cast<uint64_t>(row) * (cols >> 5) + (cb >> 5)] = static_cast<uint8_t>(s);
    }
#pragma unroll
    for (int c = 0; c < NRG; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 b = lds_read_b128(&pt[(16 * c + lr) * PT + 32 * g + 8 * i]);
        acc[c] = mfma_bf16_16x16x32(v[i], b, acc[c]);
      }
  }

  // acc[c][j] holds row m0 + 16*wave + 4*g + j, rank index 16*c + lr.
  if (gridDim.y == 1) {
#pragma unroll
    for (int c = 0; c < NRG; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t rr = m0 + wave * 16 + 4 * g + j;
        const int r = 16 * c + lr;
        if (rr < rows && r < R) out_lr[static_cast<uint64_t>(rr) * R + r] = f32_to_bf16_rne(acc[c][j]);
      }
    return;
  }
  float* mypart = part + (static_cast<uint64_t>(blockIdx.y) * rows) * RP;
#pragma unroll
  for (int c = 0; c < NRG; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t rr = m0 + wave * 16 + 4 * g + j;
      if (rr < rows) mypart[static_cast<uint64_t>(rr) * RP + 16 * c + lr] = acc[c][j];
    }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    const uint32_t old = atomicAdd(&cnt[blockIdx.x], 1u);
    s_last = (old == gridDim.y - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // Last workgroup of this row block: sum the column-range partials in
  // range order (independent of arrival order) and round once.
  for (int idx = t; idx < 64 * RP; idx += 256) {
    const uint32_t rr = m0 + idx / RP;
    const int r = idx % RP;
    if (rr >= rows || r >= R) continue;
    float s = 0.f;
    for (uint32_t y = 0; y < gridDim.y; ++y)
      s += __hip_atomic_load(part + (static_cast<uint64_t>(y) * rows + rr) * RP + r,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    out_lr[static_cast<uint64_t>(rr) * R + r] = f32_to_bf16_rne(s);
  }
  if (t == 0) cnt[blockIdx.x] = 0;
}

__global__ void k_fill_u32(uint32_t* p, uint32_t n, uint32_t v) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// host launchers

hipError_t launch_quant_row32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const uint64_t nblk = static_cast<uint64_t>(rows) * (cols / 32);
  uint64_t grid = (nblk + 255) / 256;
  if (grid > 8192) grid = 8192;
  hipLaunchKernelGGL(k_quant_row32, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, in,
                     static_cast<uint32_t>(rows), static_cast<uint32_t>(cols), ld, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_tile32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                               uint8_t* codes, uint8_t* scales, hipStream_t st) {
  dim3 grid(static_cast<uint32_t>((cols + 127) / 128), static_cast<uint32_t>(rows / 32));
  hipLaunchKernelGGL(k_quant_tile32, grid, dim3(256), 0, st, in, static_cast<uint32_t>(rows),
                     static_cast<uint32_t>(cols), ld, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_row32_t(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, hipStream_t st) {
  dim3 grid(static_cast<uint32_t>((cols + 63) / 64), static_cast<uint32_t>((rows + 63) / 64));
  hipLaunchKernelGGL(k_quant_row32_t, grid, dim3(256), 0, st, in, static_cast<uint32_t>(rows),
                     static_cast<uint32_t>(cols), ld, codes, scales, codes_t, scales_t);
  return hipGetLastError();
}

int quant_down_splits(int64_t rows, int64_t cols) {
  const int64_t rb = (rows + 63) / 64;
  const int64_t steps = (cols + 127) / 128;
  int64_t s = 1;
  while (rb * s < 512 && s * 2 <= steps && s < 16) s *= 2;
  return static_cast<int>(s);
}

hipError_t launch_quant_down(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                             uint8_t* codes, uint8_t* scales, const LowRankPieces& pr,
                             uint16_t* out_lr, float* part, uint32_t* cnt, hipStream_t st) {
  const int splits = quant_down_splits(rows, cols);
  const int64_t steps = (cols + 127) / 128;
  const uint32_t kc = static_cast<uint32_t>(((steps + splits - 1) / splits) * 128);
  const uint32_t rb = static_cast<uint32_t>((rows + 63) / 64);
  const uint32_t ny = static_cast<uint32_t>((cols + kc - 1) / kc);
  if (ny > 1) {
    hipLaunchKernelGGL(k_fill_u32, dim3((rb + 255) / 256), dim3(256), 0, st, cnt, rb, 0u);
  }
  dim3 grid(rb, ny);
  const int R = pr.r0 + pr.r1;
#define FT_QD(NRG)                                                                              \
  hipLaunchKernelGGL(k_quant_down<NRG>, grid, dim3(256), 0, st, in, static_cast<uint32_t>(rows), \
                     static_cast<uint32_t>(cols), ld, codes, scales, pr.p0, pr.s0c, pr.s0r,     \
                     pr.r0, pr.p1, pr.s1c, pr.s1r, R, out_lr, part, cnt, kc)
  switch ((R + 15) / 16) {
    case 1: FT_QD(1); break;
    case 2: FT_QD(2); break;
    case 3: FT_QD(3); break;
    default: FT_QD(4); break;
  }
#undef FT_QD
  return hipGetLastError();
}

size_t quant_down_part_bytes(int64_t rows, int64_t cols, int R) {
  const int splits = quant_down_splits(rows, cols);
  if (splits <= 1 || R == 0) return 0;
  const int64_t steps = (cols + 127) / 128;
  const int64_t kc = ((steps + splits - 1) / splits) * 128;
  const int64_t ny = (cols + kc - 1) / kc;
  const int RP = ((R + 15) / 16) * 16;
  return static_cast<size_t>(ny) * rows * RP * sizeof(float);
}

size_t quant_down_cnt_bytes(int64_t rows) { return static_cast<size_t>((rows + 63) / 64) * 4; }

}  // namespace ft
