// MXFP4 GEMMs with the low-rank branches fused into the fp32 epilogue.
//
// FourTune (arXiv 2607.05711):
//   forward, Eq. (2):  Y  = GEMM4(Q(X), Q(R)) + X L_stab + X (A B)
//   dgrad,   Eq. (3):  dX = GEMM4(Q(G), Q(R)^T) + G L_stab^T + G (A B)^T
// "3.2": the square-block weight codes are fetched with their scale whether
// the access is transposed or not, so dX is computed from the same codes
// without dequantizing or requantizing them.  "3.3 Kernel Fusion / LoRA
// Fusion": the 4-bit product and the up-projections are accumulated
// together and the output is written once.
//
// With W_res stored [N, K] (rows = output features):
//   FWD  : out[m][n] = sum_k deq(QX)[m][k] deq(QW)[n][k] + sum_r U[m][r] V[r][n]
//   DGRAD: out[m][k] = sum_n deq(QG)[m][n] deq(QW)[n][k] + sum_r P[m][r] D[k][r]
//
// Tiling for gfx950: a 256-thread workgroup computes a 256x256 output tile;
// each of its 4 waves owns 128x128 = 4x4 tiles of the 32x32x64 scaled
// MXFP4 MFMA (fp32 accumulators, 16 per lane per tile).  Reduction steps
// of 128 elements (64 code bytes per row) are double-buffered in LDS.
//   A operand (QX / QG): rows of packed codes, 16 bytes per lane, read with
//     ds_read_b128 from a 16-byte-chunk XOR swizzle.
//   B operand, FWD: rows of QW (n), same as A.
//   B operand, DGRAD: the QW tile is kept row-major (rows n = reduction) in
//     LDS with an 8-byte-chunk XOR swizzle and read with ds_read_b64_tr_b4,
//     whose 16x16 nibble transpose hands each lane 32 codes down a column.
//   Scales: one E8M0 byte per 32-block; a lane passes the word holding the
//     bytes of its row and the step's four blocks and selects the byte with
//     op_sel.  The weight's 32x32 tile scale is the same byte in both
//     directions.
// The epilogue stages the rank-R factors in the freed LDS and accumulates
// them with 32x32x16 bf16 MFMAs into the same fp32 accumulators, then
// rounds to bf16 once.
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;  // BK in 4-bit elements
constexpr int ROWB = BK / 2;                 // 64 bytes of codes per row and step

__device__ __forceinline__ uint32_t swz16(uint32_t row) { return (row >> 1) & 3; }

__device__ __forceinline__ uint16_t lowrank_at(const LowRankPieces& p, int64_t c, int r) {
  return r < p.r0 ? p.p0[c * p.s0c + r * p.s0r] : p.p1[c * p.s1c + (r - p.r0) * p.s1r];
}

template <bool DGRAD, int NRQ>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * BM * ROWB];  // 32 KB
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * BN * ROWB];  // 32 KB

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * BM;
  const int64_t j0 = static_cast<int64_t>(blockIdx.x) * BN;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;
  const int64_t a_row_bytes = RED >> 1, a_row_scales = RED >> 5;
  const int64_t w_row_bytes = g.w_cols >> 1, w_row_scales = g.w_cols >> 5;
  const bool sc_aligned = (RED & 127) == 0;
  const int nks = static_cast<int>((RED + BK - 1) / BK);

  // -------- global -> register staging
  u32x4 ra[4], rb[4];
  uint32_t sa_n[4], sb_n[4];

  auto load_step = [&](int ks) {
    const int64_t k0 = static_cast<int64_t>(ks) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 2) + 64 * i, ch = t & 3;
      const int64_t m = m0 + row;
      u32x4 v = {0, 0, 0, 0};
      if (m < M && k0 + ch * 32 < RED)
        v = *reinterpret_cast<const u32x4*>(g.a_codes + m * a_row_bytes + (k0 >> 1) + ch * 16);
      ra[i] = v;
    }
    if (!DGRAD) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (t >> 2) + 64 * i, ch = t & 3;
        const int64_t n = j0 + row;
        u32x4 v = {0, 0, 0, 0};
        if (n < NOUT && k0 + ch * 32 < RED)
          v = *reinterpret_cast<const u32x4*>(g.w_codes + n * w_row_bytes + (k0 >> 1) + ch * 16);
        rb[i] = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (t >> 3) + 32 * i, ch = t & 7;
        const int64_t n = k0 + row;                 // reduction index
        const int64_t kc = j0 + ch * 32;            // first output column of the chunk
        u32x4 v = {0, 0, 0, 0};
        if (n < RED && kc < NOUT)
          v = *reinterpret_cast<const u32x4*>(g.w_codes + n * w_row_bytes + (j0 >> 1) + ch * 16);
        rb[i] = v;
      }
    }
    // scales of the A rows this lane feeds to the MFMAs
    const int64_t kb0 = k0 >> 5;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t m = m0 + wm * 128 + mt * 32 + l32;
      uint32_t w = 0x7F7F7F7Fu;
      if (m < M) {
        const uint8_t* p = g.a_scales + m * a_row_scales + kb0;
        if (sc_aligned) {
          w = *reinterpret_cast<const uint32_t*>(p);
        } else {
          w = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w |= static_cast<uint32_t>(kb0 + j < a_row_scales ? p[j] : 0x7F) << (8 * j);
        }
      }
      sa_n[mt] = w >> (8 * grp);
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (!DGRAD) {
        const int64_t nb = (j0 + wn * 128 + nt * 32) >> 5;
        uint32_t w = 0x7F7F7F7Fu;
        if (nb < (NOUT >> 5)) {
          const uint8_t* p = g.w_scales + nb * w_row_scales + kb0;
          if (sc_aligned) {
            w = *reinterpret_cast<const uint32_t*>(p);
          } else {
            w = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              w |= static_cast<uint32_t>(kb0 + j < w_row_scales ? p[j] : 0x7F) << (8 * j);
          }
        }
        sb_n[nt] = w >> (8 * grp);
      } else {
        const int64_t kcol = (j0 + wn * 128 + nt * 32) >> 5;
        uint32_t w = 0;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int64_t nb = kb0 + 2 * c + grp;
          uint32_t b = 0x7F;
          if (nb < (RED >> 5) && kcol < w_row_scales) b = g.w_scales[nb * w_row_scales + kcol];
          w |= b << (16 * c);
        }
        sb_n[nt] = w;
      }
    }
  };

  auto store_step = [&](int buf) {
    uint8_t* la = lds_a + buf * (BM * ROWB);
    uint8_t* lb = lds_b + buf * (BN * ROWB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 2) + 64 * i, ch = t & 3;
      *reinterpret_cast<u32x4*>(la + row * ROWB + ((ch ^ swz16(row)) << 4)) = ra[i];
    }
    if (!DGRAD) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (t >> 2) + 64 * i, ch = t & 3;
        *reinterpret_cast<u32x4*>(lb + row * ROWB + ((ch ^ swz16(row)) << 4)) = rb[i];
      }
    } else {
      // 128 rows x 128 bytes; 8-byte chunk c of row r lives at chunk c ^ (r & 15)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (t >> 3) + 32 * i, ch = t & 7;
        const int s = row & 15;
        const int phys = ch ^ (s >> 1);
        u32x4 v = rb[i];
        if (s & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        *reinterpret_cast<u32x4*>(lb + row * 128 + (phys << 4)) = v;
      }
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint32_t sa[4], sb[4];
  load_step(0);
  store_step(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { sa[i] = sa_n[i]; sb[i] = sb_n[i]; }
  __syncthreads();

  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < nks;
    if (more) load_step(ks + 1);
    const uint8_t* la = lds_a + cur * (BM * ROWB);
    const uint8_t* lb = lds_b + cur * (BN * ROWB);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + l32;
        af[mt] = lds_read_b128(
            (la + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4)));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (!DGRAD) {
          const int row = wn * 128 + nt * 32 + l32;
          bf[nt] = lds_read_b128(
              (lb + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4)));
        } else {
          const int h = lane >> 4, i = lane & 15;
          const int logical = 8 * wn + 2 * nt + (h & 1);
          const int rowb = c * 64 + 32 * (h >> 1) + i;
          const u32x2 lo = lds_read_tr4((
              lb + rowb * 128 + ((logical ^ i) << 3)));
          const u32x2 hi = lds_read_tr4((
              lb + (rowb + 16) * 128 + ((logical ^ i) << 3)));
          bf[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (c == 0)
            acc[mt][nt] = mfma_fp4_32x32x64<0, 0>(af[mt], bf[nt], acc[mt][nt], sa[mt], sb[nt]);
          else
            acc[mt][nt] = mfma_fp4_32x32x64<2, 2>(af[mt], bf[nt], acc[mt][nt], sa[mt], sb[nt]);
        }
    }
    if (more) store_step(cur ^ 1);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) { sa[i] = sa_n[i]; sb[i] = sb_n[i]; }
  }

  // -------- low-rank epilogue: acc += lm[m, :R] . lo[j, :R]^T (bf16 MFMA)
  if constexpr (NRQ > 0) {
    constexpr int RP = NRQ * 16;
    const int R = g.R;
    uint8_t* lm_t = lds_a;   // [256 rows][128 B], 16-byte chunks swizzled by row & 7
    uint8_t* lo_t = lds_b;
    for (int idx = t; idx < BM * RP; idx += 256) {
      const int row = idx / RP, r = idx % RP;
      const int64_t m = m0 + row;
      uint16_t v = 0;
      if (m < M && r < R) v = g.lm[m * R + r];
      *reinterpret_cast<uint16_t*>(lm_t + row * 128 + ((((r >> 3) ^ (row & 7))) << 4) + (r & 7) * 2) = v;
    }
    for (int idx = t; idx < BN * RP; idx += 256) {
      const int row = idx / RP, r = idx % RP;
      const int64_t j = j0 + row;
      uint16_t v = 0;
      if (j < NOUT && r < R) v = lowrank_at(g.lo, j, r);
      *reinterpret_cast<uint16_t*>(lo_t + row * 128 + ((((r >> 3) ^ (row & 7))) << 4) + (r & 7) * 2) = v;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NRQ; ++q) {
      u32x4 ua[4], vb[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + l32;
        ua[mt] = lds_read_b128((
            lm_t + row * 128 + (((2 * q + grp) ^ (row & 7)) << 4)));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = wn * 128 + nt * 32 + l32;
        vb[nt] = lds_read_b128((
            lo_t + row * 128 + (((2 * q + grp) ^ (row & 7)) << 4)));
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_32x32x16(ua[mt], vb[nt], acc[mt][nt]);
    }
  }

  // -------- store: lane holds rows 8*(r/4) + 4*grp + r%4, column l32 of each 32x32 tile
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = j0 + wn * 128 + nt * 32 + l32;
      if (col >= NOUT) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 128 + mt * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
        if (row < M) g.out[row * NOUT + col] = f32_to_bf16_rne(acc[mt][nt][r]);
      }
    }
}

template <bool DGRAD>
hipError_t launch(const GemmArgs& g, hipStream_t st) {
  dim3 grid(static_cast<uint32_t>((g.NOUT + BN - 1) / BN), static_cast<uint32_t>((g.M + BM - 1) / BM));
#define FT_G(NRQ) hipLaunchKernelGGL((k_gemm<DGRAD, NRQ>), grid, dim3(256), 0, st, g)
  switch ((g.R + 15) / 16) {
    case 0: FT_G(0); break;
    case 1: FT_G(1); break;
    case 2: FT_G(2); break;
    case 3: FT_G(3); break;
    default: FT_G(4); break;
  }
#undef FT_G
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fwd(const GemmArgs& g, hipStream_t st) { return launch<false>(g, st); }
hipError_t launch_gemm_dgrad(const GemmArgs& g, hipStream_t st) { return launch<true>(g, st); }

}  // namespace ft
