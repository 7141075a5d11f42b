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
// MXFP4 MFMA (fp32 accumulators in AGPRs, 16 per lane per tile).  Reduction
// steps of 128 elements (64 code bytes per row) are double-buffered in LDS:
// the global loads of step k+1 are in flight while step k runs its 32
// MFMAs per wave, and are written to the other LDS buffer afterwards.
//   A operand (QX / QG): rows of packed codes, 16 bytes per lane, read with
//     ds_read_b128 from a 16-byte-chunk XOR swizzle.
//   B operand, FWD: rows of QW (n), same as A.
//   B operand, DGRAD: the QW tile is kept row-major (rows n = reduction) in
//     LDS with an 8-byte-chunk XOR swizzle and read with ds_read_b64_tr_b4,
//     whose 16x16 nibble transpose hands each lane 32 codes down a column.
//   Scales: one E8M0 byte per 32-block; a lane passes the word holding the
//     bytes of its row and the step's blocks and selects the byte with
//     op_sel.  The weight's 32x32 tile scale is the same byte either way.
//   Global loads are raw buffer loads: addresses past the end of a tensor
//   read as zero, which covers the ragged edges without branches.
//   Workgroups are mapped so that each XCD (own L2) works on a compact
//   block of output tiles.
// The epilogue stages the rank-R factors in the freed LDS and accumulates
// them with 32x32x16 bf16 MFMAs into the same fp32 accumulators, rounds to
// bf16 once and writes the tile through LDS as 16-byte row segments.
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;  // BK in 4-bit elements
constexpr int ROWB = BK / 2;                 // 64 bytes of codes per row and step
constexpr uint32_t OOB = 0x80000000u;        // a buffer offset past every tensor

// 16-byte chunk swizzle of 64-byte rows: the 16 rows one 16-lane group reads
// land in 16 distinct 16-byte bank groups of the 256-byte LDS line.
__device__ __forceinline__ uint32_t swz16(uint32_t row) { return (row >> 2) & 3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0,
                                           (int)(bytes > 0x7FFFFFFFu ? 0x7FFFFFFFu : bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 bload128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Workgroup i of n -> logical tile index, so that the workgroups the
// hardware sends to one XCD (i % 8) get consecutive logical indices.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n) {
  const uint32_t x = i & 7, j = i >> 3, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + j;
}

// Output tile of this workgroup: XCD-contiguous logical index, then groups
// of 4 m-tiles with the n-tiles inner, so that the workgroups one XCD runs at
// the same time share A rows and B columns in its L2.
__device__ __forceinline__ void tile_origin(int64_t M, int64_t NOUT, int64_t& m0, int64_t& j0) {
  const uint32_t mt_n = static_cast<uint32_t>((M + BM - 1) / BM);
  const uint32_t nt_n = static_cast<uint32_t>((NOUT + BN - 1) / BN);
  const uint32_t lid = xcd_remap(blockIdx.x, mt_n * nt_n);
  constexpr uint32_t GM = 4;
  const uint32_t grp_sz = GM * nt_n;
  const uint32_t gidx = lid / grp_sz, gfirst = gidx * GM;
  const uint32_t gm = min(GM, mt_n - gfirst);
  const uint32_t in_g = lid - gidx * grp_sz;
  m0 = static_cast<int64_t>(gfirst + in_g % gm) * BM;
  j0 = static_cast<int64_t>(in_g / gm) * BN;
}

// Low-rank epilogue and store, shared by both GEMM kernels.  lds_a and lds_b
// must each be at least 32 KB of free LDS.
template <int NRQ>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[4][4], uint8_t* lds_a,
                                         uint8_t* lds_b, int64_t m0, int64_t j0) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, NOUT = g.NOUT;
  // -------- low-rank epilogue: acc += lm[m, :R] . lo[j, :R]^T (bf16 MFMA)
  if constexpr (NRQ > 0) {
    constexpr int RP = NRQ * 16;
    const int R = g.R;
    uint8_t* lm_t = lds_a;   // [256 rows][128 B], 16-byte chunks swizzled by row & 7
    uint8_t* lo_t = lds_b;
    auto put = [&](uint8_t* base, int row, int r, uint16_t v) {
      *reinterpret_cast<uint16_t*>(base + row * 128 + (((r >> 3) ^ (row & 7)) << 4) + (r & 7) * 2) = v;
    };
    auto put16 = [&](uint8_t* base, int row, int rc, u32x4 v) {   // 8 ranks 8 rc .. 8 rc + 7
      *reinterpret_cast<u32x4*>(base + row * 128 + ((rc ^ (row & 7)) << 4)) = v;
    };
    const LowRankPieces& p = g.lo;
    const bool col_fast = p.s0c == 1 && p.s1c == 1;     // V[r][j]; rows are N long, N % 32 == 0
    if ((p.r0 & 7) == 0 && (p.r1 & 7) == 0) {
      // 16-byte loads, all issued before the LDS writes.  Tiles of U/P and of
      // the rows of L1/A are contiguous; rows of L2/B give 8 columns a load.
      const int CPR = R >> 3;                          // 16-byte chunks per rank row
      const auto rl_m = rsrc(g.lm, static_cast<uint64_t>(M) * R * 2);
      const auto rp0 = rsrc(p.p0, piece_bytes(p.s0c, p.s0r, p.r0, NOUT));
      const auto rp1 = rsrc(p.p1, piece_bytes(p.s1c, p.s1r, p.r1, NOUT));
      u32x4 vm[NRQ * 2], vo[NRQ * 2];
#pragma unroll
      for (int e = 0; e < NRQ * 2; ++e) {
        const int c = t + 256 * e;                       // chunk index, < 32 R when e < CPR
        vm[e] = u32x4{0, 0, 0, 0};
        vo[e] = u32x4{0, 0, 0, 0};
        if (e < CPR) {
          const int row = c / CPR;
          vm[e] = bload128(rl_m, m0 + row < M ? static_cast<uint32_t>((m0 * R + c * 8) * 2) : OOB);
          if (col_fast) {
            const int r = c >> 5, j = (c & 31) * 8;
            const bool jok = j0 + j < NOUT;
            vo[e] = r < p.r0 ? bload128(rp0, jok ? static_cast<uint32_t>((r * p.s0r + j0 + j) * 2) : OOB)
                             : bload128(rp1, jok ? static_cast<uint32_t>(((r - p.r0) * p.s1r + j0 + j) * 2) : OOB);
          } else {
            const int rc = c % CPR, c0 = p.r0 >> 3;
            const bool jok = j0 + row < NOUT;
            vo[e] = rc < c0 ? bload128(rp0, jok ? static_cast<uint32_t>(((j0 + row) * p.r0 + rc * 8) * 2) : OOB)
                            : bload128(rp1, jok ? static_cast<uint32_t>(((j0 + row) * p.r1 + (rc - c0) * 8) * 2) : OOB);
          }
        }
      }
      // zero the padded rank chunks R .. RP of both tiles
      for (int c = R >> 3; c < RP / 8; ++c) {
        put16(lm_t, t, c, u32x4{0, 0, 0, 0});
        put16(lo_t, t, c, u32x4{0, 0, 0, 0});
      }
#pragma unroll
      for (int e = 0; e < NRQ * 2; ++e) {
        if (e < CPR) {
          const int c = t + 256 * e;
          put16(lm_t, c / CPR, c % CPR, vm[e]);
          if (col_fast) {
            const int r = c >> 5, j = (c & 31) * 8;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              put(lo_t, j + 2 * k, r, static_cast<uint16_t>(vo[e][k]));
              put(lo_t, j + 2 * k + 1, r, static_cast<uint16_t>(vo[e][k] >> 16));
            }
          } else {
            put16(lo_t, c / CPR, c % CPR, vo[e]);
          }
        }
      }
    } else {
      // ranks that are not multiples of 8: element by element
      for (int idx = t; idx < BM * RP; idx += 256) {
        const int row = idx / RP, r = idx % RP;
        const int64_t m = m0 + row;
        put(lm_t, row, r, (m < M && r < R) ? g.lm[m * R + r] : uint16_t(0));
      }
      for (int idx = t; idx < BN * RP; idx += 256) {
        const int row = idx / RP, r = idx % RP;
        const int64_t j = j0 + row;
        uint16_t v = 0;
        if (j < NOUT && r < R)
          v = r < p.r0 ? p.p0[j * p.s0c + r * p.s0r] : p.p1[j * p.s1c + (r - p.r0) * p.s1r];
        put(lo_t, row, r, v);
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NRQ; ++q) {
      u32x4 ua[4], vb[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + l32;
        ua[mt] = lds_read_b128(lm_t + row * 128 + (((2 * q + grp) ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int row = wn * 128 + nt * 32 + l32;
        vb[nt] = lds_read_b128(lo_t + row * 128 + (((2 * q + grp) ^ (row & 7)) << 4));
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_32x32x16(ua[mt], vb[nt], acc[mt][nt]);
    }
  }

  // -------- store through LDS: per 32-row strip, each wave writes its 32x128
  // bf16 block (8 KB) into its own LDS region, then stores 16-byte row segments.
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds_a) + wave * (32 * 128);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 8 * (r >> 2) + 4 * grp + (r & 3);
        const int col = nt * 32 + l32;
        // 16-byte chunk (col / 8) of a 256-byte row, swizzled by row
        const int chunk = (col >> 3) ^ (row & 15);
        stage[row * 128 + chunk * 8 + (col & 7)] = f32_to_bf16_rne(acc[mt][nt][r]);
      }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int idx = s * 64 + lane;          // 32 rows x 16 chunks
      const int row = idx >> 4, c16 = idx & 15;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * 128 + ((c16 ^ (row & 15)) << 3));
      const int64_t grow = m0 + wm * 128 + mt * 32 + row;
      const int64_t gcol = j0 + wn * 128 + c16 * 8;
      if (grow < M && gcol < NOUT)
        *reinterpret_cast<u32x4*>(g.out + grow * NOUT + gcol) = v;
    }
  }
}

template <bool DGRAD, int NRQ, bool SCAL>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2 * BM * ROWB];  // 32 KB
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2 * BN * ROWB];  // 32 KB

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;

  int64_t m0, j0;
  tile_origin(M, NOUT, m0, j0);

  const uint32_t a_row_bytes = static_cast<uint32_t>(RED >> 1);
  const uint32_t a_row_sc = static_cast<uint32_t>(RED >> 5);
  const uint32_t w_row_bytes = static_cast<uint32_t>(g.w_cols >> 1);
  const uint32_t w_row_sc = static_cast<uint32_t>(g.w_cols >> 5);
  const int nks = static_cast<int>((RED + BK - 1) / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * a_row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * a_row_sc);
  const uint64_t wrows = DGRAD ? static_cast<uint64_t>(RED) : static_cast<uint64_t>(NOUT);
  const auto rw_codes = rsrc(g.w_codes, wrows * w_row_bytes);
  const auto rw_sc = rsrc(g.w_scales, (wrows >> 5) * w_row_sc);

  // ---- per-thread load geometry (independent of the step)
  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = (t >> 2) + 64 * i, ch = t & 3;
    a_off[i] = static_cast<uint32_t>(m0 + row) * a_row_bytes + ch * 16;
    if (!DGRAD) {
      b_off[i] = static_cast<uint32_t>(j0 + row) * w_row_bytes + ch * 16;
    } else {
      const uint32_t rrow = (t >> 3) + 32 * i, c8 = t & 7;
      const bool col_ok = j0 + c8 * 32 < NOUT;
      b_off[i] = col_ok ? rrow * w_row_bytes + static_cast<uint32_t>(j0 >> 1) + c8 * 16 : OOB;
    }
  }
  uint32_t sa_off[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
    sa_off[mt] = static_cast<uint32_t>(m0 + wm * 128 + mt * 32 + l32) * a_row_sc;

  // Loaded values are only moved into registers here; combining scale bytes
  // into words happens at the point of use, so nothing waits on these loads
  // until the next step needs them.
  constexpr int SB = SCAL ? 1 : 4;   // scale loads per scale word
  u32x4 ra[4], rb[4];
  uint32_t sa_raw[4][SB], sb_raw[4][DGRAD ? 2 : SB];

  auto issue_loads = [&](int ks) {
    const uint32_t k0 = static_cast<uint32_t>(ks) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ch = t & 3;
      const bool kin = k0 + ch * 32 < RED;
      ra[i] = bload128(ra_codes, kin ? a_off[i] + (k0 >> 1) : OOB);
      if (!DGRAD) rb[i] = bload128(rw_codes, kin ? b_off[i] + (k0 >> 1) : OOB);
      else rb[i] = bload128(rw_codes, b_off[i] == OOB ? OOB : b_off[i] + k0 * w_row_bytes);
    }
    const uint32_t kb0 = k0 >> 5;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (SCAL) {
        sa_raw[mt][0] = bload32(ra_sc, sa_off[mt] + kb0);
      } else {
#pragma unroll
        for (int j = 0; j < SB; ++j)
          sa_raw[mt][j] = bload8(ra_sc, kb0 + j < a_row_sc ? sa_off[mt] + kb0 + j : OOB);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (!DGRAD) {
        const uint32_t nb = static_cast<uint32_t>((j0 + wn * 128 + nt * 32) >> 5);
        if (SCAL) {
          sb_raw[nt][0] = bload32(rw_sc, nb * w_row_sc + kb0);
        } else {
#pragma unroll
          for (int j = 0; j < SB; ++j)
            sb_raw[nt][j] = bload8(rw_sc, kb0 + j < w_row_sc ? nb * w_row_sc + kb0 + j : OOB);
        }
      } else {
        const uint32_t kcol = static_cast<uint32_t>((j0 + wn * 128 + nt * 32) >> 5);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const uint32_t nb = kb0 + 2 * c + grp;
          sb_raw[nt][c] = bload8(rw_sc, kcol < w_row_sc ? nb * w_row_sc + kcol : OOB);
        }
      }
    }
  };

  auto store_lds = [&](int buf) {
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

  uint32_t sa[4][SB], sb[4][DGRAD ? 2 : SB];
  auto take_scales = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < SB; ++j) sa[i][j] = sa_raw[i][j];
#pragma unroll
      for (int j = 0; j < (DGRAD ? 2 : SB); ++j) sb[i][j] = sb_raw[i][j];
    }
  };
  issue_loads(0);
  store_lds(0);
  take_scales();
  __syncthreads();

  // One basic block per step: the loads for step ks+1 are issued first and
  // stay in flight under this step's MFMAs.  On the last step they address
  // step nks, which lies past the reduction dimension, so every one of them
  // is an out-of-range buffer load that returns zero and is never used.
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    issue_loads(ks + 1);
    __builtin_amdgcn_sched_barrier(0);
    // scale words: byte (2c + grp) of a row's step word feeds k-chunk c
    uint32_t as[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t wa = sa[i][0], wb = sb[i][0];
      if (!SCAL) {
        wa = sa[i][0] | (sa[i][1] << 8) | (sa[i][2] << 16) | (sa[i][3] << 24);
        if (!DGRAD) wb = sb[i][0] | (sb[i][1] << 8) | (sb[i][2] << 16) | (sb[i][3] << 24);
      }
      as[i] = wa >> (8 * grp);
      bs[i] = DGRAD ? (sb[i][0] | (sb[i][1] << 16)) : (wb >> (8 * grp));
    }
    const uint8_t* la = lds_a + cur * (BM * ROWB);
    const uint8_t* lb = lds_b + cur * (BN * ROWB);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + l32;
        af[mt] = lds_read_b128(la + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (!DGRAD) {
          const int row = wn * 128 + nt * 32 + l32;
          bf[nt] = lds_read_b128(lb + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
        } else {
          const int h = lane >> 4, i = lane & 15;
          const int logical = 8 * wn + 2 * nt + (h & 1);
          const int rowb = c * 64 + 32 * (h >> 1) + i;
          const u32x2 lo = lds_read_tr4(lb + rowb * 128 + ((logical ^ i) << 3));
          const u32x2 hi = lds_read_tr4(lb + (rowb + 16) * 128 + ((logical ^ i) << 3));
          bf[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (c == 0)
            acc[mt][nt] = mfma_fp4_32x32x64<0, 0>(af[mt], bf[nt], acc[mt][nt], as[mt], bs[nt]);
          else
            acc[mt][nt] = mfma_fp4_32x32x64<2, 2>(af[mt], bf[nt], acc[mt][nt], as[mt], bs[nt]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    store_lds(cur ^ 1);
    __syncthreads();
    take_scales();
  }

  epilogue<NRQ>(g, acc, lds_a, lds_b, m0, j0);
}


// ---------------------------------------------------------------------------
// Pipelined variant for reduction lengths that are a multiple of 128 (every
// step holds whole 4-block scale words).  Operands and scales go from global
// memory straight into LDS with buffer_load ... lds (no registers), into one
// of 4 LDS stages, three steps ahead of the step the MFMAs consume.  Each
// wave waits for its own loads of the current stage with an explicit
// vmcnt and a plain s_barrier then makes every wave's loads visible.
constexpr int NST = 4;                      // LDS stages
constexpr int ST_A = BM * ROWB;             // 16 KB of A codes
constexpr int ST_B = BN * ROWB;             // 16 KB of B codes
constexpr int ST_SA = BM * 4;               // A scale words, one per row
constexpr int ST_SB = 4 * 256;              // B scales, one 256-byte region per wave
constexpr int ST_BYTES = ST_A + ST_B + ST_SA + ST_SB;
constexpr int LOADS_PER_STAGE = 10;         // DMA instructions per thread per stage

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FT_LDS void*)(lds), 16, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FT_LDS void*)(lds), 4, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void dma1(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FT_LDS void*)(lds), 1, (int)off, 0, 0, 0);
}

template <bool DGRAD, int NRQ>
__global__ __launch_bounds__(256, 1) void k_gemm_pipe(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * ST_BYTES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;
  int64_t m0, j0;
  tile_origin(M, NOUT, m0, j0);

  const uint32_t a_row_bytes = static_cast<uint32_t>(RED >> 1);
  const uint32_t a_row_sc = static_cast<uint32_t>(RED >> 5);
  const uint32_t w_row_bytes = static_cast<uint32_t>(g.w_cols >> 1);
  const uint32_t w_row_sc = static_cast<uint32_t>(g.w_cols >> 5);
  const int nks = static_cast<int>(RED / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * a_row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * a_row_sc);
  const uint64_t wrows = DGRAD ? static_cast<uint64_t>(RED) : static_cast<uint64_t>(NOUT);
  const auto rw_codes = rsrc(g.w_codes, wrows * w_row_bytes);
  const auto rw_sc = rsrc(g.w_scales, (wrows >> 5) * w_row_sc);

  // ---- per-lane DMA source offsets at step 0.  Instruction q of wave w
  // fills 1 KB of LDS; lane i lands at byte 16 i of it.
  uint32_t a_src[4], b_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t row = 64 * wave + 16 * q + (lane >> 2), pch = lane & 3;
    a_src[q] = static_cast<uint32_t>(m0 + row) * a_row_bytes + ((pch ^ swz16(row)) << 4);
    if (!DGRAD) {
      b_src[q] = static_cast<uint32_t>(j0 + row) * w_row_bytes + ((pch ^ swz16(row)) << 4);
    } else {
      // B tile: 128 rows (reduction) x 128 bytes; 16-byte chunk c of row r at c ^ ((r>>1)&7)
      const uint32_t brow = 32 * wave + 8 * q + (lane >> 3), bp = lane & 7;
      const uint32_t lc = bp ^ ((brow >> 1) & 7);
      b_src[q] = (j0 + lc * 32 < NOUT)
                     ? brow * w_row_bytes + static_cast<uint32_t>(j0 >> 1) + lc * 16 : OOB;
    }
  }
  const uint32_t sa_src = static_cast<uint32_t>(m0 + 64 * wave + lane) * a_row_sc;
  uint32_t sb_src = OOB;
  if (wave == 0) {
    if (!DGRAD) {
      const uint32_t nb = static_cast<uint32_t>(j0 >> 5) + lane;
      if (lane < 8 && nb < (NOUT >> 5)) sb_src = nb * w_row_sc;
    } else {
      const uint32_t q = lane >> 3, c = lane & 7;
      const uint32_t kcol = static_cast<uint32_t>(j0 >> 5) + c;
      if (lane < 32 && kcol < w_row_sc) sb_src = q * w_row_sc + kcol;
    }
  }

  auto issue_stage = [&](int ks) {
    uint8_t* st = lds + (ks % NST) * ST_BYTES;
    const uint32_t k0 = static_cast<uint32_t>(ks) * BK;
    const bool kin = k0 < RED;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      dma16(ra_codes, st + (64 * wave + 16 * q) * ROWB, kin ? a_src[q] + (k0 >> 1) : OOB);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (!DGRAD)
        dma16(rw_codes, st + ST_A + (64 * wave + 16 * q) * ROWB, kin ? b_src[q] + (k0 >> 1) : OOB);
      else
        dma16(rw_codes, st + ST_A + (32 * wave + 8 * q) * 128,
              (kin && b_src[q] != OOB) ? b_src[q] + k0 * w_row_bytes : OOB);
    }
    dma4(ra_sc, st + ST_A + ST_B + 64 * wave * 4, kin ? sa_src + (k0 >> 5) : OOB);
    const uint32_t sb_off = sb_src == OOB || !kin ? OOB
                            : (DGRAD ? sb_src + (k0 >> 5) * w_row_sc : sb_src + (k0 >> 5));
    if (!DGRAD) dma4(rw_sc, st + ST_A + ST_B + ST_SA + wave * 256, sb_off);
    else dma1(rw_sc, st + ST_A + ST_B + ST_SA + wave * 256, sb_off);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue_stage(s);

  for (int ks = 0; ks < nks; ++ks) {
    // this wave's loads of stage ks are done once at most the loads of the
    // (NST - 2) later stages are outstanding; the barrier covers the others
    __builtin_amdgcn_s_waitcnt(((NST - 2) * LOADS_PER_STAGE & 0xF) |
                               ((((NST - 2) * LOADS_PER_STAGE) >> 4) << 14) | (7 << 4) | (0xF << 8));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue_stage(ks + NST - 1);   // refills the stage consumed at step ks - 1
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* st = lds + (ks % NST) * ST_BYTES;
    const uint8_t* la = st;
    const uint8_t* lb = st + ST_A;
    const uint32_t* ssa = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B);
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B + ST_SA);
    uint32_t as[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      as[i] = ssa[wm * 128 + i * 32 + l32] >> (8 * grp);
      if (!DGRAD) bs[i] = ssb[wn * 4 + i] >> (8 * grp);
      else bs[i] = ssb[grp * 8 + wn * 4 + i] | (ssb[(2 + grp) * 8 + wn * 4 + i] << 16);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int row = wm * 128 + mt * 32 + l32;
        af[mt] = lds_read_b128(la + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        if (!DGRAD) {
          const int row = wn * 128 + nt * 32 + l32;
          bf[nt] = lds_read_b128(lb + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
        } else {
          const int h = lane >> 4, i = lane & 15;
          const int l8 = 8 * wn + 2 * nt + (h & 1);          // logical 8-byte chunk
          const int rowb = c * 64 + 32 * (h >> 1) + i;
          const int off_lo = rowb * 128 + (((l8 >> 1) ^ ((rowb >> 1) & 7)) << 4) + ((l8 & 1) << 3);
          const int off_hi = (rowb + 16) * 128 + (((l8 >> 1) ^ (((rowb + 16) >> 1) & 7)) << 4) +
                             ((l8 & 1) << 3);
          const u32x2 lo = lds_read_tr4(lb + off_lo);
          const u32x2 hi = lds_read_tr4(lb + off_hi);
          bf[nt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (c == 0)
            acc[mt][nt] = mfma_fp4_32x32x64<0, 0>(af[mt], bf[nt], acc[mt][nt], as[mt], bs[nt]);
          else
            acc[mt][nt] = mfma_fp4_32x32x64<2, 2>(af[mt], bf[nt], acc[mt][nt], as[mt], bs[nt]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  // the loads issued for steps past the end (all zero) must land before the
  // stages are reused by the epilogue
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  epilogue<NRQ>(g, acc, lds, lds + 32768, m0, j0);
}

template <bool DGRAD>
hipError_t launch(const GemmArgs& g, hipStream_t st) {
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool scal = (g.RED & 127) == 0;
#define FT_G(NRQ)                                                                          \
  do {                                                                                     \
    if (scal) hipLaunchKernelGGL((k_gemm_pipe<DGRAD, NRQ>), dim3(n), dim3(256), 0, st, g);   \
    else hipLaunchKernelGGL((k_gemm<DGRAD, NRQ, false>), dim3(n), dim3(256), 0, st, g);     \
  } while (0)
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
