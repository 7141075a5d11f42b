// MXFP4 GEMMs with the low-rank branches fused in.
//
// FourTune (arXiv 2607.05711):
//   forward, Eq. (2):  Y  = GEMM4(Q(X), Q(R)) + X L_stab + X (A B)
//   dgrad,   Eq. (3):  dX = GEMM4(Q(G), Q(R)^T) + G L_stab^T + G (A B)^T
// "3.2": the weight is quantized in square 32x32 tiles, so the transposed
// product uses the same codes and scales; they are kept a second time in
// transposed order (a layout copy of the same numbers, made when the weight
// is quantized), which makes both products the same kernel.  "3.3 Kernel
// Fusion / LoRA Fusion": the 4-bit product and the up-projections are
// accumulated together and the output is written once.
//
// One kernel computes, for both directions,
//   out[m][j] = sum_red deq(a)[m][red] deq(b)[j][red] + sum_r lm[m][r] lo[j][r]
//   forward: a = Qrow(X) [M, K],  b = Qtile(W) [N, K],   lm = U, lo = [L2^T | B^T]
//   dgrad  : a = Qrow(G) [M, N],  b = Qtile(W)^T [K, N], lm = P, lo = [L1 | A]
// with lo given as two row-major pieces [NOUT, r0] and [NOUT, R - r0].
//
// Tiling for gfx950: a 256-thread workgroup computes a 256x256 output tile;
// each of its 4 waves owns 128x128 = 4x4 tiles of the 32x32x64 scaled MXFP4
// MFMA (fp32 accumulators in AGPRs, 16 per lane per tile).
//   - The rank-R part goes first: its bf16 fragments are loaded straight
//     from global memory (rank-contiguous rows, 16 bytes per lane) while the
//     first operand stages are in flight, and 32x32x16 bf16 MFMAs put
//     lm . lo^T into the accumulators.
//   - Reduction steps of 128 elements (64 code bytes per row) go from global
//     memory into LDS with buffer_load ... lds (no registers), 4 stages deep.
//     Each step is split in two halves of 16 MFMAs (one 64-element chunk
//     each); the LDS reads of the next chunk are issued before the MFMAs that
//     need the previous one, and the 10 DMA instructions that refill a stage
//     are spread between MFMAs so that their issue overlaps matrix work.  One
//     barrier per step, between the halves, both publishes the next stage
//     and frees the stage just read.
//   - Scales: one E8M0 byte per 32-block; a lane passes the word holding the
//     bytes of its row and the step's blocks and selects the byte with
//     op_sel.
//   - Raw buffer loads: addresses past the end of a tensor read as zero,
//     which covers ragged edges without branches.
//   - Workgroups are mapped so that each XCD (own L2) works on a compact
//     block of output tiles.
//   - The accumulators are rounded to bf16 in registers (v_cvt_pk_bf16_f32,
//     round to nearest even), neighbouring lanes swap halves so that each
//     holds two adjacent columns of one row, and each store writes 4 bytes a
//     lane.
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
__device__ __forceinline__ uint32_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
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

// ---------------------------------------------------------------------------
// Rank-R part.  For the 32x32x16 bf16 MFMA a lane holds 8 consecutive ranks
// (16q + 8*grp ...) of one row (l%32) of each operand.
template <int NRQ>
struct LowRankFrags {
  u32x4 u[NRQ][4];   // lm rows  wm*128 + 32*i + l32
  u32x4 v[NRQ][4];   // lo rows  wn*128 + 32*i + l32
};

// Ranks are a multiple of 8 and the pieces meet at a multiple of 8: every
// lane segment is 16 contiguous bytes of one piece.
__device__ __forceinline__ bool lowrank_vec(const GemmArgs& g) { return (g.R & 7) == 0 && (g.r0 & 7) == 0; }

// Issue the 16-byte fragment loads (no wait).  Ranks R .. 16*NRQ read as zero.
template <int NRQ>
__device__ __forceinline__ void load_lowrank(const GemmArgs& g, int64_t m0, int64_t j0,
                                             LowRankFrags<NRQ>& f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, NOUT = g.NOUT;
  const int R = g.R, r0 = g.r0, r1 = g.R - g.r0;
  const auto rm = rsrc(g.lm, static_cast<uint64_t>(M) * R * 2);
  const auto rv0 = rsrc(g.lo0, static_cast<uint64_t>(NOUT) * r0 * 2);
  const auto rv1 = rsrc(g.lo1, static_cast<uint64_t>(NOUT) * r1 * 2);
#pragma unroll
  for (int q = 0; q < NRQ; ++q) {
    const int c8 = 16 * q + 8 * grp;        // first rank of this lane's segment
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + 32 * i + l32;
      f.u[q][i] = bload128(rm, (c8 < R && m < M) ? static_cast<uint32_t>((m * R + c8) * 2) : OOB);
      const int64_t j = j0 + wn * 128 + 32 * i + l32;
      const bool jok = j < NOUT;
      if (16 * q + 16 <= r0) {              // both halves in piece 0 (uniform)
        f.v[q][i] = bload128(rv0, jok ? static_cast<uint32_t>((j * r0 + c8) * 2) : OOB);
      } else if (16 * q >= r0) {            // both halves in piece 1 (uniform)
        f.v[q][i] = bload128(rv1, (jok && c8 < R) ? static_cast<uint32_t>((j * r1 + c8 - r0) * 2) : OOB);
      } else {                              // the pieces meet inside this rank group
        const u32x4 x = bload128(rv0, (jok && c8 < r0) ? static_cast<uint32_t>((j * r0 + c8) * 2) : OOB);
        const u32x4 y = bload128(rv1, (jok && c8 >= r0 && c8 < R)
                                          ? static_cast<uint32_t>((j * r1 + c8 - r0) * 2) : OOB);
        f.v[q][i] = x | y;
      }
    }
  }
}

template <int NRQ>
__device__ __forceinline__ void mma_lowrank(const LowRankFrags<NRQ>& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int q = 0; q < NRQ; ++q)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_32x32x16(f.u[q][mt], f.v[q][nt], acc[mt][nt]);
}

// Any other ranks: both rank tiles are staged element by element in LDS
// (rows of 16*NRQ ranks, zero-padded; `buf` holds 2 * 256 * 32 * NRQ bytes)
// and the fragments are read from there.  The loops stay rolled, so few
// registers are live.  Ends with a barrier; `buf` is free afterwards.
template <int NRQ>
__device__ __forceinline__ void lowrank_lds(const GemmArgs& g, int64_t m0, int64_t j0,
                                            f32x16 (&acc)[4][4], uint8_t* buf) {
  constexpr int RP = 16 * NRQ;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, NOUT = g.NOUT;
  const int R = g.R, r0 = g.r0, r1 = g.R - g.r0;
  uint16_t* um = reinterpret_cast<uint16_t*>(buf);
  uint16_t* vm = um + 256 * RP;
#pragma unroll 1
  for (int idx = t; idx < 256 * RP; idx += 256) {
    const int row = idx / RP, r = idx % RP;
    const int64_t m = m0 + row, j = j0 + row;
    um[idx] = (m < M && r < R) ? g.lm[m * R + r] : uint16_t(0);
    uint16_t v = 0;
    if (j < NOUT && r < R) v = r < r0 ? g.lo0[j * r0 + r] : g.lo1[j * r1 + (r - r0)];
    vm[idx] = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < NRQ; ++q) {
    u32x4 u[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u[i] = lds_read_b128(um + (wm * 128 + 32 * i + l32) * RP + 16 * q + 8 * grp);
      v[i] = lds_read_b128(vm + (wn * 128 + 32 * i + l32) * RP + 16 * q + 8 * grp);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_32x32x16(u[mt], v[nt], acc[mt][nt]);
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// bf16 output straight from the accumulators.  Accumulator element r of
// tile (mt, nt) is row 8*(r/4) + 4*grp + r%4, column l32 of the 32x32 tile.
// Rows 2p and 2p+1 of a column are rounded together into one word; lanes
// 2c and 2c+1 then swap halves, so the even lane holds row 2p and the odd
// lane row 2p+1, each for columns 2c and 2c+1.
__device__ __forceinline__ void store_tile(const GemmArgs& g, const f32x16 (&acc)[4][4], int64_t m0,
                                           int64_t j0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, l32 = lane & 31, grp = lane >> 5;
  const int odd = lane & 1;
  const int64_t M = g.M, NOUT = g.NOUT;
  const auto ro = rsrc(g.out, static_cast<uint64_t>(M) * NOUT * 2);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = j0 + wn * 128 + nt * 32 + (l32 & ~1);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const f32x2 x = {acc[mt][nt][2 * p], acc[mt][nt][2 * p + 1]};
        const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
        const uint32_t o = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(w), 0xB1, 0xF, 0xF, false));
        const uint32_t val = odd ? ((o >> 16) | (w & 0xFFFF0000u)) : ((w & 0xFFFFu) | (o << 16));
        const int64_t row = m0 + wm * 128 + mt * 32 + 8 * (p >> 1) + 4 * grp + 2 * (p & 1) + odd;
        const uint32_t off = (row < M && col < NOUT) ? static_cast<uint32_t>((row * NOUT + col) * 2) : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(val, ro, static_cast<int>(off), 0, 0);
      }
    }
}

// ---------------------------------------------------------------------------
// Pipelined kernel for reduction lengths that are a multiple of 128 (every
// step holds whole 4-block scale words).
constexpr int NST = 4;                      // LDS stages
constexpr int ST_A = BM * ROWB;             // 16 KB of A codes
constexpr int ST_B = BN * ROWB;             // 16 KB of B codes
constexpr int ST_SA = BM * 4;               // A scale words, one per row
constexpr int ST_SB = 4 * 256;              // B scale words, one 256-byte region per wave
constexpr int ST_BYTES = ST_A + ST_B + ST_SA + ST_SB;
// Per wave and stage: 4 + 4 code DMAs and 1 + 1 scale DMAs, issued as two
// halves of 5 (A part, B part).
constexpr int DMA_HALF = 5;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14); fields not waited on are at their max.
constexpr int waitcnt_imm(int vm, int lgkm) {
  return (vm & 0xF) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FT_LDS void*)(lds), 16, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FT_LDS void*)(lds), 4, (int)off, 0, 0, 0);
}

template <int NRQ>
__global__ __launch_bounds__(256, 1) void k_gemm_pipe(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * ST_BYTES];

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;
  int64_t m0, j0;
  tile_origin(M, NOUT, m0, j0);

  const uint32_t row_bytes = static_cast<uint32_t>(RED >> 1);
  const uint32_t row_sc = static_cast<uint32_t>(RED >> 5);
  const int nks = static_cast<int>(RED / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * row_sc);
  const auto rb_codes = rsrc(g.b_codes, static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, static_cast<uint64_t>(NOUT >> 5) * row_sc);

  // ---- rank-R fragments: loads go out before the operand stages
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  LowRankFrags<(NRQ > 0 ? NRQ : 1)> lrf;
  const bool lr_vec = NRQ > 0 && lowrank_vec(g);
  if constexpr (NRQ > 0) {
    if (lr_vec) load_lowrank<NRQ>(g, m0, j0, lrf);
    else lowrank_lds<NRQ>(g, m0, j0, acc, lds);
  }

  // ---- per-lane DMA source offsets at step 0.  Instruction q of wave w
  // fills 1 KB of LDS (16 rows of 64 bytes); lane i lands at byte 16 i.
  uint32_t a_src[4], b_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t row = 64 * wave + 16 * q + (lane >> 2), pch = lane & 3;
    a_src[q] = static_cast<uint32_t>(m0 + row) * row_bytes + ((pch ^ swz16(row)) << 4);
    b_src[q] = static_cast<uint32_t>(j0 + row) * row_bytes + ((pch ^ swz16(row)) << 4);
  }
  const uint32_t sa_src = static_cast<uint32_t>(m0 + 64 * wave + lane) * row_sc;
  uint32_t sb_src = OOB;
  {
    const uint32_t nb = static_cast<uint32_t>(j0 >> 5) + lane;
    if (wave == 0 && lane < 8 && nb < (NOUT >> 5)) sb_src = nb * row_sc;
  }

  // DMA instruction `item` (0..9) of stage ks for this wave
  auto dma = [&](int ks, int item) {
    uint8_t* st = lds + (ks & (NST - 1)) * ST_BYTES;
    const uint32_t k0 = static_cast<uint32_t>(ks) * BK;
    const bool kin = k0 < RED;
    if (item < 4)
      dma16(ra_codes, st + (64 * wave + 16 * item) * ROWB, kin ? a_src[item] + (k0 >> 1) : OOB);
    else if (item == 4)
      dma4(ra_sc, st + ST_A + ST_B + 64 * wave * 4, kin ? sa_src + (k0 >> 5) : OOB);
    else if (item < 9)
      dma16(rb_codes, st + ST_A + (64 * wave + 16 * (item - 5)) * ROWB,
            kin ? b_src[item - 5] + (k0 >> 1) : OOB);
    else
      dma4(rb_sc, st + ST_A + ST_B + ST_SA + wave * 256,
           (kin && sb_src != OOB) ? sb_src + (k0 >> 5) : OOB);
  };
  auto read_frags = [&](int buf, int c, u32x4 (&af)[4], u32x4 (&bf)[4]) {
    const uint8_t* st = lds + buf * ST_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wm * 128 + i * 32 + l32;
      af[i] = lds_read_b128(st + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = wn * 128 + i * 32 + l32;
      bf[i] = lds_read_b128(st + ST_A + row * ROWB + (((2 * c + grp) ^ swz16(row)) << 4));
    }
  };
  auto read_scales = [&](int buf, uint32_t (&as)[4], uint32_t (&bs)[4]) {
    const uint8_t* st = lds + buf * ST_BYTES;
    const uint32_t* ssa = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B);
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B + ST_SA);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      as[i] = ssa[wm * 128 + i * 32 + l32] >> (8 * grp);
      bs[i] = ssb[wn * 4 + i] >> (8 * grp);
    }
  };

  // ---- prologue: stages 0..2 and the A half of stage 3
#pragma unroll
  for (int s = 0; s < NST - 1; ++s)
#pragma unroll
    for (int item = 0; item < 2 * DMA_HALF; ++item) dma(s, item);
#pragma unroll
  for (int item = 0; item < DMA_HALF; ++item) dma(NST - 1, item);
  if constexpr (NRQ > 0) {
    if (lr_vec) mma_lowrank<NRQ>(lrf, acc);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(5 * DMA_HALF, 0xF));   // this wave's stage 0 landed
  __builtin_amdgcn_s_barrier();                                  // ... and every wave's
  __builtin_amdgcn_sched_barrier(0);
  u32x4 a0[4], b0[4];
  uint32_t as[4], bs[4];
  read_scales(0, as, bs);
  read_frags(0, 0, a0, b0);
  __builtin_amdgcn_sched_barrier(0);

  // Step ks: stage ks is in LDS and its chunk-0 fragments and scales are in
  // registers.  DMA order per wave: ..., B half of stage ks+3 (first half of
  // step ks), A half of stage ks+4 (second half of step ks), ...  Past the
  // end of the reduction they are zero-fill loads that are never read.
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & (NST - 1);
    u32x4 a1[4], b1[4];
    read_frags(cur, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i >> 2][i & 3] =
          mfma_fp4_32x32x64<0, 0>(a0[i >> 2], b0[i & 3], acc[i >> 2][i & 3], as[i >> 2], bs[i & 3]);
      if (i % 3 == 1) {
        __builtin_amdgcn_sched_barrier(0);
        dma(ks + NST - 1, DMA_HALF + i / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Own loads of stage ks+1 landed (the 4 younger halves may be in
    // flight) and own reads of stage ks done; after the barrier the same
    // holds for every wave: stage ks+1 is readable and stage ks reusable.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * DMA_HALF, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    uint32_t as2[4], bs2[4];
    read_scales((ks + 1) & (NST - 1), as2, bs2);
    read_frags((ks + 1) & (NST - 1), 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      acc[i >> 2][i & 3] =
          mfma_fp4_32x32x64<2, 2>(a1[i >> 2], b1[i & 3], acc[i >> 2][i & 3], as[i >> 2], bs[i & 3]);
      if (i % 3 == 1) {
        __builtin_amdgcn_sched_barrier(0);
        dma(ks + NST, i / 3);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) { as[i] = as2[i]; bs[i] = bs2[i]; }
  }
  // DMAs into LDS must land before the workgroup can end
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0xF));
  store_tile(g, acc, m0, j0);
}

// ---------------------------------------------------------------------------
// Register-staged kernel for reduction lengths that are a multiple of 32
// but not of 128: the last step is partial, so scale bytes are fetched one
// by one and code chunks past the row end read as zero.  Two LDS buffers;
// the loads of step k+1 are in flight while step k runs.
template <int NRQ>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs g) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * ROWB];  // 64 KB
  uint8_t* const lds_a = lds;                      // 2 A buffers
  uint8_t* const lds_b = lds + 2 * BM * ROWB;      // 2 B buffers

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;

  int64_t m0, j0;
  tile_origin(M, NOUT, m0, j0);

  const uint32_t row_bytes = static_cast<uint32_t>(RED >> 1);
  const uint32_t row_sc = static_cast<uint32_t>(RED >> 5);
  const int nks = static_cast<int>((RED + BK - 1) / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * row_sc);
  const auto rb_codes = rsrc(g.b_codes, static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, static_cast<uint64_t>(NOUT >> 5) * row_sc);

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  if constexpr (NRQ > 0) {
    if (lowrank_vec(g)) {
      LowRankFrags<NRQ> lrf;
      load_lowrank<NRQ>(g, m0, j0, lrf);
      mma_lowrank<NRQ>(lrf, acc);
    } else {
      lowrank_lds<NRQ>(g, m0, j0, acc, lds);
    }
  }

  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = (t >> 2) + 64 * i, ch = t & 3;
    a_off[i] = static_cast<uint32_t>(m0 + row) * row_bytes + ch * 16;
    b_off[i] = static_cast<uint32_t>(j0 + row) * row_bytes + ch * 16;
  }
  uint32_t sa_off[4], sb_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa_off[i] = static_cast<uint32_t>(m0 + wm * 128 + i * 32 + l32) * row_sc;
    sb_off[i] = static_cast<uint32_t>((j0 + wn * 128 + i * 32) >> 5) * row_sc;
  }

  // Loaded values are only moved into registers here; scale bytes are
  // combined into words at the point of use.
  u32x4 ra[4], rb[4];
  uint32_t sa_raw[4][4], sb_raw[4][4];
  auto issue_loads = [&](int ks) {
    const uint32_t k0 = static_cast<uint32_t>(ks) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool kin = k0 + (t & 3) * 32 < RED;
      ra[i] = bload128(ra_codes, kin ? a_off[i] + (k0 >> 1) : OOB);
      rb[i] = bload128(rb_codes, kin ? b_off[i] + (k0 >> 1) : OOB);
    }
    const uint32_t kb0 = k0 >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = kb0 + j < row_sc;
        sa_raw[i][j] = bload8(ra_sc, in ? sa_off[i] + kb0 + j : OOB);
        sb_raw[i][j] = bload8(rb_sc, (in && j0 + wn * 128 + i * 32 < NOUT) ? sb_off[i] + kb0 + j : OOB);
      }
  };
  auto store_lds = [&](int buf) {
    uint8_t* la = lds_a + buf * (BM * ROWB);
    uint8_t* lb = lds_b + buf * (BN * ROWB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 2) + 64 * i, ch = t & 3;
      *reinterpret_cast<u32x4*>(la + row * ROWB + ((ch ^ swz16(row)) << 4)) = ra[i];
      *reinterpret_cast<u32x4*>(lb + row * ROWB + ((ch ^ swz16(row)) << 4)) = rb[i];
    }
  };

  uint32_t sa[4][4], sb[4][4];
  auto take_scales = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) { sa[i][j] = sa_raw[i][j]; sb[i][j] = sb_raw[i][j]; }
  };
  issue_loads(0);
  store_lds(0);
  take_scales();
  __syncthreads();

  // On the last step the loads for step nks address past the reduction
  // dimension: out-of-range buffer loads that return zero and are not used.
  for (int ks = 0; ks < nks; ++ks) {
    const int cur = ks & 1;
    issue_loads(ks + 1);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t as[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      as[i] = (sa[i][0] | (sa[i][1] << 8) | (sa[i][2] << 16) | (sa[i][3] << 24)) >> (8 * grp);
      bs[i] = (sb[i][0] | (sb[i][1] << 8) | (sb[i][2] << 16) | (sb[i][3] << 24)) >> (8 * grp);
    }
    const uint8_t* la = lds_a + cur * (BM * ROWB);
    const uint8_t* lb = lds_b + cur * (BN * ROWB);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ra_row = wm * 128 + i * 32 + l32, rb_row = wn * 128 + i * 32 + l32;
        af[i] = lds_read_b128(la + ra_row * ROWB + (((2 * c + grp) ^ swz16(ra_row)) << 4));
        bf[i] = lds_read_b128(lb + rb_row * ROWB + (((2 * c + grp) ^ swz16(rb_row)) << 4));
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
  store_tile(g, acc, m0, j0);
}

}  // namespace

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool pipe = (g.RED & 127) == 0;
#define FT_G(NRQ)                                                                          \
  do {                                                                                     \
    if (pipe) hipLaunchKernelGGL((k_gemm_pipe<NRQ>), dim3(n), dim3(256), 0, st, g);         \
    else hipLaunchKernelGGL((k_gemm<NRQ>), dim3(n), dim3(256), 0, st, g);                   \
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

}  // namespace ft
