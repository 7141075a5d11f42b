// MXFP4 GEMMs with the low-rank branches fused in.
//
// FourTune (arXiv 2607.05711):
//   forward, Eq. (2):  Y  = GEMM4(Q(X), Q(R)) + X L_stab + X (A B)
//   dgrad,   Eq. (3):  dX = GEMM4(Q(G), Q(R)^T) + G L_stab^T + G (A B)^T
// "3.2": the weight is quantized in square 32x32 tiles, so the transposed
// product reads the same codes and scales: the dgrad stages [reduction rows
// x output columns] pieces of the one packed weight in LDS and takes its
// operand fragments with the 4-bit transposing LDS read (ds_read_b64_tr_b4),
// and each 32x32 tile's scale byte serves both directions.  "3.3 Kernel
// Fusion / LoRA Fusion": the 4-bit product and the up-projections are
// accumulated together and the output is written once.
//
// One kernel computes, for both directions,
//   out[m][j] = sum_red deq(a)[m][red] deq(b)[j][red] + sum_r lm[m][r] lo[j][r]
//   forward: a = Qrow(X) [M, K],  b = Qtile(W) [N, K],   lm = U, lo = [L2^T | B^T]
//   dgrad  : a = Qrow(G) [M, N],  b = Qtile(W) [N, K] read transposed,
//            lm = P, lo = [L1 | A]
// with lm and lo zero-padded to 32 * nlr ranks (written that way by the
// fused quantize + down-projection kernel that runs just before).
//
// Tiling for gfx950: a 256-thread workgroup computes 256x256 output tiles;
// each of its 4 waves owns 128x128 = 4x4 tiles of the 32x32x64 scaled MXFP4
// MFMA (fp32 accumulators in AGPRs, 16 per lane per tile).
//   - Persistent: one workgroup per CU walks its share of the output tiles.
//     Its loads run as one pipeline across tile boundaries, so only the
//     first tile waits for memory and each tile's output stores overlap the
//     next tile's loads.
//   - A tile is a sequence of 64-byte-per-row steps: first nlr rank steps
//     (32 ranks of lm and lo in bf16, 32x32x16 bf16 MFMAs), then RED/128
//     reduction steps (128 4-bit elements of a and b, scaled MXFP4 MFMAs).
//     Both kinds have the same shape, so they share the load pipeline and
//     the LDS layout.
//   - Operands go from global memory into LDS with buffer_load ... lds (no
//     registers), 4 stages deep.  Each step is split in two halves of 16
//     MFMAs (one 64-element chunk each); the barrier between them publishes
//     the next stage and frees the stage just read.  The 10 DMA instructions
//     that refill a stage are spread between the MFMAs.
//   - Even and odd steps use separate fragment and scale registers, so that
//     no LDS read or VALU result ever targets a register an MFMA still in
//     flight reads (such writes stall the wave until the MFMA is done).  An
//     odd number of reduction steps is padded by one all-zero step, so every
//     tile has an even number.
//   - No register spills: a spilled value's reload waits for all memory
//     operations (vmcnt(0)) and so drains the load pipeline; lane-dependent
//     offsets used rarely are rebuilt where they are used instead.
//   - Scales: one E8M0 byte per 32-block; a lane passes the word holding the
//     bytes of its row and the step's blocks and selects the byte with
//     op_sel.
//   - Raw buffer loads: addresses past the end of a tensor read as zero,
//     which covers ragged edges without branches.
//   - Tiles are handed out so that the workgroups one XCD (own L2) runs at
//     the same time work on a compact block of output tiles.
//   - Output: the accumulators are rounded to bf16 in registers
//     (v_cvt_pk_bf16_f32, round to nearest even), neighbouring lanes swap
//     halves so that each holds two adjacent columns of one row, and 16-row
//     strips go through a small per-wave LDS area to 16-byte global stores.
//     The stores are non-temporal (each instruction writes whole 128-byte
//     lines): the output is not read again by this layer, and keeping it out
//     of the caches leaves the inputs the next kernels read there (measured
//     on the QKV step: GEMMs unchanged, the adapter-gradient and forward
//     quantize launches after them 2-3 us faster each).
#include "gemm_pipe.hpp"

#include <algorithm>

namespace ft {

namespace {

// ---------------------------------------------------------------------------
// Register-staged kernel for reduction lengths that are a multiple of 32
// but not of 128: the last step is partial, so scale bytes are fetched one
// by one and code chunks past the row end read as zero.  Two LDS buffers;
// the loads of step k+1 are in flight while step k runs.  The rank part
// comes first, from fragments loaded straight from the padded rank rows.
// BMODE as for k_gemm_pipe (0 tiles, 1 row blocks, 3 tiles stored
// [RED, NOUT/2] and read transposed, with the same LDS layout and
// transposing reads as there).
template <int BMODE>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs g) {
  constexpr bool BROW = BMODE == 1, BT = BMODE == 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (BM + BN) * ROWB];  // 64 KB
  uint8_t* const lds_a = lds;                      // 2 A buffers
  uint8_t* const lds_b = lds + 2 * BM * ROWB;      // 2 B buffers

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5, odd = lane & 1;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;

  int64_t m0, j0;
  {
    const uint32_t mt_n = static_cast<uint32_t>((M + BM - 1) / BM);
    const uint32_t nt_n = static_cast<uint32_t>((NOUT + BN - 1) / BN);
    tile_coords(xcd_remap(blockIdx.x, mt_n * nt_n), mt_n, nt_n, m0, j0);
  }

  const uint32_t row_bytes = static_cast<uint32_t>(RED >> 1);
  const uint32_t row_sc = static_cast<uint32_t>(RED >> 5);
  const uint32_t bt_row = static_cast<uint32_t>(NOUT >> 1), bt_ks = static_cast<uint32_t>(NOUT >> 5);
  const int nks = static_cast<int>((RED + BK - 1) / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * row_sc);
  const auto rb_codes = rsrc(g.b_codes, BT ? static_cast<uint64_t>(RED) * bt_row
                                           : static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, BT ? static_cast<uint64_t>(RED >> 5) * bt_ks
                                         : static_cast<uint64_t>(BROW ? NOUT : NOUT >> 5) * row_sc);

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // rank part: lane (row l32, half grp) holds ranks 16q + 8grp .. +7
  const int lrb = g.nlr * 64;
  const auto r_lm = rsrc(g.lm, static_cast<uint64_t>(M) * lrb);
  const auto r_lo = rsrc(g.lo, static_cast<uint64_t>(NOUT) * lrb);
  for (int q = 0; q < 2 * g.nlr; ++q) {
    u32x4 u[4], v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 128 + 32 * i + l32, j = j0 + wn * 128 + 32 * i + l32;
      u[i] = bload128(r_lm, m < M ? static_cast<uint32_t>(m * lrb + 32 * q + 16 * grp) : OOB);
      v[i] = bload128(r_lo, j < NOUT ? static_cast<uint32_t>(j * lrb + 32 * q + 16 * grp) : OOB);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = mfma_bf16_32x32x16(u[mt], v[nt], acc[mt][nt]);
  }

  uint32_t a_off[4], b_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = (t >> 2) + 64 * i, ch = t & 3;
    a_off[i] = static_cast<uint32_t>(m0 + row) * row_bytes + ch * 16;
    if constexpr (BT) {
      // stored reduction row t / 8 + 32 i of the step, logical slot t % 8
      b_off[i] = ((t >> 3) + 32 * i) * bt_row + static_cast<uint32_t>(j0 >> 1) + (t & 7) * 16;
    } else {
      b_off[i] = static_cast<uint32_t>(j0 + row) * row_bytes + ch * 16;
    }
  }
  uint32_t sa_off[4], sb_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa_off[i] = static_cast<uint32_t>(m0 + wm * 128 + i * 32 + l32) * row_sc;
    sb_off[i] = BT ? static_cast<uint32_t>((j0 + wn * 128 + i * 32) >> 5)
                   : static_cast<uint32_t>(BROW ? j0 + wn * 128 + i * 32 + l32 : (j0 + wn * 128 + i * 32) >> 5) * row_sc;
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
      if constexpr (BT) {
        const bool rin = k0 + (t >> 3) + 32 * i < RED;
        rb[i] = bload128(rb_codes, rin ? b_off[i] + k0 * bt_row : OOB);
      } else {
        rb[i] = bload128(rb_codes, kin ? b_off[i] + (k0 >> 1) : OOB);
      }
    }
    const uint32_t kb0 = k0 >> 5;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = kb0 + j < row_sc;
        sa_raw[i][j] = bload8(ra_sc, in ? sa_off[i] + kb0 + j : OOB);
        if constexpr (BT)
          sb_raw[i][j] = bload8(rb_sc, (in && j0 + wn * 128 + i * 32 < NOUT) ? (kb0 + j) * bt_ks + sb_off[i] : OOB);
        else
          sb_raw[i][j] = bload8(rb_sc, (in && j0 + wn * 128 + i * 32 + (BROW ? l32 : 0) < NOUT) ? sb_off[i] + kb0 + j : OOB);
      }
  };
  auto store_lds = [&](int buf) {
    uint8_t* la = lds_a + buf * (BM * ROWB);
    uint8_t* lb = lds_b + buf * (BN * ROWB);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = (t >> 2) + 64 * i, ch = t & 3;
      *reinterpret_cast<u32x4*>(la + row * ROWB + ((ch ^ swz16(row)) << 4)) = ra[i];
      if constexpr (BT) {
        const int brow = (t >> 3) + 32 * i;
        *reinterpret_cast<u32x4*>(lb + brow * 128 + (((t & 7) ^ ((brow >> 1) & 7)) << 4)) = rb[i];
      } else {
        *reinterpret_cast<u32x4*>(lb + row * ROWB + ((ch ^ swz16(row)) << 4)) = rb[i];
      }
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
        if constexpr (BT) {
          // as read_frags_bt of k_gemm_pipe
          const int q = lane & 15, hf = (lane >> 4) & 1, sw = (q >> 1) & 7;
          const uint8_t* rbp = lb + (64 * c + 32 * grp + q) * 128 + 8 * hf + (((4 * wn + i) ^ sw) << 4);
          const u32x2 lo = lds_read_tr4(rbp);
          const u32x2 hi = lds_read_tr4(rbp + 16 * 128);
          bf[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          bf[i] = lds_read_b128(lb + rb_row * ROWB + (((2 * c + grp) ^ swz16(rb_row)) << 4));
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

  // bf16 output, 4 bytes a lane (see pair_bf16)
  const auto r_out = rsrc(g.out, static_cast<uint64_t>(M) * NOUT * 2);
  const uint32_t psel = pair_sel(odd);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int64_t col = j0 + wn * 128 + nt * 32 + (l32 & ~1);
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const uint32_t val = pair_bf16(acc[mt][nt][2 * p], acc[mt][nt][2 * p + 1], psel);
        const int64_t row = m0 + wm * 128 + mt * 32 + 8 * (p >> 1) + 4 * grp + 2 * (p & 1) + odd;
        const uint32_t off = (row < M && col < NOUT) ? static_cast<uint32_t>((row * NOUT + col) * 2) : OOB;
        __builtin_amdgcn_raw_buffer_store_b32(val, r_out, static_cast<int>(off), 0, 0);
      }
    }
}

}  // namespace

// A unit's work against the cost of its sums (times in us): a step pair
// takes about 2.1; a unit ends by storing its rows' fp32 sums, at about 25
// GB/s per workgroup; the adding kernel reads them all (5 TB/s) and costs
// about 3 more.  S is the cheapest count under that model that keeps every
// unit in one round of 256; shapes alone decide it, so the workspace size
// does not depend on the device.
namespace {
// ---------------------------------------------------------------------------
// k_gemm_rows: outputs of at most 16 rows (a modulation linear at M = 2),
// streaming b.  Waves 2 q and 2 q + 1 own 16 output columns (b rows), each
// one half of the reduction, as scaled 16x16x128 fp4 MFMAs: lane (r, g) (r =
// lane % 16, g = lane / 16) supplies 32 reduction values (16 bytes) of a
// row r and of b row r for chunk c, block 4 c + g, with its block's scale
// byte.  a's rows are the same for every wave (L2-resident); b's 32 rows of
// a workgroup are read once from HBM.  Chunks go in batches of 6, the next
// batch's loads issued before the current batch's MFMAs, so each wave keeps
// 12 KB in flight and a CU (two or three workgroups) over 100 KB.  The
// second half's sums join the first's through LDS (in that order); the rank
// part is two or four 16x16x32 bf16 MFMAs into the same accumulators (same
// layout), and the output is rounded once.  BROW: b has 1x32 row scales,
// else one scale per 32x32 tile.
constexpr int RB_NB = 6;
template <bool BROW>
__global__ __launch_bounds__(256) void k_gemm_rows(const GemmArgs g) {
  __shared__ f32x4 part[2][64];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int r = lane & 15, kg = lane >> 4, q = wave >> 1, kh = wave & 1;
  const uint32_t M = static_cast<uint32_t>(g.M), RED = static_cast<uint32_t>(g.RED);
  const uint32_t NOUT = static_cast<uint32_t>(g.NOUT);
  const uint32_t nch = RED / BK, rowb = RED / 2, rsc = RED / 32;
  const uint32_t nh = (nch + 1) / 2, cbeg = kh * nh, cend = kh ? nch : nh;
  const uint32_t n = blockIdx.x * 32 + q * 16 + r;
  const bool aok = static_cast<uint32_t>(r) < M, bok = n < NOUT;
  const auto ra = rsrc(g.a_codes, static_cast<uint64_t>(M) * rowb);
  const auto ras = rsrc(g.a_scales, static_cast<uint64_t>(M) * rsc);
  const auto rb = rsrc(g.b_codes, static_cast<uint64_t>(NOUT) * rowb);
  const auto rbs = rsrc(g.b_scales, static_cast<uint64_t>(BROW ? NOUT : (NOUT + 31) / 32) * rsc);
  const uint32_t a_row = aok ? static_cast<uint32_t>(r) * rowb : OOB;
  const uint32_t b_row = bok ? n * rowb : OOB;
  const uint32_t a_srow = aok ? static_cast<uint32_t>(r) * rsc : OOB;
  const uint32_t b_srow = bok ? (BROW ? n : n / 32) * rsc : OOB;
  struct Batch {
    u32x4 a[RB_NB], b[RB_NB];
    uint32_t as[RB_NB], bs[RB_NB];
  };
  // chunk c: codes at 64 c + 16 g of the row, scale bytes 4 c .. 4 c + 3 of
  // the row's scale run as one word (the lane's byte is g)
  auto load = [&](uint32_t c0, Batch& B) {
#pragma unroll
    for (int c = 0; c < RB_NB; ++c) {
      const bool in = c0 + c < cend;
      const uint32_t co = (c0 + c) * 64 + 16 * kg, so = 4 * (c0 + c);
      B.a[c] = bload128(ra, in && a_row != OOB ? a_row + co : OOB);
      B.b[c] = bload128(rb, in && b_row != OOB ? b_row + co : OOB);
      B.as[c] = __builtin_amdgcn_raw_buffer_load_b32(ras, static_cast<int>(in && a_srow != OOB ? a_srow + so : OOB), 0, 0);
      B.bs[c] = __builtin_amdgcn_raw_buffer_load_b32(rbs, static_cast<int>(in && b_srow != OOB ? b_srow + so : OOB), 0, 0);
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Batch& B) {
#pragma unroll
    for (int c = 0; c < RB_NB; ++c) {
      const uint32_t sa = (B.as[c] >> (8 * kg)) & 0xFFu, sb = (B.bs[c] >> (8 * kg)) & 0xFFu;
      const i32x8 av = {(int)B.a[c][0], (int)B.a[c][1], (int)B.a[c][2], (int)B.a[c][3], 0, 0, 0, 0};
      const i32x8 bv = {(int)B.b[c][0], (int)B.b[c][1], (int)B.b[c][2], (int)B.b[c][3], 0, 0, 0, 0};
      acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 4, 4, 0, (int)sa, 0, (int)sb);
    }
  };
  Batch E, O;
  load(cbeg, E);
  for (uint32_t c0 = cbeg; c0 < cend; c0 += 2 * RB_NB) {
    load(c0 + RB_NB, O);
    compute(E);
    if (c0 + 2 * RB_NB < cend) load(c0 + 2 * RB_NB, E);
    compute(O);
  }
  if (kh) part[q][lane] = acc;
  __syncthreads();
  if (kh) return;
  acc += part[q][lane];
  // rank part: 32 ranks per MFMA, lane (r, g) ranks 8 g .. 8 g + 7
  const int rp = 32 * g.nlr;
  if (rp > 0) {
    const auto rlm = rsrc(g.lm, static_cast<uint64_t>(M) * rp * 2);
    const auto rlo = rsrc(g.lo, static_cast<uint64_t>(NOUT) * rp * 2);
    for (int k = 0; k < rp; k += 32) {
      const u32x4 ua = bload128(rlm, aok ? (static_cast<uint32_t>(r) * rp + k + 8 * kg) * 2 : OOB);
      const u32x4 vb = bload128(rlo, bok ? (n * rp + k + 8 * kg) * 2 : OOB);
      acc = mfma_bf16_16x16x32(ua, vb, acc);
    }
  }
  // lane (r, g) holds column n, rows 4 g .. 4 g + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = 4 * kg + i;
    if (row < M && bok) g.out[static_cast<uint64_t>(row) * NOUT + n] = f32_to_bf16_rne(acc[i]);
  }
}
}  // namespace

SplitPlan gemm_split_plan(int64_t M, int64_t RED, int64_t NOUT) {
  SplitPlan p{1, 0};
  if (M <= 0 || RED <= 0 || (RED & 127) != 0 || (NOUT & 3) != 0) return p;
  const int64_t tiles = ((M + BM - 1) / BM) * ((NOUT + BN - 1) / BN);
  const int64_t steps = RED / BK, pairs = (steps + 1) / 2;
  if (tiles > 128 || pairs < 2) return p;
  const int64_t smax = std::min<int64_t>(pairs, 256 / tiles);
  const double unit_rows = static_cast<double>(std::min<int64_t>(M, BM));
  double best = 2.1 * pairs;
  for (int64_t sc = 2; sc <= smax; ++sc) {
    const int64_t per = (pairs + sc - 1) / sc;
    const int64_t used = (pairs + per - 1) / per;        // no empty split
    const double t = 2.1 * per + unit_rows * BN * 4 / 25e3 +
                     static_cast<double>(used) * M * NOUT * 4 / 5e6 + 3.0;
    if (t < best) {
      best = t;
      p.splits = static_cast<int>(used);
      p.pairs = static_cast<int>(per);
    }
  }
  return p;
}

namespace {
// out[m][j] = bf16(sum over splits s (in order) of part[s][m][j] + sum over
// ranks r of lm[m][r] lo[j][r]).  Workgroup: ROWS rows x 256 columns;
// thread t owns column j0 + t.  Its first batch of splits' sums and its
// rank row of lo are loaded before the rows of lm are staged in LDS, so that
// one memory latency covers all three; later splits follow a batch at a
// time.  NLR (rank steps, 32 ranks each) is a template parameter so that the
// lo row sits in registers indexed by constants.  ROWS = 4 for outputs of a
// few rows; 16 otherwise, so that each lo row read serves 16 rows (with 4,
// a 1024-row output spent 32 us here, mostly re-reading lo).
template <int NLR, int ROWS, int NS>
__global__ __launch_bounds__(256) void k_split_reduce(const GemmArgs g) {
  constexpr int RP = 32 * NLR;
  __shared__ __attribute__((aligned(16))) uint16_t slm[ROWS * (RP > 0 ? RP : 8)];
  // 32-bit indices (the sums are below 2^31 bytes); the row and split
  // tests are uniform and the column is clamped into the row, so every
  // load is a buffer load with a selected offset: no branches, and the
  // loads of a batch all issue before the first wait
  const uint32_t M = static_cast<uint32_t>(g.M), NOUT = static_cast<uint32_t>(g.NOUT);
  const uint32_t j = blockIdx.x * 256 + threadIdx.x;
  const uint32_t jc = j < NOUT ? j : NOUT - 1;
  const uint32_t m0 = blockIdx.y * ROWS;
  const int S = g.splits;
  const auto rpart = rsrc(g.part, static_cast<uint64_t>(S) * M * NOUT * 4);
  auto load_batch = [&](int sp0, float (&v)[ROWS][NS]) {
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const bool ok = sp0 + k < S && m0 + i < M;
        const uint32_t row = (static_cast<uint32_t>(sp0 + k) * M + m0 + i) * NOUT;
        v[i][k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                rpart, static_cast<int>(ok ? (row + jc) * 4 : OOB), 0, 0));
      }
  };
  float v[ROWS][NS];
  load_batch(0, v);
  u32x4 vo[RP > 0 ? RP / 8 : 1];
  if constexpr (RP > 0) {
    const auto rlo = rsrc(g.lo, static_cast<uint64_t>(NOUT) * RP * 2);
#pragma unroll
    for (int c = 0; c < RP / 8; ++c) vo[c] = bload128(rlo, (jc * RP + 8 * c) * 2);
    const auto rlm = rsrc(g.lm, static_cast<uint64_t>(M) * RP * 2);
    for (int e = threadIdx.x; e < ROWS * RP / 8; e += 256) {
      const int r = e / (RP / 8), c = e % (RP / 8);
      const u32x4 w = bload128(rlm, m0 + r < M ? ((m0 + r) * RP + 8 * c) * 2 : OOB);
      *reinterpret_cast<u32x4*>(slm + r * RP + 8 * c) = w;
    }
    __syncthreads();
  }
  float acc[ROWS];
#pragma unroll
  for (int i = 0; i < ROWS; ++i) {
    acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < NS; ++k) acc[i] += v[i][k];
  }
  for (int sp0 = NS; sp0 < S; sp0 += NS) {
    load_batch(sp0, v);
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
#pragma unroll
      for (int k = 0; k < NS; ++k) acc[i] += v[i][k];
  }
  if constexpr (RP > 0) {
    // The lm rows are the same for every lane: they are read through an
    // opaque lane offset of 0, so the compiler keeps them in vector
    // registers (as uniform values it would hold them in scalar registers,
    // and spill), and that offset is made to depend on the previous row's
    // result, so each row's reads issue when that row is next (hoisted all
    // at once, the 16 rows' reads took more registers than there are).
    int z = 0;
    float prev = 0.f;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      asm volatile("" : "+v"(z) : "v"(prev));
      const uint16_t* sl = slm + z;
      float s = acc[i];
#pragma unroll
      for (int c = 0; c < RP / 8; ++c) {
        const u32x4 uw = *reinterpret_cast<const u32x4*>(sl + i * RP + 8 * c);
        // (an opaque copy: lo is unpacked row by row, not held unpacked)
        u32x4 vc = vo[c];
        asm volatile("" : "+v"(vc));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          s = __builtin_fmaf(bf16lo_to_f32(uw[w]), bf16lo_to_f32(vc[w]), s);
          s = __builtin_fmaf(bf16hi_to_f32(uw[w]), bf16hi_to_f32(vc[w]), s);
        }
      }
      acc[i] = s;
      prev = s;
    }
  }
  if (j >= NOUT) return;
#pragma unroll
  for (int i = 0; i < ROWS; ++i)
    if (m0 + i < M) g.out[static_cast<uint64_t>(m0 + i) * NOUT + j] = f32_to_bf16_rne(acc[i]);
}
}  // namespace

uint32_t gemm_workgroups(const GemmArgs& g) {
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool bf = g.a16 != nullptr;
  if (!g.e_codes && gemm_rows_ok(g.M, g.RED, bf, g.b_transposed != 0))
    return static_cast<uint32_t>((g.NOUT + 31) / 32);
  const bool pipe = (g.RED & 127) == 0 || (bf && (g.RED & 31) == 0);
  if (!pipe) return n;
  const int cus = cu_count();
  if (cus <= 0) return 0;
  const uint32_t units = !g.e_codes && g.splits > 1 ? n * static_cast<uint32_t>(g.splits) : n;
  return std::min(units, static_cast<uint32_t>(cus));
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool bf = g.a16 != nullptr;
  // dA beside the product: the pipelined transposed-weight kernel only, its
  // grid as gemm_workgroups gives it, ranks in one pass
  if (g.side_wgs > 0 && (g.e_codes || !g.b_transposed || bf || g.b_row_scales ||
                         (g.RED & 127) != 0 || g.gemm_wgs != gemm_workgroups(g) ||
                         g.lora_a.rl < 1 || g.lora_a.rl > 64 || g.lora_a.act != 0 ||
                         (g.lora_b.nchunk > 0 && g.lora_b.rl != g.lora_a.rl)))
    return hipErrorInvalidValue;
  // MLP fusion: the fused epilogues' instantiations live in gemm_mlp.hip
  if (g.e_codes) return launch_gemm_mlp(g, st);
  if (gemm_rows_ok(g.M, g.RED, bf, g.b_transposed != 0)) {
    // at most 16 rows: stream b, 32 output columns per workgroup
    if (g.nlr != 0 && g.nlr != 2 && g.nlr != 4) return hipErrorInvalidValue;
    const dim3 grid(static_cast<uint32_t>((g.NOUT + 31) / 32));
    if (g.b_row_scales) hipLaunchKernelGGL(k_gemm_rows<true>, grid, dim3(256), 0, st, g);
    else hipLaunchKernelGGL(k_gemm_rows<false>, grid, dim3(256), 0, st, g);
    return hipGetLastError();
  }
  if (g.splits > 1) {
    // split reduction: the units without rank steps, then the sums
    if (bf || (g.RED & 127) != 0 || !g.part || g.split_pairs < 1 || (g.NOUT & 3) != 0)
      return hipErrorInvalidValue;
    if (g.nlr != 0 && g.nlr != 2 && g.nlr != 4) return hipErrorInvalidValue;
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const uint32_t units = n * static_cast<uint32_t>(g.splits);
    const uint32_t grid = (units < static_cast<uint32_t>(cus) ? units : static_cast<uint32_t>(cus)) + g.side_wgs;
    if (g.b_row_scales) hipLaunchKernelGGL((k_gemm_pipe<0, 1>), dim3(grid), dim3(256), 0, st, g);
    else if (g.b_transposed) hipLaunchKernelGGL((k_gemm_pipe<0, 3>), dim3(grid), dim3(256), 0, st, g);
    else hipLaunchKernelGGL((k_gemm_pipe<0, 0>), dim3(grid), dim3(256), 0, st, g);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const bool few = g.M <= 64;
    const int rows = few ? 4 : 16;
    const dim3 rgrid(static_cast<uint32_t>((g.NOUT + 255) / 256), static_cast<uint32_t>((g.M + rows - 1) / rows));
#define FT_SR(NL)                                                                        \
  do {                                                                                   \
    if (few) hipLaunchKernelGGL((k_split_reduce<NL, 4, 8>), rgrid, dim3(256), 0, st, g);  \
    else hipLaunchKernelGGL((k_split_reduce<NL, 16, 2>), rgrid, dim3(256), 0, st, g);     \
  } while (0)
    if (g.nlr == 4) FT_SR(4);
    else if (g.nlr == 2) FT_SR(2);
    else FT_SR(0);
#undef FT_SR
    return hipGetLastError();
  }
  if ((g.RED & 127) == 0 || (bf && (g.RED & 31) == 0)) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const uint32_t grid = (n < static_cast<uint32_t>(cus) ? n : static_cast<uint32_t>(cus)) + g.side_wgs;
#define FT_GP(NL, MODE) hipLaunchKernelGGL((k_gemm_pipe<NL, MODE>), dim3(grid), dim3(256), 0, st, g)
#define FT_GPN(MODE) do { if (g.nlr == 4) FT_GP(4, MODE); else if (g.nlr > 0) FT_GP(2, MODE); else FT_GP(0, MODE); } while (0)
    if (g.nlr != 0 && g.nlr != 2 && g.nlr != 4) return hipErrorInvalidValue;
    if (bf) FT_GPN(2);
    else if (g.b_row_scales) FT_GPN(1);
    else if (g.b_transposed) FT_GPN(3);
    else FT_GPN(0);
#undef FT_GPN
#undef FT_GP
  } else if (bf) {
    return hipErrorInvalidValue;
  } else if (g.b_row_scales) {
    hipLaunchKernelGGL(k_gemm<1>, dim3(n), dim3(256), 0, st, g);
  } else if (g.b_transposed) {
    hipLaunchKernelGGL(k_gemm<3>, dim3(n), dim3(256), 0, st, g);
  } else {
    hipLaunchKernelGGL(k_gemm<0>, dim3(n), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace ft
