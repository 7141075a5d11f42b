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
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

namespace {

constexpr int BM = 256, BN = 256, BK = 128;  // BK in 4-bit elements
constexpr int ROWB = BK / 2;                 // 64 bytes per row and step
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
__device__ __forceinline__ uint32_t bload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

// Logical tile index -> tile origin: groups of 4 m-tiles with the n-tiles
// inner, so that consecutive indices share A rows and B columns.
__device__ __forceinline__ void tile_coords(uint32_t lid, uint32_t mt_n, uint32_t nt_n, int64_t& m0,
                                            int64_t& j0) {
  constexpr uint32_t GM = 4;
  const uint32_t grp_sz = GM * nt_n;
  const uint32_t gidx = lid / grp_sz, gfirst = gidx * GM;
  const uint32_t gm = min(GM, mt_n - gfirst);
  const uint32_t in_g = lid - gidx * grp_sz;
  m0 = static_cast<int64_t>(gfirst + in_g % gm) * BM;
  j0 = static_cast<int64_t>(in_g / gm) * BN;
}

// Byte selector for pair_bf16: even lanes keep the low halves (own, then
// neighbour's), odd lanes the high halves (neighbour's, then own).
__device__ __forceinline__ uint32_t pair_sel(int odd) { return odd ? 0x03020706u : 0x05040100u; }

// Round an accumulator pair to bf16 and swap halves with the neighbouring
// lane: accumulator elements e, e+1 of tile column l32 are rows q, q+1; the
// result is row q (even lane) or q+1 (odd lane) at columns l32&~1, +1.
__device__ __forceinline__ uint32_t pair_bf16(float x0, float x1, uint32_t sel) {
  const f32x2 x = {x0, x1};
  const uint32_t w = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  const uint32_t o = static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(w), 0xB1, 0xF, 0xF, false));
  return __builtin_amdgcn_perm(o, w, sel);
}

// ---------------------------------------------------------------------------
// Pipelined persistent kernel, reduction lengths that are a multiple of 128.
constexpr int NST = 4;                      // LDS stages
constexpr int ST_A = BM * ROWB;             // 16 KB of A codes (or lm ranks)
constexpr int ST_B = BN * ROWB;             // 16 KB of B codes (or lo ranks)
constexpr int ST_SA = BM * 4;               // A scale words, one per row
constexpr int ST_SB = 4 * 256;              // B scale words, one 256-byte region per wave
constexpr int ST_BYTES = ST_A + ST_B + ST_SA + ST_SB;
constexpr int OUT_WAVE = 16 * 256;          // per-wave output strip: 16 rows x 128 bf16
// Per wave and stage: 4 + 4 row DMAs and 1 + 1 scale DMAs, issued as two
// halves of 5 (A part, B part).
constexpr int DMA_HALF = 5;
// Global stores of one tile's output per lane (8 strips x 4).
constexpr int STORES = 32;

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

// Fragments and scales of one step: chunk 0 (a0, b0), chunk 1 (a1, b1).
struct Frags {
  u32x4 a0[4], b0[4], a1[4], b1[4];
  uint32_t as[4], bs[4];
};

template <int K> struct MfmaKind { static constexpr int v = K; };   // 0: MXFP4, 1: bf16 ranks

// LR: the tiles start with two rank steps (64 padded ranks).  An odd
// number of reduction steps is padded by one step whose loads are pushed
// out of range: zero codes and zero scale bytes add exactly 0, and every
// tile then has an even number of steps for the even/odd registers.
// BMODE 0: b has one scale per 32x32 tile (the method's weight).  BMODE 1:
// b has 1x32 row blocks like a (group-wise weights): its scale words are
// loaded and read per row, as a's are.  BMODE 2 (BF): the main product is
// bf16 x bf16 (a16, b16): its steps are rank-kind steps of 32 reduction
// elements (64 bytes of a row, as a 4-bit step), and no scales are loaded.
template <bool LR, int BMODE>
__global__ __launch_bounds__(256, 1) void k_gemm_pipe(const GemmArgs g) {
  constexpr bool BF = BMODE == 2, BROW = BMODE == 1;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * ST_BYTES + 4 * OUT_WAVE];

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;

  const uint32_t mt_n = static_cast<uint32_t>((M + BM - 1) / BM);
  const uint32_t nt_n = static_cast<uint32_t>((NOUT + BN - 1) / BN);
  const uint32_t ntiles = mt_n * nt_n, G = gridDim.x, bid = blockIdx.x;
  const uint32_t full = ntiles / G, nlast = ntiles % G;
  const uint32_t my_tiles = full + (bid < nlast ? 1u : 0u);
  constexpr int NLR = LR ? 2 : 0;
  const int nks_real = static_cast<int>(BF ? RED / 32 : RED / BK);
  const int nks = nks_real + (nks_real & 1);             // padded to even
  const int spt = nks + NLR;                             // steps per tile
  const int total = static_cast<int>(my_tiles) * spt;
  const bool tiny = spt < 3;                              // see the barrier waits

  // k-th tile of this workgroup: rounds of G tiles, XCD-compact in a round
  auto tile_of = [&](uint32_t k, int64_t& m0, int64_t& j0) {
    const uint32_t n_round = k < full ? G : nlast;
    tile_coords(k * G + xcd_remap(bid, n_round), mt_n, nt_n, m0, j0);
  };

  const uint32_t row_bytes = static_cast<uint32_t>(BF ? RED * 2 : RED >> 1);
  const uint32_t row_sc = static_cast<uint32_t>(RED >> 5);
  constexpr uint32_t LR_BYTES = 64 * 2;                  // a padded rank row: 64 bf16
  const auto ra_codes = rsrc(BF ? static_cast<const void*>(g.a16) : g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, BF ? 0 : static_cast<uint64_t>(M) * row_sc);
  const auto rb_codes = rsrc(BF ? static_cast<const void*>(g.b16) : g.b_codes, static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, BF ? 0 : static_cast<uint64_t>(BROW ? NOUT : NOUT >> 5) * row_sc);
  const auto r_lm = rsrc(g.lm, LR ? static_cast<uint64_t>(M) * LR_BYTES : 0);
  const auto r_lo = rsrc(g.lo, LR ? static_cast<uint64_t>(NOUT) * LR_BYTES : 0);

  // Per-lane parts of the DMA source offsets (rows relative to the tile
  // origin; A and B tiles have the same shape).  Instruction q of wave w
  // fills 1 KB of LDS (16 rows of 64 bytes); lane i lands at byte 16 i.
  uint32_t code_row[4], lr_row[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t row = 64 * wave + 16 * q + (lane >> 2), ch = (lane & 3) ^ swz16(row);
    code_row[q] = row * row_bytes + (ch << 4);
    lr_row[q] = row * LR_BYTES + (ch << 4);
  }

  // DMA cursor: the (tile, step) whose A or B half is loaded next, with the
  // tile's base offsets.  A cursors use m0, B cursors j0.
  struct Cursor {
    int gs, s;
    uint32_t k, code, sc, lr;
  };
  auto cursor_tile = [&](Cursor& c, bool is_b) {
    int64_t m0 = 0, j0 = 0;
    if (c.k < my_tiles) tile_of(c.k, m0, j0);
    const uint32_t o = static_cast<uint32_t>(is_b ? j0 : m0);
    c.code = o * row_bytes;
    c.sc = (is_b && !BROW) ? (o >> 5) * row_sc : o * row_sc;
    c.lr = o * LR_BYTES;
  };
  auto cursor_next = [&](Cursor& c, bool is_b) {
    ++c.gs;
    if (++c.s == spt) {
      c.s = 0;
      ++c.k;
      cursor_tile(c, is_b);
    }
  };
  // The uniform part of one half (A or B) of cursor c's step, computed once
  // per half: source, offsets (pushed out of range when the step lies past
  // this workgroup's last tile) and the LDS region.  Each DMA instruction
  // then only adds its lane's row offset.
  struct HalfDma {
    __amdgpu_buffer_rsrc_t rows, sc;
    uint32_t base, sbase;
    uint8_t* dst;        // this wave's rows of the stage's A or B part
    uint8_t* sdst;       // this wave's scale words
    bool lr;
  };
  auto half_dma = [&](const Cursor& c, bool is_b) {
    HalfDma h;
    const bool live = c.gs < total;
    const bool lrs = LR && c.s < NLR;
    const int ks = c.s - NLR;
    h.lr = lrs;
    h.rows = lrs ? (is_b ? r_lo : r_lm) : (is_b ? rb_codes : ra_codes);
    h.sc = is_b ? rb_sc : ra_sc;
    const bool pad = !lrs && ks >= nks_real;                 // the padding step
    h.base = (!live || pad) ? OOB : (lrs ? c.lr + static_cast<uint32_t>(c.s) * 64 : c.code + static_cast<uint32_t>(ks) * 64);
    h.sbase = (BF || !live || lrs || pad) ? OOB : c.sc + static_cast<uint32_t>(ks) * 4;
    uint8_t* st = lds + (c.gs & (NST - 1)) * ST_BYTES;
    h.dst = st + (is_b ? ST_A : 0) + 64 * wave * ROWB;
    h.sdst = is_b ? st + ST_A + ST_B + ST_SA + (BROW ? 64 * wave * 4 : wave * 256)
                  : st + ST_A + ST_B + 64 * wave * 4;
    return h;
  };
  // DMA instruction `item` (0..4) of a half.  Offsets stay below 2^32: lane
  // parts are below 2^31 and OOB is 2^31.
  auto dma = [&](const HalfDma& h, int item, bool is_b) {
    if (item < 4) {
      const uint32_t lane_off = h.lr ? lr_row[item] : code_row[item];
      dma16(h.rows, h.dst + item * 16 * ROWB, lane_off + h.base);
    } else {
      // the scale lane offsets are recomputed from an opaque copy of the
      // thread id at each use: kept in registers across the K loop they were
      // spilled, and each reload's full memory wait drained the pipeline
      uint32_t tl = static_cast<uint32_t>(t);
      asm volatile("" : "+v"(tl));
      if (!is_b || BROW) {
        dma4(h.sc, h.sdst, tl * row_sc + h.sbase);                 // row 64 wave + lane
      } else {
        const uint32_t sb = (tl < 8) ? tl * row_sc : OOB;         // wave 0, lanes 0..7
        dma4(h.sc, h.sdst, sb == OOB ? OOB : sb + h.sbase);
      }
    }
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
  // raw scale words (the lane's byte is selected later by a shift)
  auto read_scales = [&](int buf, uint32_t (&as)[4], uint32_t (&bs)[4]) {
    const uint8_t* st = lds + buf * ST_BYTES;
    const uint32_t* ssa = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B);
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B + ST_SA);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      as[i] = ssa[wm * 128 + i * 32 + l32];
      bs[i] = BROW ? ssb[wn * 128 + i * 32 + l32] : ssb[wn * 4 + i];
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // Output of the finished tile (m0, j0): 8 strips of 16 rows per wave,
  // then the accumulators are cleared for the next tile.
  uint8_t* ostage = lds + NST * ST_BYTES + wave * OUT_WAVE;
  const auto r_out = rsrc(g.out, static_cast<uint64_t>(M) * NOUT * 2);
  // 32-bit output offsets: (M + 256) * NOUT * 2 < 2^31 (host check), so a
  // row past M lands past the end of the buffer and is dropped without a
  // test; only columns past NOUT are masked.
  const uint32_t out_row = static_cast<uint32_t>(NOUT) * 2;
  auto store_tile = [&](int64_t m0, int64_t j0) {
    // lane-dependent addresses are rebuilt for each tile from an opaque copy
    // of the lane id: hoisted out of the tile loop, they stay live across the
    // K loop and push it into scratch
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lgrp = ln >> 5, lodd = ln & 1, ll32 = ln & 31;
    const uint32_t psel = pair_sel(lodd);
    const uint32_t gcol = static_cast<uint32_t>(j0) + wn * 128 + (ln & 15) * 8;
    const uint32_t out_base = gcol < static_cast<uint32_t>(NOUT)
                                  ? (static_cast<uint32_t>(m0) + wm * 128 + (ln >> 4)) * out_row + gcol * 2
                                  : OOB;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // accumulator elements 8h .. 8h+7 are rows 16h .. 16h+15 of tile mt
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t v = pair_bf16(acc[mt][nt][8 * h + 2 * p], acc[mt][nt][8 * h + 2 * p + 1], psel);
            const int row = 8 * (p >> 1) + 4 * lgrp + 2 * (p & 1) + lodd;   // 0 .. 15
            const int sw = (row & 1) | (((row >> 2) & 1) << 1);             // 64-byte segment swizzle
            const int col = nt * 32 + (ll32 & ~1);
            *reinterpret_cast<uint32_t*>(ostage + row * 256 + (((col >> 5) ^ sw) << 6) + (col & 31) * 2) = v;
          }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = e * 64 + ln, row = idx >> 4, c16 = idx & 15;
          const int sw = (row & 1) | (((row >> 2) & 1) << 1);
          const u32x4 v = lds_read_b128(ostage + row * 256 + ((((c16 >> 2) ^ sw) << 6) | ((c16 & 3) << 4)));
          const uint32_t off = out_base == OOB ? OOB : out_base + static_cast<uint32_t>(mt * 32 + 16 * h + 4 * e) * out_row;
          __builtin_amdgcn_raw_buffer_store_b128(v, r_out, static_cast<int>(off), 0, 2);
        }
      }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  };

  // ---- prologue: stages 0..2 and the A half of stage 3
  Cursor ca{0, 0, 0, 0, 0, 0}, cb{0, 0, 0, 0, 0, 0};
  cursor_tile(ca, false);
  cursor_tile(cb, true);
  for (int s = 0; s < NST - 1; ++s) {
    const HalfDma ha = half_dma(ca, false), hb = half_dma(cb, true);
#pragma unroll
    for (int item = 0; item < DMA_HALF; ++item) dma(ha, item, false);
#pragma unroll
    for (int item = 0; item < DMA_HALF; ++item) dma(hb, item, true);
    cursor_next(ca, false);
    cursor_next(cb, true);
  }
  {
    const HalfDma ha = half_dma(ca, false);
#pragma unroll
    for (int item = 0; item < DMA_HALF; ++item) dma(ha, item, false);
    cursor_next(ca, false);
  }
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(5 * DMA_HALF, 0xF));   // this wave's stage 0 landed
  __builtin_amdgcn_s_barrier();                                  // ... and every wave's
  __builtin_amdgcn_sched_barrier(0);
  Frags E, O;
  read_scales(0, E.as, E.bs);
  read_frags(0, 0, E.a0, E.b0);
#pragma unroll
  for (int i = 0; i < 4; ++i) { E.as[i] >>= 8 * grp; E.bs[i] >>= 8 * grp; }
  __builtin_amdgcn_sched_barrier(0);

  int gs = 0;   // global step of this workgroup

  // One step.  Cur holds this step's chunk-0 fragments and scales; Nxt gets
  // the next step's.  DMA
  // order per wave: ..., B half of stage gs+3 (first half of step gs), A
  // half of stage gs+4 (second half), [a tile's 32 output stores after its
  // last step], ...  after_store: one of the last two steps ended a tile.
  // Keeps a half's MFMAs ahead of what follows: without it the compiler may
  // sink these side-effect-free instructions past the barrier and the DMA
  // issues of the step, next to their first use, which serializes the step.
  auto pin_acc = [&]() {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) asm volatile("" : "+a"(acc[a][b]));
  };
  // Empty uses that extend live ranges: the registers an MFMA of the
  // previous half may still read are not reused for values loaded now.
  auto keep4 = [](const u32x4 (&x)[4]) {
    asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  };
  auto keep_s = [](const uint32_t (&x)[4]) {
    asm volatile("" ::"v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
  };
  // The bookkeeping of a step (DMA addresses, fragment and scale reads,
  // scale shifts, cursor advance) is spread between the MFMAs of its two
  // halves, so that it issues while the matrix core is busy instead of
  // leaving it idle between the halves.
  auto step = [&](Frags& Cur, Frags& Nxt, auto kind, bool after_store) {
    constexpr bool RANK = decltype(kind)::v == 1;
    const int buf = gs & (NST - 1);
    const int nbuf = (gs + 1) & (NST - 1);
    auto mma = [&](int i, const u32x4 (&af)[4], const u32x4 (&bf)[4], auto opsel) {
      constexpr int OP = decltype(opsel)::v;
      if constexpr (RANK)
        acc[i >> 2][i & 3] = mfma_bf16_32x32x16(af[i >> 2], bf[i & 3], acc[i >> 2][i & 3]);
      else
        acc[i >> 2][i & 3] = mfma_fp4_32x32x64<OP, OP>(af[i >> 2], bf[i & 3], acc[i >> 2][i & 3],
                                                       Cur.as[i >> 2], Cur.bs[i & 3]);
    };
    const MfmaKind<0> op0;
    const MfmaKind<2> op2;
    // ---- first half: chunk 0 of this step; chunk 1 is read meanwhile
    HalfDma hb;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mma(i, Cur.a0, Cur.b0, op0);
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) {
        hb = half_dma(cb, true);
        read_frags(buf, 1, Cur.a1, Cur.b1);
        keep4(Nxt.a1);
        keep4(Nxt.b1);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i % 3 == 1) {
        dma(hb, i / 3, true);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    // Own loads of stage gs+1 landed (the 4 younger halves, and a tile's
    // stores issued in the last two steps, may be in flight) and own reads
    // of stage gs done; after the barrier the same holds for every wave:
    // stage gs+1 is readable and stage gs reusable.  With fewer than 3
    // steps per tile two store batches can be in that window: drain.
    if (tiny) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    else if (after_store) __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * DMA_HALF + STORES, 0));
    else __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * DMA_HALF, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // ---- second half: chunk 1; the next step's chunk 0 and scales are read
    HalfDma ha;
    uint32_t ras[4], rbs[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mma(i, Cur.a1, Cur.b1, op2);
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) {
        ha = half_dma(ca, false);
        read_scales(nbuf, ras, rbs);
        read_frags(nbuf, 0, Nxt.a0, Nxt.b0);
        keep4(Cur.a0);
        keep4(Cur.b0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i % 3 == 1) {
        dma(ha, i / 3, false);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 8) {
        cursor_next(cb, true);
        cursor_next(ca, false);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (i == 12) {
#pragma unroll
        for (int j = 0; j < 4; ++j) { Nxt.as[j] = ras[j] >> (8 * grp); Nxt.bs[j] = rbs[j] >> (8 * grp); }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    pin_acc();
    __builtin_amdgcn_sched_barrier(0);
    keep_s(Cur.as);
    keep_s(Cur.bs);
    keep_s(Nxt.as);
    keep_s(Nxt.bs);
    ++gs;
    __builtin_amdgcn_sched_barrier(0);
  };

  const MfmaKind<0> fp4;
  const MfmaKind<1> rank;
  for (uint32_t k = 0; k < my_tiles; ++k) {
    const bool after = k > 0;
    if constexpr (LR) {
      step(E, O, rank, after);
      step(O, E, rank, after);
      for (int p = 0; p < nks / 2; ++p) {
        if constexpr (BF) {
          step(E, O, rank, false);
          step(O, E, rank, false);
        } else {
          step(E, O, fp4, false);
          step(O, E, fp4, false);
        }
      }
    } else {
      for (int p = 0; p < nks / 2; ++p) {
        if constexpr (BF) {
          step(E, O, rank, after && p == 0);
          step(O, E, rank, after && p == 0);
        } else {
          step(E, O, fp4, after && p == 0);
          step(O, E, fp4, after && p == 0);
        }
      }
    }
    int64_t m0, j0;
    tile_of(k, m0, j0);
    store_tile(m0, j0);
  }
  // DMAs into LDS must land before the workgroup can end
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0xF));
}

// ---------------------------------------------------------------------------
// Register-staged kernel for reduction lengths that are a multiple of 32
// but not of 128: the last step is partial, so scale bytes are fetched one
// by one and code chunks past the row end read as zero.  Two LDS buffers;
// the loads of step k+1 are in flight while step k runs.  The rank part
// comes first, from fragments loaded straight from the padded rank rows.
template <bool BROW>
__global__ __launch_bounds__(256, 1) void k_gemm(const GemmArgs g) {
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
  const int nks = static_cast<int>((RED + BK - 1) / BK);

  const auto ra_codes = rsrc(g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, static_cast<uint64_t>(M) * row_sc);
  const auto rb_codes = rsrc(g.b_codes, static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, static_cast<uint64_t>(BROW ? NOUT : NOUT >> 5) * row_sc);

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
    b_off[i] = static_cast<uint32_t>(j0 + row) * row_bytes + ch * 16;
  }
  uint32_t sa_off[4], sb_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sa_off[i] = static_cast<uint32_t>(m0 + wm * 128 + i * 32 + l32) * row_sc;
    sb_off[i] = static_cast<uint32_t>(BROW ? j0 + wn * 128 + i * 32 + l32 : (j0 + wn * 128 + i * 32) >> 5) * row_sc;
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

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool bf = g.a16 != nullptr;
  if ((g.RED & 127) == 0 || (bf && (g.RED & 31) == 0)) {
    const int cus = cu_count();
    if (cus <= 0) return hipErrorInvalidDevice;
    const uint32_t grid = n < static_cast<uint32_t>(cus) ? n : static_cast<uint32_t>(cus);
#define FT_GP(LR, MODE) hipLaunchKernelGGL((k_gemm_pipe<LR, MODE>), dim3(grid), dim3(256), 0, st, g)
    if (bf) {
      if (g.nlr > 0) FT_GP(true, 2); else FT_GP(false, 2);
    } else if (g.b_row_scales) {
      if (g.nlr > 0) FT_GP(true, 1); else FT_GP(false, 1);
    } else {
      if (g.nlr > 0) FT_GP(true, 0); else FT_GP(false, 0);
    }
#undef FT_GP
  } else if (bf) {
    return hipErrorInvalidValue;
  } else if (g.b_row_scales) {
    hipLaunchKernelGGL(k_gemm<true>, dim3(n), dim3(256), 0, st, g);
  } else {
    hipLaunchKernelGGL(k_gemm<false>, dim3(n), dim3(256), 0, st, g);
  }
  return hipGetLastError();
}

}  // namespace ft
