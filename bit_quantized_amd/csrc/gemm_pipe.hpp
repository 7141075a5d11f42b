// The pipelined persistent MXFP4 GEMM kernel (k_gemm_pipe) and its helpers,
// shared by gemm.hip (the plain products) and gemm_mlp.hip (the MLP-fused
// epilogues), so that the two sets of instantiations compile in parallel.
// The design is described at the top of gemm.hip.
#pragma once

#include "ft_device.hpp"
#include "ft_kernels.h"
#include "lora_block.hpp"

#include <algorithm>

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

// The LDS destination of a DMA goes in as an opaque (wave-uniform) LDS
// address.  The compiler then does not track the DMA's LDS write, and adds
// no memory wait of its own before the LDS reads of the stages, which the
// kernel orders itself (explicit vmcnt waits and barriers per stage).  With
// the destination visible it drains every DMA in flight (vmcnt(0)) before
// each ds_read_b64_tr_b4.
__device__ __forceinline__ FT_LDS void* opaque_lds(uint8_t* p) {
  uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((FT_LDS uint8_t*)(p)));
  asm volatile("" : "+s"(a));
  return (FT_LDS void*)(static_cast<uintptr_t>(a));
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, opaque_lds(lds), 16, (int)off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, opaque_lds(lds), 4, (int)off, 0, 0, 0);
}

// Fragments and scales of one step: chunk 0 (a0, b0), chunk 1 (a1, b1).
struct Frags {
  u32x4 a0[4], b0[4], a1[4], b1[4];
  uint32_t as[4], bs[4];
};

template <int K> struct MfmaKind { static constexpr int v = K; };   // 0: MXFP4, 1: bf16 ranks
template <bool B> struct Flag { static constexpr bool v = B; };

// NLR_: the tiles start with NLR_ rank steps (32 NLR_ padded ranks: 2 or 4
// steps, rank rows of 64 or 128 bf16).  An odd
// number of reduction steps is padded by one step whose loads are pushed
// out of range: zero codes and zero scale bytes add exactly 0, and every
// tile then has an even number of steps for the even/odd registers.
// BMODE 0: b has one scale per 32x32 tile (the method's weight).  BMODE 1:
// b has 1x32 row blocks like a (group-wise weights): its scale words are
// loaded and read per row, as a's are.  BMODE 2 (BF): the main product is
// bf16 x bf16 (a16, b16): its steps are rank-kind steps of 32 reduction
// elements (64 bytes of a row, as a 4-bit step), and no scales are loaded.
// BMODE 3 (BT): b is the 32x32-tile weight stored [RED, NOUT/2] (the dgrad
// reading the forward's weight): a 4-bit step stages 128 reduction rows x
// 128 bytes (256 output columns) in LDS, 16-byte slots swizzled by
// (row >> 1) & 7, and each operand fragment is two ds_read_b64_tr_b4 (16
// reduction rows of 16 columns per 16-lane group), conflict-free per half
// wave; the tile scales of a step are 4 runs of 8 bytes (one per reduction
// block, strided by NOUT/32), loaded as 3 aligned words each and turned
// into per-column words (byte j = reduction block j) by byte permutes.
// A workgroup barrier for LDS data passed between waves: this wave's LDS
// accesses complete, then s_barrier; the memory clobber keeps the compiler
// from moving memory accesses across it.  (No wait on vector memory: the
// loads and stores in flight stay in flight.)
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// The adapter gradients beside a transposed-weight product (GemmArgs::
// lora_a, lora_b): workgroup j of the side_wgs after the product's takes
// dA's 64-column blocks j, j + side_wgs, ... over every 512-token chunk (no
// partials: each block's chunks are added in chunk order and rounded once,
// the bits the adapter-gradient kernels give), in the LDS the product's
// stages would use; then every side thread adds its share of the column
// quads of dB from the quantizer's partials (lora_b.nchunk of them), in
// chunk order.  RG rank groups of 16; X as is (ACT 0: with GELU recomputed
// on X the product's own registers spilled, so a layer with a GELU input
// runs its adapter gradients as their own launch).
template <int RG>
__device__ __forceinline__ void side_lora_rg(const GemmArgs& g, uint8_t* lds) {
  using namespace lora_dev;
  static_assert(2 * MS * PB * 2 + MC * small_pitch<RG>() * 2 <= NST * ST_BYTES,
                "the adapter-gradient work item fits in the stages");
  auto* bigL = reinterpret_cast<uint16_t (*)[MS * PB]>(lds);
  uint16_t* smL = reinterpret_cast<uint16_t*>(lds + 2 * MS * PB * 2);
  const uint32_t j = blockIdx.x - g.gemm_wgs;
  const uint32_t nib = static_cast<uint32_t>((g.lora_a.I + IB - 1) / IB);
  for (uint32_t cb = j; cb < nib; cb += g.side_wgs) lora_column_block<RG, 0>(g.lora_a, cb, bigL, smL);
}
__device__ __forceinline__ void side_lora(const GemmArgs& g, uint8_t* lds) {
  const int rg = (g.lora_a.rl + 15) / 16;
  switch (rg) {
    case 1: side_lora_rg<1>(g, lds); break;
    case 2: side_lora_rg<2>(g, lds); break;
    case 3: side_lora_rg<3>(g, lds); break;
    default: side_lora_rg<4>(g, lds); break;
  }
  if (g.lora_b.nchunk > 0) {
    const uint32_t j = blockIdx.x - g.gemm_wgs;
    const uint64_t nq = static_cast<uint64_t>(g.lora_b.rl) * (g.lora_b.I / 4);
    for (uint64_t idx = static_cast<uint64_t>(j) * 256 + threadIdx.x; idx < nq;
         idx += static_cast<uint64_t>(g.side_wgs) * 256)
      lora_dev::lora_reduce_quad(g.lora_b, rg * 16, idx);
  }
}

// EPI > 0: the MLP-fused epilogue (GemmArgs::e_codes): EPI 1..5 the
// forward (EPI - 1 rank groups of 16 in the second linear's
// down-projection), 6..10 the backward mirror (EPI - 6 groups in the first
// linear's V1).
template <int NLR_, int BMODE, int EPI = 0>
__global__ __launch_bounds__(256, 1) void k_gemm_pipe(const GemmArgs g) {
  constexpr bool LR = NLR_ > 0;
  constexpr bool BF = BMODE == 2, BROW = BMODE == 1, BT = BMODE == 3;
  __shared__ __attribute__((aligned(16))) uint8_t lds[NST * ST_BYTES];
  // the output strips: a separate LDS object (the stages are DMA targets)
  __shared__ __attribute__((aligned(16))) uint8_t lds_out[4 * OUT_WAVE];

  // the workgroups past the product's compute the adapter gradients
  // (transposed-weight products only; the host sets side_wgs)
  constexpr bool SIDE = BT && EPI == 0;
  if constexpr (SIDE) {
    if (g.side_wgs > 0 && blockIdx.x >= g.gemm_wgs) {
      side_lora(g, lds);
      return;
    }
  }

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, grp = lane >> 5;
  const int64_t M = g.M, RED = g.RED, NOUT = g.NOUT;

  const uint32_t mt_n = static_cast<uint32_t>((M + BM - 1) / BM);
  const uint32_t nt_n = static_cast<uint32_t>((NOUT + BN - 1) / BN);
  // Split reduction (few output tiles): unit u is tile u / S over steps
  // (u % S) * nks .. + nks of the reduction, its fp32 sums stored to
  // g.part; S = 1 otherwise (a unit is a whole tile).
  // (only without rank steps: a split launch leaves the rank part to the
  // kernel that adds the splits)
  const uint32_t S = (!LR && EPI == 0 && g.splits > 1) ? static_cast<uint32_t>(g.splits) : 1u;
  const uint32_t G = SIDE && g.side_wgs > 0 ? g.gemm_wgs : gridDim.x;
  const uint32_t ntiles = mt_n * nt_n * S, bid = blockIdx.x;
  const uint32_t full = ntiles / G, nlast = ntiles % G;
  const uint32_t my_tiles = full + (bid < nlast ? 1u : 0u);
  constexpr int NLR = NLR_;                              // rank steps: 0, 2 or 4
  const int nks_real = static_cast<int>(BF ? RED / 32 : RED / BK);
  const int nks = S > 1 ? 2 * g.split_pairs             // steps per unit; a split past
                        : nks_real + (nks_real & 1);     // the end loads zeros; padded to even
  const int spt = nks + NLR;                             // steps per tile
  const int total = static_cast<int>(my_tiles) * spt;
  const bool tiny = spt < 3;                              // see the barrier waits

  // k-th tile of this workgroup: rounds of G tiles, XCD-compact in a round;
  // ko: the unit's first reduction step
  auto tile_of = [&](uint32_t k, int64_t& m0, int64_t& j0, int& ko) {
    const uint32_t n_round = k < full ? G : nlast;
    const uint32_t u = k * G + xcd_remap(bid, n_round);
    tile_coords(u / S, mt_n, nt_n, m0, j0);
    ko = static_cast<int>(u % S) * nks;
  };

  const uint32_t row_bytes = static_cast<uint32_t>(BF ? RED * 2 : RED >> 1);
  const uint32_t row_sc = static_cast<uint32_t>(RED >> 5);
  constexpr uint32_t LR_BYTES = NLR * 64;                // a padded rank row: 32 NLR bf16
  const auto ra_codes = rsrc(BF ? static_cast<const void*>(g.a16) : g.a_codes, static_cast<uint64_t>(M) * row_bytes);
  const auto ra_sc = rsrc(g.a_scales, BF ? 0 : static_cast<uint64_t>(M) * row_sc);
  // BT: b rows are reduction rows of NOUT/2 bytes; its scale grid is
  // [RED/32, NOUT/32], read in whole aligned words (the size is rounded up
  // to a word so the last bytes are not cut off by the range check)
  const uint32_t bt_row = static_cast<uint32_t>(NOUT >> 1), bt_ks = static_cast<uint32_t>(NOUT >> 5);
  const auto rb_codes = rsrc(BF ? static_cast<const void*>(g.b16) : g.b_codes,
                             BT ? static_cast<uint64_t>(RED) * bt_row : static_cast<uint64_t>(NOUT) * row_bytes);
  const auto rb_sc = rsrc(g.b_scales, BF ? 0
                                      : BT ? ((static_cast<uint64_t>(RED >> 5) * bt_ks + 3) & ~uint64_t(3))
                                           : static_cast<uint64_t>(BROW ? NOUT : NOUT >> 5) * row_sc);
  const auto r_lm = rsrc(g.lm, LR ? static_cast<uint64_t>(M) * LR_BYTES : 0);
  // BT: lo is given as nibble planes, [2 rank steps x 128 rows, NOUT/2]
  // bytes (see half_dma)
  const auto r_lo = rsrc(g.lo, !LR ? 0 : BT ? static_cast<uint64_t>(128 * NLR) * bt_row
                                         : static_cast<uint64_t>(NOUT) * LR_BYTES);

  // Per-lane parts of the DMA source offsets (rows relative to the tile
  // origin; A and B tiles have the same shape).  Instruction q of wave w
  // fills 1 KB of LDS (16 rows of 64 bytes); lane i lands at byte 16 i.
  // Only lane constants are kept; the rest of each offset is wave-uniform.
  //  - rows 64 wave + 16 q + lane / 4: the chunk swizzle (row >> 2) & 3 is
  //    (lane >> 4) for every q, so lane part (lane >> 2) * pitch + chunk;
  //  - stored rows 32 wave + 8 q + lane / 8 of a BT 4-bit step of b: the
  //    slot swizzle (row >> 1) & 7 is (lane >> 4) ^ 4 (q & 1), so two lane
  //    parts, for even and odd q;
  //  - fragment reads (read_frags_bt): see there.
  // (Per-instruction offsets held across the K loop were spilled at four
  // rank steps, and each reload's memory wait drained the pipeline.)
  //  - row-major fragment reads (read_frags_rows): row 32 i + l32 of a
  //    wave's half, chunk (2 c + grp) ^ ((l32 >> 2) & 3), which is c = 0's
  //    with byte bit 5 toggled.
  uint32_t bt_ca, bt_cl, bt_p[2] = {0, 0}, bt_fb = 0, bt_lc;
  {
    const uint32_t ch = (lane & 3) ^ (lane >> 4);
    bt_ca = (lane >> 2) * row_bytes + (ch << 4);
    bt_cl = (lane >> 2) * LR_BYTES + (ch << 4);
    bt_lc = l32 * ROWB + ((grp ^ ((l32 >> 2) & 3)) << 4);
  }
  if constexpr (BT) {
    const uint32_t sl = (lane & 7) ^ (lane >> 4);
    bt_p[0] = (lane >> 3) * bt_row + (sl << 4);
    bt_p[1] = (lane >> 3) * bt_row + ((sl ^ 4) << 4);
    const uint32_t q = lane & 15, hf = (lane >> 4) & 1, sw = (q >> 1) & 7;
    bt_fb = (32 * (lane >> 5) + q) * 128 + 8 * hf + (((4 * wn) ^ (sw & 4)) << 4) + ((sw & 3) << 4);
  }

  // DMA cursor: the (tile, step) whose A or B half is loaded next, with the
  // tile's base offsets.  A cursors use m0, B cursors j0.
  struct Cursor {
    int gs, s, ko;
    uint32_t k, code, sc, lr;
  };
  auto cursor_tile = [&](Cursor& c, bool is_b) {
    int64_t m0 = 0, j0 = 0;
    c.ko = 0;
    if (c.k < my_tiles) tile_of(c.k, m0, j0, c.ko);
    const uint32_t o = static_cast<uint32_t>(is_b ? j0 : m0);
    if (BT && is_b) {
      // the tile's first byte column and scale column of every stored row
      c.code = o >> 1;
      c.sc = o >> 5;
    } else {
      c.code = o * row_bytes;
      c.sc = (is_b && !BROW) ? (o >> 5) * row_sc : o * row_sc;
    }
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
    const int ks = c.s - NLR + c.ko;                         // reduction step
    h.lr = lrs;
    h.rows = lrs ? (is_b ? r_lo : r_lm) : (is_b ? rb_codes : ra_codes);
    h.sc = is_b ? rb_sc : ra_sc;
    const bool pad = !lrs && ks >= nks_real;                 // the padding step
    const bool bt = BT && is_b;
    // a 4-bit step advances 128 reduction elements: 64 bytes along a row, or
    // (BT) 128 stored rows, and 4 scale bytes along a row or (BT) 4 rows of
    // the scale grid
    // BT b: rank steps too read 128 stored rows (of lo's nibble planes)
    const uint32_t kstep = bt ? static_cast<uint32_t>(lrs ? c.s : ks) * 128 * bt_row
                              : static_cast<uint32_t>(ks) * 64;
    const uint32_t sstep = bt ? static_cast<uint32_t>(ks) * 4 * bt_ks : static_cast<uint32_t>(ks) * 4;
    h.base = (!live || pad) ? OOB
             : (lrs && !bt) ? c.lr + static_cast<uint32_t>(c.s) * 64 : c.code + kstep;
    h.sbase = (BF || !live || lrs || pad) ? OOB : c.sc + sstep;
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
      uint32_t lane_off;
      if constexpr (BT) {
        // BT 4-bit step of b: stored row 32 wave + 8 item + lane / 8 (1 KB =
        // 8 rows of 128 bytes per instruction), physical slot lane % 8
        // holding logical slot (lane % 8) ^ ((row >> 1) & 7); otherwise as
        // above.  Lane constants plus a uniform part, one selected: no branch.
        uint32_t tp = bt_p[item & 1], ca = bt_ca, cl = bt_cl;
        asm volatile("" : "+v"(tp), "+v"(ca), "+v"(cl));
        const uint32_t t_off = tp + static_cast<uint32_t>(32 * wave + 8 * item) * bt_row;
        const uint32_t r_off = h.lr ? cl + static_cast<uint32_t>(64 * wave + 16 * item) * LR_BYTES
                                    : ca + static_cast<uint32_t>(64 * wave + 16 * item) * row_bytes;
        lane_off = is_b ? t_off : r_off;
      } else {
        uint32_t ca = bt_ca, cl = bt_cl;
        asm volatile("" : "+v"(ca), "+v"(cl));
        lane_off = h.lr ? cl + static_cast<uint32_t>(64 * wave + 16 * item) * LR_BYTES
                        : ca + static_cast<uint32_t>(64 * wave + 16 * item) * row_bytes;
      }
      dma16(h.rows, h.dst + item * 16 * ROWB, lane_off + h.base);
    } else {
      // the scale lane offsets are recomputed from an opaque copy of the
      // thread id at each use: kept in registers across the K loop they were
      // spilled, and each reload's full memory wait drained the pipeline
      uint32_t tl = static_cast<uint32_t>(t);
      asm volatile("" : "+v"(tl));
      if (!is_b || BROW) {
        dma4(h.sc, h.sdst, tl * row_sc + h.sbase);                 // row 64 wave + lane
      } else if constexpr (BT) {
        // wave 0, lanes 4 j + d (d < 3): word d of the run of reduction
        // block j, from the aligned word at or below the run's start
        const uint32_t j = tl >> 2, d = tl & 3;
        const uint32_t sb = (tl < 16 && d < 3) ? ((j * bt_ks) & ~3u) + 4 * d : OOB;
        dma4(h.sc, h.sdst, sb == OOB ? OOB : sb + h.sbase);
      } else {
        const uint32_t sb = (tl < 8) ? tl * row_sc : OOB;         // wave 0, lanes 0..7
        dma4(h.sc, h.sdst, sb == OOB ? OOB : sb + h.sbase);
      }
    }
  };
  // The lane part comes from an opaque copy of a lane constant: the
  // compiler otherwise precomputes an address per fragment and chunk, and
  // spills them.
  auto read_frags_rows = [&](int buf, int c, u32x4 (&af)[4], u32x4 (&bf)[4], bool with_b) {
    uint32_t lc = bt_lc;
    asm volatile("" : "+v"(lc));
    const uint32_t lcc = lc ^ (32u * c);
    const uint32_t base = static_cast<uint32_t>(buf * ST_BYTES + wm * 128 * ROWB) + lcc;
#pragma unroll
    for (int i = 0; i < 4; ++i) af[i] = lds_read_b128(lds + base + i * 32 * ROWB);
    if (BT || !with_b) return;
    const uint32_t bbase = static_cast<uint32_t>(buf * ST_BYTES + ST_A + wn * 128 * ROWB) + lcc;
#pragma unroll
    for (int i = 0; i < 4; ++i) bf[i] = lds_read_b128(lds + bbase + i * 32 * ROWB);
  };
  // BT, a 4-bit step: the b fragments of chunk c from the stored reduction
  // rows.  Lane (column half hf = bit 4, reduction group grp, q = lane % 16)
  // addresses reduction row 64 c + 32 grp + 16 h + q at the 8 bytes of
  // columns 16 hf .. 16 hf + 15 of its 32-column tile; the transposing read
  // hands lane q of each 16-lane group those 16 rows of column q, so two
  // reads (h = 0, 1) give a lane its 32 reduction values in nibble order.
  // The slot of column tile i is (4 wn + i) ^ sw, sw = (row >> 1) & 7 =
  // (q >> 1) & 7 for every row read, = ((4 wn) ^ (sw & 4)) | (i ^ (sw & 3)):
  // with the lane constant bt_fb (holding the i = 0 slot) and a uniform part
  // that is a multiple of 256, tile i's address is (uniform + bt_fb) ^ 16 i.
  // Each address is one integer offset from the LDS array: longer address
  // chains lose the array's alias information on the way to the
  // memory-wait pass, which then drains every DMA in flight before the read.
  auto read_frags_bt = [&](int buf, int c, u32x4 (&bf)[4]) {
    uint32_t fb = bt_fb;
    asm volatile("" : "+v"(fb));
    const uint32_t rb = static_cast<uint32_t>(buf * ST_BYTES + ST_A + 64 * c * 128) + fb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t a = rb ^ (16u * i);
      asm volatile("" : "+v"(a));
      const u32x2 lo = lds_read_tr4(lds + a);
      const u32x2 hi = lds_read_tr4(lds + a + 16 * 128);
      bf[i] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // Fragments of chunk c of a step; bt (a Flag): b read transposed (every
  // BT step: a rank step's lo comes as nibble planes that this read turns
  // into bf16 fragments).
  auto read_frags = [&](int buf, int c, u32x4 (&af)[4], u32x4 (&bf)[4], auto bt) {
    constexpr bool tr = BT && decltype(bt)::v;
    read_frags_rows(buf, c, af, bf, !tr);
    if constexpr (tr) read_frags_bt(buf, c, bf);
  };
  // raw scale words (the lane's byte is selected later by a shift).  BT:
  // the b words come from load_scales_bt / shuffle_scales_bt below.
  auto read_scales = [&](int buf, uint32_t (&as)[4], uint32_t (&bs)[4]) {
    const uint8_t* st = lds + buf * ST_BYTES;
    const uint32_t* ssa = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B);
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(st + ST_A + ST_B + ST_SA);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      as[i] = ssa[wm * 128 + i * 32 + l32];
      if constexpr (!BT) bs[i] = BROW ? ssb[wn * 128 + i * 32 + l32] : ssb[wn * 4 + i];
    }
  };
  // BT b scales in two parts, the LDS reads issued a few MFMAs ahead of the
  // byte shuffles that use them.  Run j (reduction block j of the step)
  // holds the scale bytes of the tile's 8 column blocks from byte
  // (j * NOUT/32) % 4 of its 3 words (words 4 j .. 4 j + 2 of the region):
  // load the two words around this wave's 4 column tiles, then
  auto load_scales_bt = [&](int buf, uint32_t (&raw)[8]) {
    const uint32_t* ssb = reinterpret_cast<const uint32_t*>(lds + buf * ST_BYTES + ST_A + ST_B + ST_SA);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      raw[2 * j] = ssb[4 * j + wn];
      raw[2 * j + 1] = ssb[4 * j + wn + 1];
    }
  };
  // ... align each run's 4 bytes and transpose the 4x4 bytes: bs[i] byte j =
  // scale of (reduction block j, column tile i).  The byte offsets come
  // from an opaque copy of NOUT/32 at each use (hoisted out of the loop
  // they cost scalar registers the kernel does not have).
  auto shuffle_scales_bt = [&](const uint32_t (&raw)[8], uint32_t (&bs)[4]) {
    uint32_t ksc = bt_ks;
    asm volatile("" : "+s"(ksc));
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = __builtin_amdgcn_alignbyte(raw[2 * j + 1], raw[2 * j], (j * ksc) & 3);
    const uint32_t l01 = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t h01 = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t l23 = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t h23 = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    bs[0] = __builtin_amdgcn_perm(l23, l01, 0x05040100u);
    bs[1] = __builtin_amdgcn_perm(l23, l01, 0x07060302u);
    bs[2] = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
    bs[3] = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
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
  uint8_t* ostage = lds_out + wave * OUT_WAVE;
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

  // MLP fusion: the tile's h strips as above, and from each the second
  // linear's input a = gelu(h), computed by the fused quantizer's own
  // activation function from the same bf16 values (so the same bits):
  //   - quantized in 1x32 row blocks where each strip is read back: 4
  //     consecutive lanes hold one block (quad DPP amax), 4 code bytes per
  //     lane and one scale byte per block go out as buffer stores;
  //   - written back over the strip, where all four waves' strips then hold
  //     the 16 rows x 256 columns of a for the down-projection: wave wn
  //     takes rank groups wn EGW .. wn EGW + EGW - 1 of D2 over all 256
  //     columns (16x16x32 bf16 MFMAs; D2's fragments for the tile are
  //     loaded once, before the first strip) and stores its fp32 sums into
  //     the quantizer's partial slab of these rows and this column split.
  // Two barriers per strip: the strips are complete before they are read
  // across waves, and read before the next strip overwrites them.
  // The backward mirror (EACT 2, the dgrad of the second linear): the
  // strips hold dX2, the epilogue reads the matching rows of h (one strip
  // ahead), writes dY1 = bf16(dX2 gelu'(h)) as the output instead of dX2,
  // and quantizes and projects dY1 for the first linear's backward the same
  // way (its V1 in place of D2).
  constexpr int ENRG = EPI > 0 ? (EPI - 1) % 5 : 0;
  constexpr int EACT = EPI > 5 ? 2 : 1;
  constexpr int EGW = (ENRG + 1) / 2;
  auto store_tile_mlp = [&](int64_t m0, int64_t j0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int lgrp = ln >> 5, lodd = ln & 1, ll32 = ln & 31;
    const uint32_t psel = pair_sel(lodd);
    const uint32_t gcol = static_cast<uint32_t>(j0) + wn * 128 + (ln & 15) * 8;
    const bool col_ok = gcol < static_cast<uint32_t>(NOUT);
    const uint32_t srow0 = static_cast<uint32_t>(m0) + wm * 128;
    const uint32_t out_base = col_ok ? (srow0 + (ln >> 4)) * out_row + gcol * 2 : OOB;
    const uint32_t cpr = static_cast<uint32_t>(NOUT >> 1), spr = static_cast<uint32_t>(NOUT >> 5);
    const auto r_ec = rsrc(g.e_codes, static_cast<uint64_t>(M) * cpr);
    const auto r_es = rsrc(g.e_scales, static_cast<uint64_t>(M) * spr);
    const uint32_t nrb = static_cast<uint32_t>((M + 63) >> 6);
    const auto r_ep = rsrc(g.e_part, static_cast<uint64_t>(nt_n) * nrb * 4 * ENRG * 1024);
    // D2 fragments: rank 16 (wn EGW + gi) + ln % 16, columns j0 + 32 ks +
    // 8 (ln / 16) .. +7; zero past the ranks and columns
    u32x4 bfr[EGW > 0 ? EGW : 1][8];
    if constexpr (ENRG > 0) {
      const RankRows& p = g.e_pr;
      const auto rp0 = rsrc(p.p0, static_cast<uint64_t>(p.r0) * p.ld * 2);
      const auto rp1 = rsrc(p.p1, static_cast<uint64_t>(p.r1) * p.ld * 2);
#pragma unroll
      for (int gi = 0; gi < EGW; ++gi)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const int r = 16 * (wn * EGW + gi) + (ln & 15);
          const uint32_t c = static_cast<uint32_t>(j0) + 32 * ks + 8 * (ln >> 4);
          const bool ok = r < g.e_R && c < static_cast<uint32_t>(NOUT);
          const uint32_t o0 = ok && r < p.r0 ? static_cast<uint32_t>((r * p.ld + c) * 2) : OOB;
          const uint32_t o1 = ok && r >= p.r0 ? static_cast<uint32_t>(((r - p.r0) * p.ld + c) * 2) : OOB;
          bfr[gi][ks] = bload128(rp0, o0) | bload128(rp1, o1);
        }
    }
    // h of strip (mt, hh), chunk e: the output's own offsets ([M, NOUT] bf16)
    const auto r_h = rsrc(g.e_h, EACT == 2 ? static_cast<uint64_t>(M) * NOUT * 2 : 0);
    auto strip_off = [&](int mt, int hh, int e) {
      return out_base == OOB ? OOB : out_base + static_cast<uint32_t>(mt * 32 + 16 * hh + 4 * e) * out_row;
    };
    u32x4 hcur[EACT == 2 ? 4 : 1], hnxt[EACT == 2 ? 4 : 1];
    if constexpr (EACT == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hcur[e] = bload128(r_h, strip_off(0, 0, e));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t srow = srow0 + 32 * mt + 16 * h;     // the strip's first row
        if constexpr (EACT == 2) {
          // the next strip's h, in flight while this one is worked
          const int sn = 2 * mt + h + 1;
          if (sn < 8) {
#pragma unroll
            for (int e = 0; e < 4; ++e) hnxt[e] = bload128(r_h, strip_off(sn >> 1, sn & 1, e));
          }
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t v = pair_bf16(acc[mt][nt][8 * h + 2 * p], acc[mt][nt][8 * h + 2 * p + 1], psel);
            const int row = 8 * (p >> 1) + 4 * lgrp + 2 * (p & 1) + lodd;
            const int sw = (row & 1) | (((row >> 2) & 1) << 1);
            const int col = nt * 32 + (ll32 & ~1);
            *reinterpret_cast<uint32_t*>(ostage + row * 256 + (((col >> 5) ^ sw) << 6) + (col & 31) * 2) = v;
          }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = e * 64 + ln, row = idx >> 4, c16 = idx & 15;
          const int sw = (row & 1) | (((row >> 2) & 1) << 1);
          uint8_t* sp = ostage + row * 256 + ((((c16 >> 2) ^ sw) << 6) | ((c16 & 3) << 4));
          const u32x4 v = lds_read_b128(sp);
          const uint32_t off = strip_off(mt, h, e);
          u32x4 av;
          if constexpr (EACT == 2) {
            av = act_bf16x8<2>(v, hcur[e]);
            __builtin_amdgcn_raw_buffer_store_b128(av, r_out, static_cast<int>(off), 0, 2);
          } else {
            __builtin_amdgcn_raw_buffer_store_b128(v, r_out, static_cast<int>(off), 0, 2);
            av = act_bf16x8<1>(v, v);
          }
          const uint32_t m = max_u16x2(max_u16x2(abs_bf16x2(av[0]), abs_bf16x2(av[1])),
                                       max_u16x2(abs_bf16x2(av[2]), abs_bf16x2(av[3])));
          uint32_t am = hmax_u16x2(m);
          am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
          am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
          const uint32_t sc8 = e8m0_from_amax_bits(am);
          const uint32_t code = encode8(av[0], av[1], av[2], av[3], e8m0_to_f32(sc8));
          const uint32_t grow = srow + row;
          __builtin_amdgcn_raw_buffer_store_b32(code, r_ec, static_cast<int>(col_ok ? grow * cpr + (gcol >> 1) : OOB), 0, 0);
          __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(sc8), r_es,
                                               static_cast<int>(col_ok && (ln & 3) == 0 ? grow * spr + (gcol >> 5) : OOB), 0, 0);
          *reinterpret_cast<u32x4*>(sp) = av;
        }
        if constexpr (ENRG > 0) {
          lds_barrier();
          f32x4 pacc[EGW];
#pragma unroll
          for (int gi = 0; gi < EGW; ++gi) pacc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
          const int ar = ln & 15;
          const int asw = (ar & 1) | (((ar >> 2) & 1) << 1);
          auto frag = [&](int ks) {
            return lds_read_b128(lds_out + (wm * 2 + (ks >> 2)) * OUT_WAVE + ar * 256 +
                                 ((((ks & 3) ^ asw) << 6) | (16 * (ln >> 4))));
          };
          if constexpr (EACT == 1) {
            // the strip's eight fragments are read before the first MFMA, so
            // their LDS latencies overlap instead of each stalling its MFMAs
            // (the backward mirror holds h as well: there the eight
            // fragments would not fit beside it without spilling)
            u32x4 afs[8];
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) afs[ks] = frag(ks);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 8; ++ks)
#pragma unroll
              for (int gi = 0; gi < EGW; ++gi) pacc[gi] = mfma_bf16_16x16x32(afs[ks], bfr[gi][ks], pacc[gi]);
          } else {
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
              const u32x4 af = frag(ks);
#pragma unroll
              for (int gi = 0; gi < EGW; ++gi) pacc[gi] = mfma_bf16_16x16x32(af, bfr[gi][ks], pacc[gi]);
            }
          }
          lds_barrier();
          const uint32_t rb = srow >> 6, sl = (srow >> 4) & 3;
#pragma unroll
          for (int gi = 0; gi < EGW; ++gi) {
            const int gr = wn * EGW + gi;
            const uint32_t off = rb < nrb && gr < ENRG
                                     ? ((((static_cast<uint32_t>(j0) >> 8) * nrb + rb) * 4 + sl) * ENRG + gr) * 1024 + ln * 16
                                     : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pacc[gi]), r_ep, static_cast<int>(off), 0, 0);
          }
        }
        if constexpr (EACT == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) hcur[e] = hnxt[e];
        }
      }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  };

  // Split units: the fp32 sums of rows below M to g.part[split][row][col],
  // 128 bytes of a row per half wave; row groups past M are skipped whole
  // (a uniform test: a few-row output stores a few groups).  The stores are
  // then drained, so the waits of the next unit's steps, which budget for a
  // tile's 32 bf16 stores, still hold.
  auto store_part = [&](int64_t m0, int64_t j0, int split) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    float* dst = g.part + static_cast<int64_t>(split) * M * NOUT;
    const int64_t col0 = j0 + wn * 128 + (ln & 31);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t rbase = m0 + wm * 128 + 32 * mt + 8 * q;
        if (rbase >= M) continue;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t row = rbase + 4 * (ln >> 5) + e, col = col0 + 32 * nt;
            if (row < M && col < NOUT) dst[row * NOUT + col] = acc[mt][nt][4 * q + e];
          }
      }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0xF));
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  };

  // ---- prologue: stages 0..2 and the A half of stage 3
  Cursor ca{0, 0, 0, 0, 0, 0, 0}, cb{0, 0, 0, 0, 0, 0, 0};
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
  if constexpr (BT) {
    uint32_t raw[8];
    load_scales_bt(0, raw);
    shuffle_scales_bt(raw, E.bs);
  }
  read_frags(0, 0, E.a0, E.b0, Flag<BT>{});
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
  // kind: this step's MfmaKind.
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
      // BT: each instruction is pinned at its place in the step (an empty
      // use of its result): unpinned, the compiler sinks the half's 16 MFMAs
      // below the step's DMA issues and LDS reads, which then no longer
      // overlap them
      if constexpr (BT) asm volatile("" : "+a"(acc[i >> 2][i & 3]));
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
        read_frags(buf, 1, Cur.a1, Cur.b1, Flag<BT>{});
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
    uint32_t sraw[BT ? 8 : 1];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mma(i, Cur.a1, Cur.b1, op2);
      __builtin_amdgcn_sched_barrier(0);
      if (i == 0) {
        ha = half_dma(ca, false);
        read_scales(nbuf, ras, rbs);
        read_frags(nbuf, 0, Nxt.a0, Nxt.b0, Flag<BT>{});
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
      // BT: the next step's b scale words: raw words read at i == 4 (held
      // only until i == 12), shuffled in place into Nxt's words (the step
      // that last read them is long done)
      if constexpr (BT) {
        if (i == 4) {
          load_scales_bt(nbuf, sraw);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (i == 12) {
        if constexpr (BT) shuffle_scales_bt(sraw, Nxt.bs);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          Nxt.as[j] = ras[j] >> (8 * grp);
          Nxt.bs[j] = (BT ? Nxt.bs[j] : rbs[j]) >> (8 * grp);
        }
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
#pragma unroll
      for (int r = 0; r < NLR / 2; ++r) {
        step(E, O, rank, after && r == 0);
        step(O, E, rank, after && r == 0);
      }
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
    int ko;
    tile_of(k, m0, j0, ko);
    if constexpr (!LR && EPI == 0) {
      if (S > 1) {
        store_part(m0, j0, ko / nks);
        continue;
      }
    }
    if constexpr (EPI > 0) store_tile_mlp(m0, j0);
    else store_tile(m0, j0);
  }
  // DMAs into LDS must land before the workgroup can end
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0xF));
}

}  // namespace
}  // namespace ft
