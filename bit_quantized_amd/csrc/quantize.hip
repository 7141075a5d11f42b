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
//   k_quant_dual      one read of the input, codes of the input and of
//                     its transpose: 1x32 blocks (row32_t) or 32x32
//                     tiles (tile32 with both layouts)              (HBM bound)
//   k_quant_down      1x32 blocks along rows fused with the rank-R
//                     down-projection (bf16 MFMA, fp32 accumulation),
//                     split over columns into fp32 partials          (HBM bound)
//   k_rank_reduce     ordered sum of those partials, bf16 rounding, and
//                     the padded rank operands of the 4-bit GEMM     (HBM bound)
//   k_dequant_tile32  32x32-tile codes back to bf16 (16-bit products) (HBM bound)
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

// ---------------------------------------------------------------------------
// 1x32 row blocks.  Four consecutive lanes hold one block (16 bytes = 8
// values each), so one load instruction of a wave reads 16 consecutive
// blocks (1 KB) and one store writes their 256 bytes of codes; the block
// amax takes two quad DPP steps.  Each lane has U blocks in flight.  ACT
// applies the input activation first (0: none; 1: gelu(in); 2: in *
// gelu'(in2)), rounded to bf16 as the quantizer's input.  CONTIG: rows are
// contiguous (ld == cols), so block b starts at element 32 b.
template <int ACT, bool CONTIG, bool NTS>
__global__ __launch_bounds__(256) void k_quant_row32(const uint16_t* __restrict__ in,
                                                     const uint16_t* __restrict__ in2,
                                                     uint32_t rows, uint32_t cols, int64_t ld,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  constexpr int U = 4;
  const uint32_t bpr = cols >> 5;
  const uint32_t nblk = rows * bpr;                 // < 2^26 (host checks rows * ld * 2 < 2^31)
  const int lane = threadIdx.x & 63;
  const uint32_t q = lane & 3;
  const uint64_t bytes = static_cast<uint64_t>(rows) * ld * 2;
  const auto r1 = make_rsrc(in, bytes);
  const auto r2 = make_rsrc(in2, ACT == 2 ? bytes : 0);
  const uint32_t ld32 = static_cast<uint32_t>(ld);
  const uint32_t step = gridDim.x * 4 * 16 * U;
  const auto rcodes = make_rsrc(codes, static_cast<uint64_t>(nblk) * 16);
  const auto rscales = make_rsrc(scales, nblk);
  for (uint32_t b0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 16 * U; b0 < nblk; b0 += step) {
    u32x4 v[U], h[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t b = b0 + 16 * k + (lane >> 2);
      uint32_t e0 = b * 32;
      if constexpr (!CONTIG) {
        const uint32_t r = b / bpr;
        e0 = r * ld32 + (b - r * bpr) * 32;
      }
      const uint32_t off = b < nblk ? (e0 + q * 8) * 2 : BUF_OOB;
      v[k] = buf_load128_nt(r1, off);
      if constexpr (ACT == 2) h[k] = buf_load128_nt(r2, off);
      else h[k] = v[k];
    }
#pragma unroll
    for (int k = 0; k < U; ++k) {
      const uint32_t b = b0 + 16 * k + (lane >> 2);
      const u32x4 x = act_bf16x8<ACT>(v[k], h[k]);
      uint32_t am = hmax_u16x2(max_u16x2(max_u16x2(abs_bf16x2(x[0]), abs_bf16x2(x[1])),
                                         max_u16x2(abs_bf16x2(x[2]), abs_bf16x2(x[3]))));
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
      const uint32_t s = e8m0_from_amax_bits(am);
      const uint32_t o = encode8(x[0], x[1], x[2], x[3], e8m0_to_f32(s));
      // unconditional stores, masked by offset (exact wait counts)
      __builtin_amdgcn_raw_buffer_store_b32(o, rcodes, static_cast<int>(b < nblk ? b * 16 + q * 4 : BUF_OOB), 0,
                                            NTS ? 2 : 0);
      buf_store8(rscales, b < nblk && q == 0 ? b : BUF_OOB, s);
    }
  }
}

// ---------------------------------------------------------------------------
// 32x32 tiles, one layout.  Each wave quantizes 32 rows x 256 columns (8
// tiles) on its own: lane l holds columns 8 (l % 32) .. +7 of rows 2 i +
// l / 32 (i < 16), so every load instruction reads two whole 512-byte row
// pieces and every code store writes two whole 128-byte code lines.  The 8
// lanes of a tile (a quad in each half of the wave) reduce its amax with
// two quad DPP steps and one exchange between the halves; no LDS and no
// barrier, so each wave streams at its own pace.  A workgroup's 4 waves
// take the same 256 columns of 128 consecutive rows, and workgroups run in
// plain row-major order (an XCD-compact order in bands of 8 row groups
// made this one 10% slower: 70.7 against 63.5 us on 12288^2).
__global__ __launch_bounds__(256) void k_quant_tile32(const uint16_t* __restrict__ in,
                                                      uint32_t rows, uint32_t cols, int64_t ld,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t nx = (cols + 255) / 256, ny = rows / 32;
  const uint32_t x = blockIdx.x % nx, y = (blockIdx.x / nx) * 4 + wave;
  if (y >= ny) return;
  const uint32_t col = x * 256 + 8 * (lane & 31);
  const bool ok = col < cols;
  const uint32_t ld2 = static_cast<uint32_t>(ld) * 2;
  const uint32_t row0 = y * 32 + (lane >> 5);
  const auto rin = make_rsrc(in, static_cast<uint64_t>(rows) * ld * 2);
  const uint32_t base = ok ? row0 * ld2 + col * 2 : BUF_OOB;
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = buf_load128_nt(rin, base == BUF_OOB ? BUF_OOB : base + 2 * i * ld2);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max_u16x2(m, abs_bf16x2(v[i][j]));
  uint32_t am = hmax_u16x2(m);
  am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
  am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
  am = max(am, static_cast<uint32_t>(__builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, static_cast<int>(am))));
  const uint32_t s = e8m0_from_amax_bits(am);
  const float sc = e8m0_to_f32(s);
  // streaming (non-temporal) stores: weights are quantized once, ahead of use
  const uint32_t cpr = cols >> 1;
  const auto rcodes = make_rsrc(codes, static_cast<uint64_t>(rows) * cpr);
  const uint32_t cbase = ok ? row0 * cpr + (col >> 1) : BUF_OOB;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_raw_buffer_store_b32(encode8(v[i][0], v[i][1], v[i][2], v[i][3], sc), rcodes,
                                          static_cast<int>(cbase == BUF_OOB ? BUF_OOB : cbase + 2 * i * cpr), 0, 2);
  const auto rscales = make_rsrc(scales, static_cast<uint64_t>(ny) * (cols >> 5));
  buf_store8(rscales, ok && lane < 32 && (lane & 3) == 0 ? y * (cols >> 5) + (col >> 5) : BUF_OOB, s);
}

// ---------------------------------------------------------------------------
// Dual output from one read: 1x32 blocks along rows (codes [rows, cols/2],
// scales [rows, cols/32]) and along columns (the row blocks of the
// transpose: codes_t [cols, rows/2], scales_t [cols, rows/32]).
//
// A 512-thread workgroup covers a 256 x 256 tile.  Thread (rg = t / 32,
// cg = t % 32) holds rows 16 rg .. 16 rg + 15 of columns 8 cg .. 8 cg + 7;
// a column block (32 rows of one column) is lanes l and l + 32 of one wave:
//   - loads: one instruction reads two rows x 512 contiguous bytes;
//   - row blocks: four consecutive lanes hold one block, amax by two quad
//     DPP steps; one store instruction writes two full 128-byte code lines;
//   - column blocks: each lane's max over its 16 rows, then the partner
//     lane's (one shuffle); the codes come from vertical pairs (rows 2p,
//     2p+1 of one column share a scale), so each converted byte is a byte of
//     the transposed layout; the partners swap halves so that each owns four
//     whole 16-byte column blocks;
//   - the transposed codes meet in LDS (16-byte chunks, XOR-swizzled by
//     column so that neither the writes nor the reads conflict) and leave as
//     full 128-byte lines (256 rows of one column), eight per store
//     instruction; both scale arrays are gathered in LDS into 8-byte runs;
//   - code stores are non-temporal: the outputs are not read again soon
//     (measured: 146 -> 133 us on a 16384 x 12288 tensor).
// Rows are a multiple of 32 and columns of 32 (host checks), so a column
// block and a lane's 32-column row block are wholly inside or outside.
//
// TILE: 32 x 32 tiles instead (scales [rows/32, cols/32] and, transposed,
// [cols/32, rows/32]).  A tile is a quad of lanes and its partner quad; its
// one scale (two quad DPP steps and one shuffle) encodes both layouts, so no
// scale goes through LDS; one lane per tile writes the tile's two scale
// bytes.  Measured on a 12288 x 12288 weight: 93 -> 89 us against 32-row
// slabs with an LDS transpose.
//
// Registers are capped for 4 waves per SIMD (two workgroups per CU):
// ROW32_T then takes 128 registers (one spilled value) instead of 141 and
// runs in 121 instead of 129 us on the stress activation.
template <bool TILE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4)))
void k_quant_dual(const uint16_t* __restrict__ in, uint32_t rows, uint32_t cols, int64_t ld,
                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                  uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
  __shared__ __attribute__((aligned(16))) uint8_t ct[256 * 128];   // [column][16-byte chunk ^ swz]
  __shared__ __attribute__((aligned(16))) uint8_t st[256 * 8];     // column scales [column][block]
  __shared__ __attribute__((aligned(16))) uint8_t sr[256 * 8];     // row scales [row][block]
  const int t = threadIdx.x;
  const int rg = t >> 5, cg = t & 31;
  const bool upper = (rg & 1) != 0;                        // second 16 rows of the column block
  // plain row-major workgroup order: measured faster than bands of 8 row
  // groups made XCD-compact (ROW32_T 127 against 133 us, TILE32 with both
  // layouts 82 against 89 us at the stress shapes)
  const uint32_t nx = (cols + 255) / 256;
  const uint32_t x = blockIdx.x % nx, y = blockIdx.x / nx;
  const uint32_t row0 = y * 256 + 16 * rg;                 // this thread's first row
  const uint32_t col = x * 256 + 8 * cg;                   // this lane's first column
  // rows come in whole 32-row blocks, so both partners agree on this
  const bool ok = y * 256 + 32 * (rg >> 1) < rows && col < cols;
  const uint32_t ld2 = static_cast<uint32_t>(ld) * 2;
  const uint32_t cpr = cols >> 1, spr = cols >> 5, ncb = rows >> 5;
  const auto rin = make_rsrc(in, static_cast<uint64_t>(rows) * ld * 2);
  u32x4 v[16];
  {
    const uint32_t base = ok ? row0 * ld2 + col * 2 : BUF_OOB;
    // row i's offset rides in the uniform soffset, so one lane register
    // addresses all 16 loads (a lane out of range has its vector offset
    // past the end, and the range check keeps it there)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rin, static_cast<int>(base),
                                                                              static_cast<int>(i * ld2), 2));
  }

  // ---- TILE: one scale per 32x32 tile, the max over the thread's 16 x 8
  // values, its quad (32 columns) and its partner lane (the other 16 rows)
  uint32_t ts8 = 0;
  float tsc = 0.f;
  if constexpr (TILE) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max_u16x2(m, abs_bf16x2(v[i][k]));
    uint32_t am = hmax_u16x2(m);
    am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
    am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
    am = max(am, static_cast<uint32_t>(__shfl_xor(static_cast<int>(am), 32)));
    ts8 = e8m0_from_amax_bits(am);
    tsc = e8m0_to_f32(ts8);
    // the tile's scale in both grids, from one lane per tile
    const bool w = ok && !upper && (cg & 3) == 0;
    const uint32_t tr = y * 8 + (rg >> 1), tc = x * 8 + (cg >> 2);
    buf_store8(make_rsrc(scales, static_cast<uint64_t>(ncb) * spr), w ? tr * spr + tc : BUF_OOB, ts8);
    if (scales_t) buf_store8(make_rsrc(scales_t, static_cast<uint64_t>(spr) * ncb), w ? tc * ncb + tr : BUF_OOB, ts8);
  }

  // ---- row blocks (TILE: with the tile's scale)
  const auto rcodes = make_rsrc(codes, static_cast<uint64_t>(rows) * cpr);
  const uint32_t cbase = ok ? row0 * cpr + (col >> 1) : BUF_OOB;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t s8;
    if constexpr (TILE) {
      s8 = ts8;
    } else {
      uint32_t am = hmax_u16x2(max_u16x2(max_u16x2(abs_bf16x2(v[i][0]), abs_bf16x2(v[i][1])),
                                         max_u16x2(abs_bf16x2(v[i][2]), abs_bf16x2(v[i][3]))));
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
      s8 = e8m0_from_amax_bits(am);
    }
    const uint32_t o = encode8(v[i][0], v[i][1], v[i][2], v[i][3], TILE ? tsc : e8m0_to_f32(s8));
    __builtin_amdgcn_raw_buffer_store_b32(o, rcodes, static_cast<int>(cbase), static_cast<int>(i * cpr), 2);
    if constexpr (!TILE) {
      if ((cg & 3) == 0) sr[(16 * rg + i) * 8 + (cg >> 2)] = static_cast<uint8_t>(s8);
    }
  }
  if constexpr (TILE) {
    if (!codes_t) return;                                  // weight codes in one layout only
  }

  // ---- column blocks: amax of columns 2k (low half) and 2k+1 (high half)
  // over the 32 rows of both partners
  u32x4 cm = {0, 0, 0, 0};
  if constexpr (!TILE) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) cm[k] = max_u16x2(cm[k], abs_bf16x2(v[i][k]));
#pragma unroll
    for (int k = 0; k < 4; ++k) cm[k] = max_u16x2(cm[k], static_cast<uint32_t>(__shfl_xor(static_cast<int>(cm[k]), 32)));
  }
  // The lower partner keeps columns 0..3 of its 8, the upper one 4..7: each
  // sends the halves (its 16 rows, 8 bytes) of the other four columns and
  // receives their partner halves; the lower 16 rows are the first 8 bytes
  // of a column block.  Columns j and 4 + j travel together, so they are
  // made together: the pairs of words k and k + 2 of the loads (columns
  // 2k, 2k + 1 and 2k + 4, 2k + 5), after which those words are dead.
  const int jb = upper ? 4 : 0;
  const int swz = cg & 7;
  const int cb = rg >> 1;                                  // 32-row block of the tile
  uint32_t cs[8];
#pragma unroll
  for (int kp = 0; kp < 2; ++kp) {
    uint32_t hf[2][2][2];                                  // [k = kp, kp + 2][column parity][16-row half]
#pragma unroll
    for (int wk = 0; wk < 2; ++wk) {
      const int k = kp + 2 * wk;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t s8 = TILE ? ts8 : e8m0_from_amax_bits(h ? cm[k] >> 16 : cm[k] & 0xFFFFu);
        cs[2 * k + h] = s8;
        const float sc = TILE ? tsc : e8m0_to_f32(s8);
        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
        // byte p of word m = rows 8m + 2p (low nibble) and 8m + 2p + 1
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          auto vp = [&](int p) {
            return __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(v[8 * m + 2 * p + 1][k], v[8 * m + 2 * p][k], sel));
          };
          uint32_t r = 0;
          r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, vp(0), sc, 0);
          r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, vp(1), sc, 1);
          r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, vp(2), sc, 2);
          r = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(r, vp(3), sc, 3);
          hf[wk][h][m] = r;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int j = 2 * kp + h;                            // columns j (wk 0) and 4 + j (wk 1)
      uint32_t blk[4];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t send = upper ? hf[0][h][m] : hf[1][h][m];
        const uint32_t got = static_cast<uint32_t>(__shfl_xor(static_cast<int>(send), 32));
        const uint32_t mine = upper ? hf[1][h][m] : hf[0][h][m];
        blk[m] = upper ? got : mine;
        blk[2 + m] = upper ? mine : got;
      }
      const int c = 8 * cg + jb + j;                       // column within the tile
      *reinterpret_cast<u32x4*>(&ct[c * 128 + ((cb ^ swz) << 4)]) = u32x4{blk[0], blk[1], blk[2], blk[3]};
    }
  }
  // column scales: the same split (constant indices: a lane-dependent index
  // into cs would put the array in scratch)
  if constexpr (!TILE) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j >= 4) == upper) st[(8 * cg + j) * 8 + cb] = static_cast<uint8_t>(cs[j]);
  }
  __syncthreads();

  // ---- transposed codes: chunk u = t + 512 s is column u / 8, 16-byte
  // piece u % 8 (rows 32 q .. 32 q + 31) of the column's 128-byte line
  const auto rcodes_t = make_rsrc(codes_t, static_cast<uint64_t>(cols) * (rows >> 1));
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const int u = t + 512 * s2, c = u >> 3, q = u & 7;
    const u32x4 w = *reinterpret_cast<const u32x4*>(&ct[c * 128 + ((q ^ ((c >> 3) & 7)) << 4)]);
    const uint32_t gc = x * 256 + c, gr = y * 256 + 32 * q;
    const bool in = gc < cols && gr < rows;
    __builtin_amdgcn_raw_buffer_store_b128(w, rcodes_t, static_cast<int>(in ? gc * (rows >> 1) + (gr >> 1) : BUF_OOB), 0, 2);
  }
  // ---- scales: threads 0..255 write row t's 8 row-scale bytes, threads
  // 256..511 column t-256's 8 column-scale bytes (one 8-byte store when the
  // run is aligned and whole); TILE wrote its tile scales above
  if constexpr (TILE) return;
  if (t < 256) {
    const auto rscales = make_rsrc(scales, static_cast<uint64_t>(rows) * spr);
    const uint32_t gr = y * 256 + t;
    const u32x2 rs = *reinterpret_cast<const u32x2*>(&sr[t * 8]);
    if ((spr & 7) == 0) {
      __builtin_amdgcn_raw_buffer_store_b64(rs, rscales, static_cast<int>(gr < rows ? gr * spr + 8 * x : BUF_OOB), 0, 0);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        buf_store8(rscales, gr < rows && 8 * x + b < spr ? gr * spr + 8 * x + b : BUF_OOB, rs[b >> 2] >> (8 * (b & 3)));
    }
  } else {
    const auto rscales_t = make_rsrc(scales_t, static_cast<uint64_t>(cols) * ncb);
    const int tc = t - 256;
    const uint32_t gc = x * 256 + tc;
    const u32x2 cs2 = *reinterpret_cast<const u32x2*>(&st[tc * 8]);
    if ((ncb & 7) == 0) {
      __builtin_amdgcn_raw_buffer_store_b64(cs2, rscales_t, static_cast<int>(gc < cols ? gc * ncb + 8 * y : BUF_OOB), 0, 0);
    } else {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        buf_store8(rscales_t, gc < cols && 8 * y + b < ncb ? gc * ncb + 8 * y + b : BUF_OOB, cs2[b >> 2] >> (8 * (b & 3)));
    }
  }
}

// ---------------------------------------------------------------------------
// Fused 1x32 row quantization + rank-R down-projection, in two kernels.
//
// out_lr[row][r] = bf16( sum_c in[row][c] * proj[r][c] ),  r < R,
// with proj given rank-major (one row of `cols` values per rank) as two
// pieces of r0 and r1 rows.
//
// k_quant_down: persistent.  The columns are cut into splits of KC = 128*NS;
// `wg_per_split` workgroups share a split and walk its 64-row blocks
// (workgroup j takes blocks j, j + G, ...).  A workgroup stages the
// projection slice of its split [RP ranks x KC columns] in LDS once.  Each
// wave then streams its own 16 rows of every block it visits:
//   - loads: one instruction reads KC/8 lanes x 16 bytes of rows (two rows
//     of 512 bytes at KC = 256); the loads of block b + G go out as soon as
//     block b is quantized, so a block is in flight while the wave projects,
//     and the two workgroups a CU holds at KC = 256 hide each other's waits;
//   - quantize in the load layout: 4 consecutive lanes hold one 32-element
//     block, amax by two quad DPP steps; codes go out as 4 bytes per lane
//     (a row's codes contiguous), scales from every 4th lane;
//   - the same bf16 values go to the wave's LDS area and come back as
//     16x16x32 MFMA fragments (row = lane % 16, 8 columns of group
//     lane / 16) against the projection in LDS: fp32 sums over the split;
//   - the 16 x RP result goes to a workspace slab, laid out as the
//     accumulators are held (16 contiguous bytes per lane);
//   - backward with the adapter gradient fused (DBR rank groups): after a
//     barrier every wave reads all four slabs back transposed
//     (ds_read_b64_tr_b16) for its quarter of the columns and accumulates
//     dB[r][col] += sum_row u[row][r] x[row][col] with 16x16x16 MFMAs; a
//     second barrier frees the slabs.  At the end each workgroup writes its
//     partial, which the adapter-gradient reduce sums in workgroup order.
//
// k_rank_reduce (the next kernel on the stream, so every slab is visible):
// sums the slabs in split order (deterministic), rounds once, and writes
// out_lr [rows, R] and out_pad [rows, rpad] (the same values with zero ranks
// R .. rpad-1, for the 4-bit GEMM).  It also copies the GEMM's other rank
// operand transposed, cp_dst[i][r] = cp[r][i], zero-padded to rpad ranks.
struct QDArgs {
  const uint16_t* in;
  const uint16_t* in2;  // second input of ACT 2 (gelu' argument), else unused
  uint32_t rows, cols;
  int64_t ld;
  uint8_t* codes;
  uint8_t* scales;
  RankRows pr;
  int R;
  uint32_t wg_per_split;
  float* part;          // [splits][rows/64][4 waves][NRG][64 lanes][4]
  // adapter gradient dB of the backward (DBR > 0): sum over rows of
  // u[row][u_r0 + r] * in[row][col], r < u_rl, per workgroup of a split
  const uint16_t* u;
  int64_t ld_u;
  int u_r0, u_rl;
  float* dbpart;        // [wg_per_split][16 DBR][cols], rank-major
};

template <int NRG, int NS, int ACT, int DBR>
__global__ __launch_bounds__(256, 1) void k_quant_down(const QDArgs a) {
  constexpr int RP = NRG * 16;
  constexpr int KC = 128 * NS;
  constexpr int PT = KC + 8;
  constexpr int LPR = KC / 8;
  constexpr int RPI = 64 / LPR;
  constexpr int NI = 16 / RPI;
  constexpr int NT = KC / 16;                 // 16-column tiles of a split (dB)
  constexpr int LDS_PT = RP * PT * 2, LDS_XT = 4 * 16 * PT * 2;
  // per wave: the codes [16 rows][KC/2 bytes] and scales [16 rows][KC/32]
  // of its rows in a block, gathered so that they leave as 16-byte stores
  constexpr int CSC = 16 * (KC / 2), CSS = 16 * (KC / 32);
  constexpr int LDS_CS = 4 * (CSC + CSS);
  constexpr int LDS_BYTES = LDS_PT + LDS_XT + LDS_CS;
  __shared__ __attribute__((aligned(16))) uint8_t lds[LDS_BYTES];
  uint16_t* pt = reinterpret_cast<uint16_t*>(lds);
  uint16_t (*xt)[16 * PT] = reinterpret_cast<uint16_t (*)[16 * PT]>(lds + LDS_PT);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const uint32_t rows = a.rows, cols = a.cols;
  const uint32_t nrb = (rows + 63) / 64;
  const uint32_t G = a.wg_per_split;
  const uint32_t y = blockIdx.x / G;
  const uint32_t cbeg = y * KC;
  const int lrow = lane / LPR, lcol = (lane % LPR) * 8;
  const uint32_t col = cbeg + lcol;
  const bool col_ok = col < cols;
  const uint32_t ld2 = static_cast<uint32_t>(a.ld) * 2;
  const auto rin = make_rsrc(a.in, static_cast<uint64_t>(rows) * a.ld * 2);
  // Byte offset of this lane's element in row block 0, instruction 0.  Rows
  // past the end read as zero through the buffer size (32-bit offsets:
  // rows * ld * 2 < 2^31); columns past the end are masked here.
  const uint32_t lane_off = col_ok ? (static_cast<uint32_t>(16 * wave + lrow) * ld2 + col * 2) : BUF_OOB;
  const auto rin2 = make_rsrc(a.in2, ACT == 2 ? static_cast<uint64_t>(rows) * a.ld * 2 : 0);
  // dB: every wave takes all 64 rows of the block and a quarter of its
  // columns.  For row group h (rows 16h .. 16h+15) lane (group g, q) holds
  // u[row][u_r0 + 16 c + q] of rows 16h + 4g .. 16h + 4g + 3 (the A operand
  // of a 16x16x16 MFMA).
  const int g = lane >> 4, lr = lane & 15;
  constexpr int UA = DBR > 0 ? 4 * DBR : 1;   // (row group, rank group) pairs
  auto load = [&](u32x4* v, u32x4* h, uint32_t bx) {
    // past the end stays past the end: the host keeps (rows + 64) * ld * 2
    // below 2^31, so BUF_OOB plus any row offset here does not wrap
    const uint32_t base = bx < nrb ? bx * 64 * ld2 + lane_off : BUF_OOB;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t off = base + i * RPI * ld2;
      // X is read again by the adapter gradients, and so is dY when dB is not
      // fused here: cached.  With dB fused, dY (and h) are read only here.
      if constexpr (DBR > 0) {
        v[i] = buf_load128_nt(rin, off);
        if constexpr (ACT == 2) h[i] = buf_load128_nt(rin2, off);
      } else {
        v[i] = buf_load128(rin, off);
        if constexpr (ACT == 2) h[i] = buf_load128(rin2, off);
      }
    }
  };
  // The adapter operand of block bx, loaded when the block starts (its
  // quantize and projection phases cover the latency) and held only within
  // the block: plain 16-bit loads, zero-extended by the load itself.  Indices
  // are clamped into the tensor: a row past the end meets x = 0, and ranks
  // past u_rl only feed partial rows the reduce never reads.
  auto load_u = [&](uint32_t (*uu)[4], uint32_t bx) {
#pragma unroll
    for (int hc = 0; hc < 4 * DBR; ++hc)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t row = min(bx * 64 + 16 * (hc / DBR) + 4 * g + e, rows - 1);
        const int r = min(16 * (hc % DBR) + lr, a.u_rl - 1);
        uu[hc][e] = a.u[row * static_cast<uint32_t>(a.ld_u) + a.u_r0 + r];
      }
  };
  u32x4 va[NI], ha[NI];
  uint32_t bx = blockIdx.x % G;
  load(va, ha, bx);
  {
    const RankRows& p = a.pr;
    const int R = a.R;
    const auto r0s = make_rsrc(p.p0, static_cast<uint64_t>(p.r0) * p.ld * 2);
    const auto r1s = make_rsrc(p.p1, static_cast<uint64_t>(p.r1) * p.ld * 2);
    constexpr int CPR = KC / 8;
    constexpr int PER = (RP * CPR + 255) / 256;
    u32x4 w[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;
      const int r = c / CPR, cc = (c % CPR) * 8;
      const uint32_t pc = cbeg + cc;
      const bool ok = c < RP * CPR && pc < cols;
      const uint32_t o0 = (ok && r < p.r0) ? static_cast<uint32_t>((r * p.ld + pc) * 2) : BUF_OOB;
      const uint32_t o1 = (ok && r >= p.r0 && r < R) ? static_cast<uint32_t>(((r - p.r0) * p.ld + pc) * 2) : BUF_OOB;
      w[e] = buf_load128(r0s, o0) | buf_load128(r1s, o1);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = t + 256 * e;
      if (c < RP * CPR) *reinterpret_cast<u32x4*>(&pt[(c / CPR) * PT + (c % CPR) * 8]) = w[e];
    }
  }
  __syncthreads();
  uint16_t* xw = xt[wave];
  const uint32_t cpr = cols >> 1, spr = cols >> 5;
  // no codes wanted (a 16-bit product follows): empty buffers drop the stores
  const auto rcodes = make_rsrc(a.codes, a.codes ? static_cast<uint64_t>(rows) * cpr : 0);
  const auto rscales = make_rsrc(a.scales, a.scales ? static_cast<uint64_t>(rows) * spr : 0);
  const auto rpart = make_rsrc(a.part, static_cast<uint64_t>(gridDim.x / G) * nrb * 4 * NRG * 256 * 4);
  constexpr int NTW = NT / 4;                 // dB column tiles per wave
  f32x4 dacc[DBR > 0 ? DBR : 1][DBR > 0 ? NTW : 1];
  if constexpr (DBR > 0) {
#pragma unroll
    for (int c = 0; c < DBR; ++c)
#pragma unroll
      for (int n = 0; n < NTW; ++n) dacc[c][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  uint8_t* csc = lds + LDS_PT + LDS_XT + wave * (CSC + CSS);
  uint8_t* css = csc + CSC;
  auto quant = [&](const u32x4* vin, const u32x4* hin, uint32_t b) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const u32x4 v = act_bf16x8<ACT>(vin[i], ACT == 2 ? hin[i] : vin[i]);
      uint32_t m = max_u16x2(max_u16x2(abs_bf16x2(v[0]), abs_bf16x2(v[1])),
                             max_u16x2(abs_bf16x2(v[2]), abs_bf16x2(v[3])));
      uint32_t am = hmax_u16x2(m);
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0xB1, 0xF, 0xF, false)));
      am = max(am, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(am), 0x4E, 0xF, 0xF, false)));
      const uint32_t sc8 = e8m0_from_amax_bits(am);
      const uint32_t o = encode8(v[0], v[1], v[2], v[3], e8m0_to_f32(sc8));
      const int rl = i * RPI + lrow;
      *reinterpret_cast<uint32_t*>(&csc[rl * (KC / 2) + (lcol >> 1)]) = o;
      if ((lane & 3) == 0) css[rl * (KC / 32) + (lcol >> 5)] = static_cast<uint8_t>(sc8);
      *reinterpret_cast<u32x4*>(&xw[rl * PT + lcol]) = v;
    }
    // the wave's codes leave as 16-byte pieces (one 32-value block each),
    // its scales as one run per row where the split is whole and the rows
    // of the scale array are 4-byte aligned, else byte by byte
    const uint32_t row0 = b * 64 + 16 * wave;
#pragma unroll
    for (int q = 0; q < CSC / 1024; ++q) {
      const int c = q * 64 + lane, rl = c / (KC / 32), pc = c % (KC / 32);
      const uint32_t row = row0 + rl;
      const bool ok = row < rows && cbeg + 32 * pc < cols;
      buf_store128(rcodes, ok ? row * cpr + (cbeg >> 1) + 16 * pc : BUF_OOB,
                   *reinterpret_cast<const u32x4*>(&csc[c * 16]));
    }
    // (both forms are always issued, the one not taken with out-of-range
    // offsets: no branch, so the compiler's memory counts stay exact)
    const bool runs = cbeg + KC <= cols && (spr & 3) == 0;
    if constexpr (KC >= 512) {
      // KC/32 >= 16 scale bytes per row: lane l < 16 * PPR stores 16 bytes
      constexpr int PPR = KC / 512;               // 16-byte pieces per row
      const int rl = lane / PPR, pc = lane % PPR;
      const uint32_t row = row0 + rl;
      const bool ok = runs && lane < 16 * PPR && row < rows;
      buf_store128(rscales, ok ? row * spr + (cbeg >> 5) + 16 * pc : BUF_OOB,
                   *reinterpret_cast<const u32x4*>(&css[lane < 16 * PPR ? lane * 16 : 0]));
    } else {
      // fewer than 16 scale bytes per row: 4-byte runs
      constexpr int WPR = KC / 128;               // 4-byte words per row
      const int rl = lane / WPR, pc = lane % WPR;
      const uint32_t row = row0 + rl;
      const bool ok = runs && lane < 16 * WPR && row < rows;
      buf_store32(rscales, ok ? row * spr + (cbeg >> 5) + 4 * pc : BUF_OOB,
                  *reinterpret_cast<const uint32_t*>(&css[lane < 16 * WPR ? lane * 4 : 0]));
    }
#pragma unroll
    for (int q = 0; q < (CSS + 63) / 64; ++q) {
      const int c = q * 64 + lane, rl = c / (KC / 32), pc = c % (KC / 32);
      const uint32_t row = row0 + rl;
      const bool ok = !runs && c < CSS && row < rows && cbeg + 32 * pc < cols;
      buf_store8(rscales, ok ? row * spr + (cbeg >> 5) + pc : BUF_OOB, css[c < CSS ? c : 0]);
    }
  };
  auto mma = [&](uint32_t b, uint32_t (*uu)[4]) {
    f32x4 acc[NRG];
#pragma unroll
    for (int c = 0; c < NRG; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KC / 32; ++ks) {
      const u32x4 af = lds_read_b128(&xw[lr * PT + 32 * ks + 8 * g]);
#pragma unroll
      for (int c = 0; c < NRG; ++c)
        acc[c] = mfma_bf16_16x16x32(af, lds_read_b128(&pt[(16 * c + lr) * PT + 32 * ks + 8 * g]), acc[c]);
      if ((ks & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    // this wave's slab; nothing is stored for a block past the end
    const uint32_t slab = b < nrb ? ((y * nrb + b) * 4 + wave) * (NRG * 256 * 4) + lane * 16 : BUF_OOB;
#pragma unroll
    for (int c = 0; c < NRG; ++c)
      buf_store128(rpart, slab + c * 1024, __builtin_bit_cast(u32x4, acc[c]));
    if constexpr (DBR > 0) {
      // dB += u^T x over the block's 64 rows and this wave's columns
      // KC/4 * wave .. +KC/4: B operand = rows 4g .. 4g+3 of row group h at
      // column 16 n + q, read transposed from wave h's row-major slab (all
      // four slabs are complete: barrier before this phase)
      // The empty asm marks the loaded values as used here, so the compiler
      // neither packs them nor waits for their loads any earlier.
      i32x2 au[UA];
#pragma unroll
      for (int hc = 0; hc < 4 * DBR; ++hc) {
        asm volatile("" : "+v"(uu[hc][0]), "+v"(uu[hc][1]), "+v"(uu[hc][2]), "+v"(uu[hc][3]));
        au[hc] = i32x2{static_cast<int>(__builtin_amdgcn_perm(uu[hc][1], uu[hc][0], 0x05040100u)),
                       static_cast<int>(__builtin_amdgcn_perm(uu[hc][3], uu[hc][2], 0x05040100u))};
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < 4; ++h) {
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          const u32x2 bx2 = lds_read_tr16(&xt[h][(4 * g + (lr >> 2)) * PT + (KC / 4) * wave + 16 * n + 4 * (lr & 3)]);
#pragma unroll
          for (int c = 0; c < DBR; ++c) dacc[c][n] = mfma_bf16_16x16x16(au[h * DBR + c], bx2, dacc[c][n]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the slabs are rewritten by the next block's quantize
      __syncthreads();
    }
  };
  // one block: its adapter operand (dB), quantize, refill the registers
  // with the workgroup's next block, project.  The body is straight-line (a
  // block past the end reads zeros and stores nothing), so the compiler's
  // count of outstanding loads and stores stays exact.
  auto block = [&](uint32_t b) {
    uint32_t uu[UA][4];
    if constexpr (DBR > 0) load_u(uu, b);
    quant(va, ha, b);
    load(va, ha, b + G);
    mma(b, uu);
  };
  for (; bx < nrb; bx += G) block(bx);
  if constexpr (DBR > 0) {
    // the workgroup's partial dbpart[j][r][col]: each wave owns its columns
    const uint32_t j = blockIdx.x % G;
    float* dst = a.dbpart + static_cast<uint64_t>(j) * (DBR * 16) * cols;
#pragma unroll
    for (int c = 0; c < DBR; ++c)
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        const uint32_t cc = cbeg + (KC / 4) * wave + 16 * n + lr;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (cc < cols) dst[static_cast<uint64_t>(16 * c + 4 * g + e) * cols + cc] = dacc[c][n][e];
      }
  }
}

struct RRArgs {
  const float* part;
  uint32_t rows, splits;
  int R, rpad;
  uint16_t* out_lr;
  uint16_t* out_pad;
  RankRows cp;
  int64_t cp_rows;
  uint16_t* cp_dst;
  int cp_planes;        // cp_dst as nibble planes (copy_rank_planes) instead
};

// k_rank_reduce: blocks [0, 4 * rowblocks) each sum one 16-row slab (one
// wave's accumulators of k_quant_down) over the column splits; the blocks
// after them copy the GEMM's other rank operand.
//
// Sum: thread t < 64 * NRG owns accumulator item t (4 rows x 1 rank); it
// issues the loads of 8 splits at a time and adds them in split order, so
// the result does not depend on the launch shape.  The 16 x rpad result goes
// through LDS to contiguous stores.
template <int NRG>
__device__ __forceinline__ void rank_sum_slab(const RRArgs& a, uint32_t b) {
  constexpr int RP = NRG * 16;
  __shared__ float sum[16][RP + 1];
  const int t = threadIdx.x;
  const uint32_t nrb = (a.rows + 63) / 64;
  const uint32_t bx = b >> 2, wave = b & 3;
  const uint64_t slab = static_cast<uint64_t>(NRG) * 256;                 // floats per wave slab
  const uint64_t stride = static_cast<uint64_t>(nrb) * 4 * slab;          // between splits
  // (more than 4 rank groups: a thread owns items t and t + 256).  The
  // loads of 16 splits go out together as buffer loads, the ones past the
  // last split answered with zero: no branch between them, so a batch
  // costs one memory latency (the sum still runs in split order).
  const auto rpart = make_rsrc(a.part, stride * a.splits * 4);
  for (int it = t; it < 64 * NRG; it += 256) {
    const uint32_t base = static_cast<uint32_t>(((static_cast<uint64_t>(bx) * 4 + wave) * slab + it * 4) * 4);
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (uint32_t y0 = 0; y0 < a.splits; y0 += 16) {
      f32x4 v[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t off = y0 + k < a.splits ? base + static_cast<uint32_t>((y0 + k) * stride * 4) : BUF_OOB;
        v[k] = __builtin_bit_cast(f32x4, buf_load128(rpart, off));
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) s += v[k];
    }
    const int c = it >> 6, lane = it & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) sum[4 * (lane >> 4) + j][16 * c + (lane & 15)] = s[j];
  }
  __syncthreads();
  const int R = a.R, rpad = a.rpad;
  const uint32_t r0 = bx * 64 + wave * 16;
  // out_pad: 16 rows x rpad ranks, contiguous; 8 ranks (16 bytes) per thread
  for (int idx = t; idx < 16 * (rpad >> 3); idx += 256) {
    const int rl = idx / (rpad >> 3), r8 = (idx % (rpad >> 3)) * 8;
    if (r0 + rl >= a.rows) continue;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = r8 + 2 * k;
      const uint32_t lo = r < R ? f32_to_bf16_rne(sum[rl][r]) : 0u;
      const uint32_t hi = r + 1 < R ? f32_to_bf16_rne(sum[rl][r + 1]) : 0u;
      w[k] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4*>(a.out_pad + static_cast<uint64_t>(r0 + rl) * rpad + r8) =
        u32x4{w[0], w[1], w[2], w[3]};
  }
  // out_lr: 16 rows x R ranks, contiguous
  for (int idx = t; idx < 16 * R; idx += 256) {
    const int rl = idx / R, r = idx % R;
    if (r0 + rl < a.rows) a.out_lr[static_cast<uint64_t>(r0 + rl) * R + r] = f32_to_bf16_rne(sum[rl][r]);
  }
}

// Copy: cp_dst[i][r] = cp[r][i] (r < R) or 0 (R <= r < rpad).  A thread
// makes one 16-byte chunk (8 ranks of row i) from 8 loads issued together;
// consecutive lanes take consecutive i, so each load is coalesced.
__device__ __forceinline__ void copy_rank_chunk(const RRArgs& a, uint64_t e) {
  const RankRows& p = a.cp;
  const uint64_t total = static_cast<uint64_t>(a.cp_rows) * (a.rpad >> 3);
  if (e >= total) return;
  const int c = static_cast<int>(e / a.cp_rows);         // chunk: ranks 8c .. 8c+7
  const int64_t i = static_cast<int64_t>(e % a.cp_rows);
  uint32_t h[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int r = 8 * c + q;
    h[q] = r < p.r0 ? p.p0[r * p.ld + i] : (r < a.R ? p.p1[(r - p.r0) * p.ld + i] : uint16_t(0));
  }
  *reinterpret_cast<u32x4*>(a.cp_dst + i * a.rpad + 8 * c) =
      u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// The other rank operand as nibble planes, for a GEMM that reads its b
// operand with the 4-bit transposing LDS read (ds_read_b64_tr_b4): rpad ranks
// (zero past R) of cp_rows columns become 4 rpad plane rows of cp_rows / 2
// bytes, plane row 128 s + R for ranks 32 s .. 32 s + 31 holding, for
// every column, nibble R % 4 of rank 32 s + R / 4's bf16 value (low nibble:
// even column).  Such a read takes, for 16 lanes, 16 consecutive plane rows
// of one column each, so lane k of a 32-column block receives the 4 nibbles
// of 4 consecutive ranks in order: 8 bf16 ranks of its column per two
// reads, the bf16 fragment of a rank step, from the same staging, lane
// offsets and reads as the 4-bit steps.  A thread makes the 4 plane rows of
// one rank and 32 columns (64 bytes read, 4 x 16 bytes written).
__device__ __forceinline__ void copy_rank_planes(const RRArgs& a, uint64_t e) {
  const RankRows& p = a.cp;
  const uint32_t pieces = static_cast<uint32_t>(a.cp_rows / 32);
  if (e >= static_cast<uint64_t>(a.rpad) * pieces) return;
  const int r = static_cast<int>(e / pieces);
  const uint32_t piece = static_cast<uint32_t>(e % pieces);
  const uint16_t* src = r < p.r0 ? p.p0 + static_cast<int64_t>(r) * p.ld
                      : r < a.R ? p.p1 + static_cast<int64_t>(r - p.r0) * p.ld : nullptr;
  uint32_t v[16];                                        // 32 bf16, two per word
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const u32x4 w = src ? *reinterpret_cast<const u32x4*>(src + 32 * piece + 8 * k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) v[4 * k + j] = w[j];
  }
  uint8_t* dst = reinterpret_cast<uint8_t*>(a.cp_dst);
  const uint64_t pitch = static_cast<uint64_t>(a.cp_rows / 2);
#pragma unroll
  for (int nib = 0; nib < 4; ++nib) {
    // byte m: columns 2m (low nibble) and 2m + 1, i.e. the two bf16 of word m
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t b = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t w = v[4 * q + m];
        const uint32_t lo = (w >> (4 * nib)) & 0xFu, hi = (w >> (16 + 4 * nib)) & 0xFu;
        b |= (lo | (hi << 4)) << (8 * m);
      }
      o[q] = b;
    }
    const uint64_t prow = static_cast<uint64_t>(128 * (r >> 5) + 4 * (r & 31) + nib);
    *reinterpret_cast<u32x4*>(dst + prow * pitch + 16 * piece) = u32x4{o[0], o[1], o[2], o[3]};
  }
}

template <int NRG>
__global__ __launch_bounds__(256) void k_rank_reduce(const RRArgs a) {
  const uint32_t nsum = ((a.rows + 63) / 64) * 4;
  if (blockIdx.x < nsum)
    rank_sum_slab<NRG>(a, blockIdx.x);
  else if (a.cp_planes)
    copy_rank_planes(a, static_cast<uint64_t>(blockIdx.x - nsum) * 256 + threadIdx.x);
  else
    copy_rank_chunk(a, static_cast<uint64_t>(blockIdx.x - nsum) * 256 + threadIdx.x);
}

// ---------------------------------------------------------------------------
// host launchers

// ---------------------------------------------------------------------------
// 32x32-tile MXFP4 back to bf16, the weight operand of a 16-bit product.
// Lane i takes 16 code bytes (32 values, one tile row piece, one scale) of a
// row: a load instruction reads 1 KB contiguous, four stores write the 4 KB
// of bf16 they make.  Each value is built
// directly as bf16 bits, exactly: an E2M1 magnitude m = 1..7 is 2^E (1 + f)
// with E = m/2 - 1 and f = 1/2 for odd m > 1, so times the tile's 2^(s-127)
// its bf16 exponent field is E + s; where that is below 1 the value is a bf16
// subnormal, (2 + 2f) * 2^(E + s + 5) units of 2^-133 (a left shift, since
// E + s >= -1); at 255 and above it is infinite (no finite weight gives a
// scale that large).
__device__ __forceinline__ uint32_t e2m1_to_bf16(uint32_t n, int s) {
  const uint32_t m = n & 7u, sg = (n & 8u) << 12;
  const int ex = static_cast<int>(m >> 1) - 1 + s;
  const uint32_t f = m > 1u ? (m & 1u) : 0u;
  const uint32_t normal = (static_cast<uint32_t>(ex) << 7) | (f << 6);
  const uint32_t sub = (2u + f) << (ex + 5 > 0 ? ex + 5 : 0);
  const uint32_t mag = m == 0u ? 0u : ex >= 255 ? 0x7F80u : ex >= 1 ? normal : sub;
  return sg | mag;
}

__global__ __launch_bounds__(256) void k_dequant_tile32(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        uint32_t rows, uint32_t cols,
                                                        uint16_t* __restrict__ out) {
  const uint32_t cpr = cols >> 1, spr = cols >> 5;
  const uint32_t total = rows * spr;                      // 32-value row pieces, one per lane
  const auto rc = make_rsrc(codes, static_cast<uint64_t>(rows) * cpr);
  const auto rs = make_rsrc(scales, static_cast<uint64_t>(rows >> 5) * spr);
  const auto ro = make_rsrc(out, static_cast<uint64_t>(rows) * cols * 2);
  const uint32_t stride = gridDim.x * 256;
  // two pieces per lane per pass, both loads issued before either is used;
  // a piece past the end reads zeros and stores nothing
  for (uint32_t i = blockIdx.x * 256 + threadIdx.x; i < total; i += 2 * stride) {
    uint32_t p[2], r[2], c[2];
    u32x4 w[2];
    uint32_t sb[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      p[h] = i + h * stride;
      const bool ok = p[h] < total;
      r[h] = ok ? p[h] / spr : 0;
      c[h] = ok ? p[h] - r[h] * spr : 0;
      w[h] = buf_load128_nt(rc, ok ? r[h] * cpr + 16 * c[h] : BUF_OOB);
      sb[h] = __builtin_amdgcn_raw_buffer_load_b8(rs, static_cast<int>(ok ? (r[h] >> 5) * spr + c[h] : BUF_OOB), 0, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int sc = static_cast<int>(sb[h]);
      const uint32_t base = p[h] < total ? (r[h] * cols + 32 * c[h]) * 2 : BUF_OOB;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t byte = w[h][q] >> (8 * j);
          o[j] = e2m1_to_bf16(byte & 0xFu, sc) | (e2m1_to_bf16((byte >> 4) & 0xFu, sc) << 16);
        }
        buf_store128(ro, base == BUF_OOB ? BUF_OOB : base + 16 * q, o);
      }
    }
  }
}

// The same dequantization written transposed: out [cols, rows] =
// deq(codes)^T (a 16-bit dgrad's weight operand, from the forward's tiles).
// A workgroup takes 64 x 64 values: thread t dequantizes 16 values of row
// t / 4 into LDS at their transposed places, then writes 32 contiguous bytes
// of output row (column) t / 4.  rows and cols are multiples of 32, so a
// 32-value piece is wholly inside or outside.
__global__ __launch_bounds__(256) void k_dequant_tile32_t(const uint8_t* __restrict__ codes,
                                                          const uint8_t* __restrict__ scales,
                                                          uint32_t rows, uint32_t cols,
                                                          uint16_t* __restrict__ out) {
  __shared__ uint16_t tr[64][64 + 2];
  const uint32_t nbx = (cols + 63) / 64;
  const uint32_t r0 = (blockIdx.x / nbx) * 64, c0 = (blockIdx.x % nbx) * 64;
  const int t = threadIdx.x;
  const uint32_t cpr = cols >> 1, spr = cols >> 5;
  {
    const int rl = t >> 2, cl = (t & 3) * 16;               // 16 values: columns cl .. cl+15
    const uint32_t r = r0 + rl, c = c0 + cl;
    const bool ok = r < rows && c < cols;
    const auto rc = make_rsrc(codes, static_cast<uint64_t>(rows) * cpr);
    const u32x2 w = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, static_cast<int>(ok ? r * cpr + (c >> 1) : BUF_OOB), 0, 0));
    const int sc = ok ? scales[(r >> 5) * spr + (c >> 5)] : 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) tr[cl + k][rl] = static_cast<uint16_t>(e2m1_to_bf16((w[k >> 3] >> (4 * (k & 7))) & 0xFu, sc));
  }
  __syncthreads();
  const int cl = t >> 2, rl = (t & 3) * 16;                 // output row c0 + cl, 16 values from rl
  const uint32_t c = c0 + cl, r = r0 + rl;
  const bool ok = c < cols && r < rows;
  const auto ro = make_rsrc(out, static_cast<uint64_t>(rows) * cols * 2);
  uint32_t v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = tr[cl][rl + 2 * k] | (static_cast<uint32_t>(tr[cl][rl + 2 * k + 1]) << 16);
  const uint32_t base = ok ? (c * rows + r) * 2 : BUF_OOB;
  buf_store128(ro, base, u32x4{v[0], v[1], v[2], v[3]});
  buf_store128(ro, base == BUF_OOB ? BUF_OOB : base + 16, u32x4{v[4], v[5], v[6], v[7]});
}

hipError_t launch_quant_row32(const uint16_t* in, const uint16_t* in2, int act, int64_t rows,
                              int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                              hipStream_t st, bool streaming) {
  const uint64_t nblk = static_cast<uint64_t>(rows) * (cols / 32);
  uint64_t grid = (nblk + 1023) / 1024;             // 1024 blocks per workgroup pass
  if (grid > 16384) grid = 16384;
  const dim3 g(static_cast<uint32_t>(grid));
  const uint32_t r = static_cast<uint32_t>(rows), c = static_cast<uint32_t>(cols);
#define FT_QR(A, C, N) hipLaunchKernelGGL((k_quant_row32<A, C, N>), g, dim3(256), 0, st, in, in2, r, c, ld, codes, scales)
#define FT_QRA(A) do { if (ld == cols) FT_QR(A, true, false); else FT_QR(A, false, false); } while (0)
  if (streaming && act == 0) {
    // stand-alone quantization: the codes are not read again right away
    if (ld == cols) FT_QR(0, true, true); else FT_QR(0, false, true);
  } else if (act == 1) FT_QRA(1);
  else if (act == 2) FT_QRA(2);
  else FT_QRA(0);
#undef FT_QRA
#undef FT_QR
  return hipGetLastError();
}

hipError_t launch_quant_tile32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                               uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                               uint8_t* scales_t, hipStream_t st) {
  if (!codes_t) {
    // one layout: 32 x 256 pieces, each wave on its own (more workgroups
    // in flight than the 256x256 tiles the transpose needs)
    const uint32_t n = static_cast<uint32_t>(((cols + 255) / 256) * ((rows / 32 + 3) / 4));
    hipLaunchKernelGGL(k_quant_tile32, dim3(n), dim3(256), 0, st, in, static_cast<uint32_t>(rows),
                       static_cast<uint32_t>(cols), ld, codes, scales);
  } else {
    const uint32_t n = static_cast<uint32_t>(((cols + 255) / 256) * ((rows + 255) / 256));
    hipLaunchKernelGGL(k_quant_dual<true>, dim3(n), dim3(512), 0, st, in, static_cast<uint32_t>(rows),
                       static_cast<uint32_t>(cols), ld, codes, scales, codes_t, scales_t);
  }
  return hipGetLastError();
}

hipError_t launch_quant_row32_t(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, hipStream_t st) {
  const uint32_t n = static_cast<uint32_t>(((cols + 255) / 256) * ((rows + 255) / 256));
  hipLaunchKernelGGL(k_quant_dual<false>, dim3(n), dim3(512), 0, st, in, static_cast<uint32_t>(rows),
                     static_cast<uint32_t>(cols), ld, codes, scales, codes_t, scales_t);
  return hipGetLastError();
}

hipError_t launch_dequant_tile32_t(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                   int64_t cols, uint16_t* out, hipStream_t st) {
  const int64_t nb = ((rows + 63) / 64) * ((cols + 63) / 64);
  hipLaunchKernelGGL(k_dequant_tile32_t, dim3(static_cast<uint32_t>(nb)), dim3(256), 0, st, codes,
                     scales, static_cast<uint32_t>(rows), static_cast<uint32_t>(cols), out);
  return hipGetLastError();
}

hipError_t launch_dequant_tile32(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int64_t cols, uint16_t* out, hipStream_t st) {
  const int64_t lanes = rows * (cols / 32);
  int64_t grid = (lanes + 511) / 512;                      // two row pieces per lane
  if (grid < 1) grid = 1;
  if (grid > 16384) grid = 16384;
  hipLaunchKernelGGL(k_dequant_tile32, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, codes,
                     scales, static_cast<uint32_t>(rows), static_cast<uint32_t>(cols), out);
  return hipGetLastError();
}

// Plan of the fused kernel: columns per split, splits and workgroups per
// split.  KC: 256 when that still gives one row block and split per CU of
// the device, else 128.  (KC = 512, one workgroup per CU with two register
// sets, measured slower on every layer of a DiT block: QKV backward 46.8 ->
// 42.1 us, MLP forward 56 -> 47.6 us at 256, while 128 was slower again.)
// Workgroups per split: as many as fit on the device at once (LDS allows
// two per CU at KC = 256, four at 128, half that for ranks above 64), at
// most one per row block.  The device's CU count (256 on an MI355X; 256 when
// no device is current, as for a workspace query on a host without one)
// sets the plan, so the workspace size is that of the device it runs on.
struct QDPlan {
  int kc;
  uint32_t nrb, splits, G;
};
static uint32_t plan_cus() {
  const int c = cu_count();
  return c > 0 ? static_cast<uint32_t>(c) : 256u;
}
static QDPlan quant_down_plan(int64_t rows, int64_t cols, int R, int dbr) {
  QDPlan p;
  const uint32_t cus = plan_cus();
  const int64_t rb = (rows + 63) / 64;
  p.kc = rb * ((cols + 255) / 256) >= cus ? 256 : 128;
  (void)dbr;                                   // both widths hold the dB accumulators
  p.nrb = static_cast<uint32_t>(rb);
  p.splits = static_cast<uint32_t>((cols + p.kc - 1) / p.kc);
  const uint32_t per_cu = static_cast<uint32_t>(512 / p.kc) / (R > 64 ? 2u : 1u);
  uint32_t G = cus * per_cu / p.splits;
  p.G = G < 1 ? 1 : (G > p.nrb ? p.nrb : G);
  return p;
}

// Adapter rank groups whose dB is fused into the kernel (0: not fused).
static int quant_down_dbr(int rl) { return rl > 0 && rl <= 64 ? (rl + 15) / 16 : 0; }

// Rank groups of 16 the kernel is instantiated for: 1-4, 6 and 8 (5 and 7
// run as 6 and 8, the extra ranks zero).
static int quant_down_nrg(int R) {
  const int g = (R + 15) / 16;
  return g <= 4 ? g : g <= 6 ? 6 : 8;
}

size_t quant_down_part_bytes(int64_t rows, int64_t cols, int R, int rl_db) {
  if (R == 0) return 0;
  const QDPlan p = quant_down_plan(rows, cols, R, quant_down_dbr(rl_db));
  const int64_t nrg = quant_down_nrg(R);
  return static_cast<size_t>(p.splits) * p.nrb * 4 * nrg * 256 * sizeof(float);
}

int quant_down_db_chunks(int64_t rows, int64_t cols, int R, int rl) {
  const int dbr = quant_down_dbr(rl);
  return dbr ? static_cast<int>(quant_down_plan(rows, cols, R, dbr).G) : 0;
}

size_t quant_down_db_bytes(int64_t rows, int64_t cols, int R, int rl) {
  const int dbr = quant_down_dbr(rl);
  if (!dbr) return 0;
  const QDPlan p = quant_down_plan(rows, cols, R, dbr);
  return static_cast<size_t>(p.G) * dbr * 16 * cols * sizeof(float);
}

// Forward: act 0 or 1, no dB.  Backward: act 0 or 2, dB fused (1 to 4 rank
// groups, never more than the kernel's NRG: r_l <= R) or not.
template <int NRG, int NS>
static void launch_qd(const QDArgs& a, dim3 grid, int act, int dbr, hipStream_t st) {
#define FT_QDA(ACT, D) hipLaunchKernelGGL((k_quant_down<NRG, NS, ACT, D>), grid, dim3(256), 0, st, a)
#define FT_QDB(D)                                        \
  do {                                                   \
    if constexpr (D <= NRG) {                            \
      if (act == 2) FT_QDA(2, D); else FT_QDA(0, D);     \
    }                                                    \
  } while (0)
  if (act == 1) {
    FT_QDA(1, 0);
  } else {
    switch (dbr) {
      case 0: FT_QDB(0); break;
      case 1: FT_QDB(1); break;
      case 2: FT_QDB(2); break;
      case 3: FT_QDB(3); break;
      default: FT_QDB(4); break;
    }
  }
#undef FT_QDB
#undef FT_QDA
}

hipError_t launch_quant_down(const uint16_t* in, const uint16_t* in2, int act, int64_t rows,
                             int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                             const RankRows& pr, uint16_t* out_lr, uint16_t* out_pad,
                             const RankRows& cp, int64_t cp_rows, uint16_t* cp_dst, float* part,
                             const DbFuse* db, hipStream_t st, bool cp_planes) {
  const int R = pr.r0 + pr.r1;
  const int dbr = db ? quant_down_dbr(db->rl) : 0;
  if (db && !dbr) return hipErrorInvalidValue;
  const QDPlan pl = quant_down_plan(rows, cols, R, dbr);
  const int kc = pl.kc;
  const uint32_t nrb = pl.nrb, splits = pl.splits, G = pl.G;
  QDArgs a{in, in2, static_cast<uint32_t>(rows), static_cast<uint32_t>(cols), ld, codes, scales,
           pr, R, G, part,
           db ? db->u : nullptr, db ? db->ld_u : 0, db ? db->r0 : 0, db ? db->rl : 0,
           db ? db->part : nullptr};
  const dim3 grid(splits * G);
  const int nrg = quant_down_nrg(R);
  if (dbr > nrg) return hipErrorInvalidValue;
#define FT_QD_NS(NRG)                                                                         \
  do {                                                                                        \
    if (kc == 256) launch_qd<NRG, 2>(a, grid, act, dbr, st);                                  \
    else launch_qd<NRG, 1>(a, grid, act, dbr, st);                                            \
  } while (0)
  switch (nrg) {
    case 1: FT_QD_NS(1); break;
    case 2: FT_QD_NS(2); break;
    case 3: FT_QD_NS(3); break;
    case 4: FT_QD_NS(4); break;
    case 6: FT_QD_NS(6); break;
    default: FT_QD_NS(8); break;
  }
#undef FT_QD_NS
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  (void)nrb;
  return launch_rank_reduce(part, rows, static_cast<int>(splits), R, out_lr, out_pad, cp, cp_rows,
                            cp_dst, st, cp_planes);
}

int rank_reduce_nrg(int R) { return R > 0 ? quant_down_nrg(R) : 0; }

hipError_t launch_rank_reduce(const float* part, int64_t rows, int splits, int R, uint16_t* out_lr,
                              uint16_t* out_pad, const RankRows& cp, int64_t cp_rows,
                              uint16_t* cp_dst, hipStream_t st, bool cp_planes) {
  if (R <= 0 || splits < 1) return hipErrorInvalidValue;
  const uint32_t nrb = static_cast<uint32_t>((rows + 63) / 64);
  const int nrg = quant_down_nrg(R);
  RRArgs b{part, static_cast<uint32_t>(rows), static_cast<uint32_t>(splits), R, rank_pad(R), out_lr,
           out_pad, cp, cp_rows, cp_dst, cp_planes ? 1 : 0};
  const uint64_t ncopy = cp_planes ? (static_cast<uint64_t>(rank_pad(R)) * (cp_rows / 32) + 255) / 256
                                   : (static_cast<uint64_t>(cp_rows) * (rank_pad(R) / 8) + 255) / 256;
  const dim3 rgrid(static_cast<uint32_t>(nrb * 4 + ncopy));
#define FT_RR(NRG) hipLaunchKernelGGL((k_rank_reduce<NRG>), rgrid, dim3(256), 0, st, b)
  switch (nrg) {
    case 1: FT_RR(1); break;
    case 2: FT_RR(2); break;
    case 3: FT_RR(3); break;
    case 4: FT_RR(4); break;
    case 6: FT_RR(6); break;
    default: FT_RR(8); break;
  }
#undef FT_RR
  return hipGetLastError();
}

}  // namespace ft
