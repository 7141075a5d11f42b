// Internal launchers of libfourtune (host side).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ft {

// A rank-R operand stored rank-major: rank r < r0 is row r of p0, rank
// r >= r0 row r - r0 of p1; every row holds `ld` bf16 values (ld % 8 == 0,
// rows 16-byte aligned).
struct RankRows {
  const uint16_t* p0;
  const uint16_t* p1;
  int r0, r1;
  int64_t ld;
};

// Compute units of the current device (cached per device); 0 if unknown.
int cu_count();

// Input activation of the row quantizers (FT_ACT_* of the C ABI): 0 none,
// 1 gelu(in), 2 in * gelu'(in2) with in2 of the same shape and stride.
// quantize.hip
hipError_t launch_quant_row32(const uint16_t* in, const uint16_t* in2, int act, int64_t rows,
                              int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                              hipStream_t st, bool streaming = false);
// codes_t / scales_t: optional transposed copy (both null or both set).
hipError_t launch_quant_tile32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                               uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                               uint8_t* scales_t, hipStream_t st);
hipError_t launch_quant_row32_t(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, hipStream_t st);
// Ranks of the zero-padded rank operands the GEMM reads: 64 whenever there
// is a rank part (two 32-rank steps per tile), 128 (FT_MAX_RANK, four steps)
// above 64.
inline int rank_pad(int R) { return R > 64 ? 128 : R > 0 ? 64 : 0; }

// Row quantization fused with the down-projection out_lr = bf16(in . pr^T)
// (pr rank-major, `cols` values per rank), as two launches (partial sums per
// column range into `part`, then their ordered sum).  Also writes out_pad
// [rows, rank_pad(R)], the same values zero-padded, and the transposed copy
// cp_dst [cp_rows, rank_pad(R)] of the rank-major operand cp (cp_planes: cp
// as the nibble planes [4 rank_pad(R), cp_rows / 2] bytes of the GEMM's
// transposing b read, same size; quantize.hip, copy_rank_planes).  `part`
// needs quant_down_part_bytes(rows, cols, R, db ? db->rl : 0) bytes.
// db (backward, optional): also the adapter-gradient partials
//   db->part[j][r][c] = sum over the rows workgroup j of a split visits of
//                       u[row][r0 + r] * act(in)[row][c],   r < rl <= 64,
// j < quant_down_db_chunks(rows, cols, R, rl); the rows >= rl of a 16-rank
// group are zero.  quant_down_db_bytes(rows, cols, R, rl) bytes.
struct DbFuse {
  const uint16_t* u;              // bf16 [rows, ld_u]
  int64_t ld_u;
  int r0, rl;
  float* part;
};
hipError_t launch_quant_down(const uint16_t* in, const uint16_t* in2, int act, int64_t rows,
                             int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                             const RankRows& pr, uint16_t* out_lr, uint16_t* out_pad,
                             const RankRows& cp, int64_t cp_rows, uint16_t* cp_dst, float* part,
                             const DbFuse* db, hipStream_t st, bool cp_planes = false);
size_t quant_down_part_bytes(int64_t rows, int64_t cols, int R, int rl_db);
// The second kernel of launch_quant_down on its own: out_lr, out_pad and
// cp_dst as there, from partials [splits][ceil(rows/64)][4][nrg][64][4]
// fp32 (nrg = rank_reduce_nrg(R)) that another kernel wrote.
int rank_reduce_nrg(int R);
hipError_t launch_rank_reduce(const float* part, int64_t rows, int splits, int R, uint16_t* out_lr,
                              uint16_t* out_pad, const RankRows& cp, int64_t cp_rows,
                              uint16_t* cp_dst, hipStream_t st, bool cp_planes = false);
int quant_down_db_chunks(int64_t rows, int64_t cols, int R, int rl);   // 0: dB is not fused for this rl
size_t quant_down_db_bytes(int64_t rows, int64_t cols, int R, int rl);

// Dequantize 32x32-tile MXFP4 data to bf16: out [rows, cols] from codes
// [rows, cols/2] and tile scales [rows/32, cols/32]; rows % 32 == 0,
// cols % 32 == 0.
hipError_t launch_dequant_tile32(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int64_t cols, uint16_t* out, hipStream_t st);
// The same, written transposed: out [cols, rows].
hipError_t launch_dequant_tile32_t(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                   int64_t cols, uint16_t* out, hipStream_t st);

// lora.hip: out[r][i] = sum_m act(big)[m][i] * small[m][r0 + r], r < rl,
// act as for the row quantizers (big2 is the second input of act 2).
struct LoraGradArgs {
  int64_t M, I;                   // rows, columns of big
  const uint16_t* big;            // bf16 [M, I]
  const uint16_t* big2;           // bf16 [M, I], act 2 only
  int act;
  const uint16_t* small;          // bf16 [M, ld_small], columns r0 .. r0+rl used
  int ld_small, r0, rl;
  void* out;                      // [rl, I]
  int out_f32;                    // 0 bf16, 1 fp32
  float* part;                    // workspace: fp32 partials per 512-token chunk
  int nchunk;                     // partials to add (set by launch_lora_grads unless precomputed)
};

// gemm.hip: out[m][j] = sum_red deq(a)[m][red] deq(b)[j][red] + sum_r lm[m][r] lo[j][r]
// forward: a = Qrow(X) [M, K], b = Qtile(W) [N, K], lm = U, lo = [L2^T | B^T]
// dgrad  : a = Qrow(dY) [M, N], b = Qtile(W) [N, K] read transposed
//          (b_transposed), lm = P, lo = [L1 | A] (with b_transposed and a
//          reduction that is a multiple of 128: lo as nibble planes)
// The rank operands are the zero-padded copies, rank_pad(R) = 32 * nlr ranks.
struct GemmArgs {
  int64_t M, RED, NOUT;           // rows, reduction length, output columns
  const uint8_t* a_codes;         // [M, RED/2]
  const uint8_t* a_scales;        // [M, RED/32]
  const uint8_t* b_codes;         // [NOUT, RED/2]
  const uint8_t* b_scales;        // [NOUT/32, RED/32] (one scale per 32x32 tile), or
                                  // [NOUT, RED/32] with b_row_scales (1x32 row blocks)
  const uint16_t* lm;             // bf16 [M, 32 * nlr], may be null when nlr == 0
  const uint16_t* lo;             // bf16 [NOUT, 32 * nlr]
  int nlr;                        // 32-rank groups: 0, 2 or 4 (rank_pad / 32)
  uint16_t* out;                  // bf16 [M, NOUT]
  // bf16 main product instead of the 4-bit one (a16 set: codes and scales
  // are not read): out = a16 b16^T + lm lo^T; RED % 32 == 0.
  const uint16_t* a16;            // bf16 [M, RED]
  const uint16_t* b16;            // bf16 [NOUT, RED]
  int b_row_scales;               // b quantized in 1x32 row blocks (group-wise weights)
  // b given as the 32x32-tile weight of the other product, stored
  // [RED, NOUT/2] with tile scales [RED/32, NOUT/32]: b[j][red] is read as
  // element (red, j) (the dgrad on the forward's weight)
  int b_transposed;
  // Split reduction, for outputs of few tiles (gemm_split_plan): splits
  // units per tile, each over split_pairs pairs of 128-element steps, write
  // fp32 sums to part [splits, M, NOUT]; a second kernel adds them in split
  // order, adds lm lo^T and rounds to out.  splits <= 1: one pass.
  int splits, split_pairs;
  float* part;
  // MLP fusion (e_codes set): the forward of the first linear of an MLP
  // block, whose output h feeds gelu and the second linear.  Besides out =
  // h, each tile's epilogue writes, from the same rounded values, the
  // second linear's quantized input Qrow(gelu(h)) (e_codes [M, NOUT/2],
  // e_scales [M, NOUT/32]) and the fp32 sums of its down-projection
  // gelu(h) D2 over the tile's 256 columns (e_part, in the partial layout
  // of the fused quantizer's 256-column splits, which launch_rank_reduce
  // adds up: [ceil(NOUT/256)][ceil(M/64)][4][e_nrg][64][4]).  e_pr: D2^T
  // rank-major, e_R ranks of NOUT values; e_nrg = rank_reduce_nrg(e_R)
  // (0 when e_R == 0: codes and scales only).  Pipelined kernel, b as
  // 32x32 tiles, no split (gemm_mlp_ok).
  // e_h set (the backward mirror, on the dgrad of the second linear with b
  // read transposed): the output is written as dY1 = bf16(acc gelu'(h))
  // with h = e_h [M, NOUT] (the first linear's saved output), and dY1 is
  // what is quantized and projected (e_pr: the first linear's V1).
  uint8_t* e_codes;
  uint8_t* e_scales;
  float* e_part;
  RankRows e_pr;
  int e_R, e_nrg;
  const uint16_t* e_h;
  // The adapter gradients beside a transposed-weight product (b_transposed,
  // no MLP epilogue) whose tiles leave CUs free: the launch has gemm_wgs
  // workgroups for the product and side_wgs more, which compute lora_a
  // (dA, X without an activation, rl <= 64) whole and add lora_b's
  // partials (dB from the backward quantizer, lora_b.nchunk > 0; none when
  // 0), with the bits the adapter-gradient kernels give (side_wgs = 0: none).
  LoraGradArgs lora_a, lora_b;
  uint32_t gemm_wgs, side_wgs;
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// Workgroups of the product kernel launch_gemm starts for g, side
// workgroups not counted (0 when no device is current): a persistent grid
// of at most one per CU for the pipelined kernel.
uint32_t gemm_workgroups(const GemmArgs& g);
// The fused-epilogue instantiations (g.e_codes set), gemm_mlp.hip;
// launch_gemm hands such calls over.
hipError_t launch_gemm_mlp(const GemmArgs& g, hipStream_t st);
// The split plan of a 4-bit product [M, RED] x [RED, NOUT] (RED % 128 == 0):
// splits > 1 when the output has at most 128 tiles of 256 x 256 and the
// shorter units outweigh the traffic of their sums (gemm.hip); fixed by the
// shapes, not the device.
struct SplitPlan {
  int splits, pairs;
};
SplitPlan gemm_split_plan(int64_t M, int64_t RED, int64_t NOUT);
// Outputs of at most 16 rows with a 4-bit product over a multiple of 128
// and b stored row-wise (not the transposed read): one streaming kernel
// (k_gemm_rows), no split; launch_gemm takes that path by itself.
inline bool gemm_rows_ok(int64_t M, int64_t RED, bool bf, bool b_transposed) {
  return M >= 1 && M <= 16 && RED > 0 && (RED & 127) == 0 && !bf && !b_transposed;
}
// The MLP-fused forward GEMM applies: a 4-bit product over a multiple of
// 128 on 32x32-tile weights that runs the pipelined kernel in one pass
// (more than 16 rows, no split), with D2 of at most 64 ranks.
inline bool gemm_mlp_ok(int64_t M, int64_t RED, int64_t NOUT, int R2) {
  return M > 16 && RED > 0 && (RED & 127) == 0 && (NOUT & 31) == 0 && R2 >= 0 && R2 <= 64 &&
         gemm_split_plan(M, RED, NOUT).splits <= 1;
}
inline size_t gemm_split_bytes(int64_t M, int64_t RED, int64_t NOUT) {
  const SplitPlan p = gemm_split_plan(M, RED, NOUT);
  // (with few rows the streaming kernel may run instead; the bytes stay
  // reserved either way)
  return p.splits > 1 ? static_cast<size_t>(p.splits) * M * NOUT * sizeof(float) : 0;
}

// dA and dB of one backward: one launch computes the partials of both
// problems, a second adds them in chunk order.  dB_done: dB's partials
// [dB.nchunk][16 ceil(rl/16)][I] are already in dB.part (made by the
// backward quantize kernel); only the reduction runs for dB.
hipError_t launch_lora_grads(const LoraGradArgs& dA, const LoraGradArgs& dB, bool dB_done,
                             hipStream_t st);
size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl);
// 512-token chunks and 64-column blocks of one adapter-gradient problem.
uint32_t lora_chunks(int64_t M);
uint32_t lora_col_blocks(int64_t I);

// scratch.hip: the workspace of the forward that allocates nothing, a
// device array of kNoAllocScratchBytes (FT_NOALLOC_SCRATCH_BYTES of the C
// ABI) per GPU; nullptr if the current device's copy cannot be located.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
void* noalloc_scratch();

// act.hip: out = bf16(gelu(h)) (act 1) or bf16(g * gelu'(h)) (act 2), n elements.
hipError_t launch_act(int act, const uint16_t* h, const uint16_t* g, int64_t n, uint16_t* out,
                      hipStream_t st);

}  // namespace ft
