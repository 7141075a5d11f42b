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
// Ranks of the zero-padded rank operands the GEMM reads: 64 (FT_MAX_RANK)
// whenever there is a rank part, so that every tile has the same two rank
// steps.
inline int rank_pad(int R) { return R > 0 ? 64 : 0; }

// Row quantization fused with the down-projection out_lr = bf16(in . pr^T)
// (pr rank-major, `cols` values per rank), as two launches (partial sums per
// column range into `part`, then their ordered sum).  Also writes out_pad
// [rows, rank_pad(R)], the same values zero-padded, and the transposed copy
// cp_dst [cp_rows, rank_pad(R)] of the rank-major operand cp.  `part` needs
// quant_down_part_bytes(rows, cols, R, db ? db->rl : 0) bytes.
// db (backward, optional): also the adapter-gradient partials
//   db->part[j][r][c] = sum over the rows workgroup j of a split visits of
//                       u[row][r0 + r] * act(in)[row][c],   r < rl <= 32,
// j < quant_down_db_chunks(rows, cols, rl); the rows >= rl of a 16-rank
// group are zero.  quant_down_db_bytes(rows, cols, rl) bytes.
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
                             const DbFuse* db, hipStream_t st);
size_t quant_down_part_bytes(int64_t rows, int64_t cols, int R, int rl_db);
int quant_down_db_chunks(int64_t rows, int64_t cols, int rl);   // 0: dB is not fused for this rl
size_t quant_down_db_bytes(int64_t rows, int64_t cols, int rl);

// Dequantize 32x32-tile MXFP4 data to bf16: out [rows, cols] from codes
// [rows, cols/2] and tile scales [rows/32, cols/32]; rows % 32 == 0,
// cols % 32 == 0.
hipError_t launch_dequant_tile32(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int64_t cols, uint16_t* out, hipStream_t st);

// gemm.hip: out[m][j] = sum_red deq(a)[m][red] deq(b)[j][red] + sum_r lm[m][r] lo[j][r]
// forward: a = Qrow(X) [M, K], b = Qtile(W) [N, K], lm = U, lo = [L2^T | B^T]
// dgrad  : a = Qrow(dY) [M, N], b = Qtile(W)^T [K, N], lm = P, lo = [L1 | A]
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
  int nlr;                        // 32-rank groups: 0 or 2 (rank_pad)
  uint16_t* out;                  // bf16 [M, NOUT]
  // bf16 main product instead of the 4-bit one (a16 set: codes and scales
  // are not read): out = a16 b16^T + lm lo^T; RED % 32 == 0.
  const uint16_t* a16;            // bf16 [M, RED]
  const uint16_t* b16;            // bf16 [NOUT, RED]
  int b_row_scales;               // b quantized in 1x32 row blocks (group-wise weights)
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

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
// dA and dB of one backward: one launch computes the partials of both
// problems, a second adds them in chunk order.  dB_done: dB's partials
// [dB.nchunk][16 ceil(rl/16)][I] are already in dB.part (made by the
// backward quantize kernel); only the reduction runs for dB.
hipError_t launch_lora_grads(const LoraGradArgs& dA, const LoraGradArgs& dB, bool dB_done,
                             hipStream_t st);
size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl);

// act.hip: out = bf16(gelu(h)) (act 1) or bf16(g * gelu'(h)) (act 2), n elements.
hipError_t launch_act(int act, const uint16_t* h, const uint16_t* g, int64_t n, uint16_t* out,
                      hipStream_t st);

}  // namespace ft
