// Internal launchers of libfourtune (host side).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ft {

// A rank-R operand given as two bf16 pieces along the rank axis: element
// (c, r) = r < r0 ? p0[c*s0c + r*s0r] : p1[c*s1c + (r-r0)*s1r], where c runs
// over the long axis (K or N) of the layer.
struct LowRankPieces {
  const uint16_t* p0;
  int64_t s0c, s0r;
  int r0;
  const uint16_t* p1;
  int64_t s1c, s1r;
  int r1;
};

// quantize.hip
hipError_t launch_quant_row32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, uint8_t* scales, hipStream_t st);
// codes_t / scales_t: optional transposed copy (both null or both set).
hipError_t launch_quant_tile32(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                               uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                               uint8_t* scales_t, hipStream_t st);
hipError_t launch_quant_row32_t(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                                uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                                uint8_t* scales_t, hipStream_t st);
// Row quantization fused with the down-projection; `cnt` is a workspace array
// of 64-bit arrival slots (any contents), `epoch` a value unique to this call.
hipError_t launch_quant_down(const uint16_t* in, int64_t rows, int64_t cols, int64_t ld,
                             uint8_t* codes, uint8_t* scales, const LowRankPieces& pr,
                             uint16_t* out_lr, float* part, unsigned long long* cnt,
                             uint32_t epoch, hipStream_t st);
size_t quant_down_part_bytes(int64_t rows, int64_t cols, int R);
size_t quant_down_cnt_bytes(int64_t rows);

// gemm.hip: out[m][j] = sum_red deq(a)[m][red] deq(b)[j][red] + sum_r lm[m][r] lo[j][r]
// forward: a = Qrow(X) [M, K], b = Qtile(W) [N, K], lm = U, lo = [L2^T | B^T]
// dgrad  : a = Qrow(dY) [M, N], b = Qtile(W)^T [K, N], lm = P, lo = [L1 | A]
struct GemmArgs {
  int64_t M, RED, NOUT;           // rows, reduction length, output columns
  const uint8_t* a_codes;         // [M, RED/2]
  const uint8_t* a_scales;        // [M, RED/32]
  const uint8_t* b_codes;         // [NOUT, RED/2]
  const uint8_t* b_scales;        // [NOUT/32, RED/32] (one scale per 32x32 tile)
  const uint16_t* lm;             // bf16 [M, R], may be null when R == 0
  const uint16_t* lo0;            // bf16 [NOUT, r0]: ranks 0 .. r0-1 of lo
  const uint16_t* lo1;            // bf16 [NOUT, R - r0]: ranks r0 .. R-1
  int R, r0;
  uint16_t* out;                  // bf16 [M, NOUT]
};
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);

// lora.hip: out[i][r] = sum_m big[m][i] * small[m][r0 + r], r < rl.
struct LoraGradArgs {
  int64_t M, I;                   // rows, columns of big
  const uint16_t* big;            // bf16 [M, I]
  const uint16_t* small;          // bf16 [M, ld_small], columns r0 .. r0+rl used
  int ld_small, r0, rl;
  void* out;                      // [I, rl]
  int out_f32;                    // 0 bf16, 1 fp32
  float* part;                    // workspace partials
  unsigned long long* cnt;        // workspace arrival slots (any contents)
  uint32_t epoch;                 // unique to this call
};
// dA and dB of one backward in a single launch (both problems in one grid).
hipError_t launch_lora_grads(const LoraGradArgs& dA, const LoraGradArgs& dB, hipStream_t st);
size_t lora_grad_part_bytes(int64_t M, int64_t I, int rl);
size_t lora_grad_cnt_bytes(int64_t I);

}  // namespace ft
