// MLP fusion (FourTune, "3.3 Kernel Fusion for Efficiency / MLP Fusion"):
// the instantiations of k_gemm_pipe whose epilogue also makes the next
// linear's quantized input and down-projection sums (the forward of an MLP
// block's first linear) or, mirrored, the first linear's quantized incoming
// gradient and its down-projection sums (the dgrad of the second linear).
// The epilogue itself is store_tile_mlp in gemm_pipe.hpp.
#include "gemm_pipe.hpp"

namespace ft {

hipError_t launch_gemm_mlp(const GemmArgs& g, hipStream_t st) {
  if (!g.e_codes) return hipErrorInvalidValue;
  const uint32_t n = static_cast<uint32_t>(((g.NOUT + BN - 1) / BN) * ((g.M + BM - 1) / BM));
  const bool bf = g.a16 != nullptr;
  // the pipelined kernel on 32x32-tile weights, one pass; the forward
  // reads them row-wise, the backward mirror (e_h) transposed
  const bool mirror = g.e_h != nullptr;
  if (bf || g.M <= 16 || (g.RED & 127) != 0 || g.b_row_scales || (g.b_transposed != 0) != mirror ||
      g.splits > 1 || !g.e_scales || g.e_nrg < 0 || g.e_nrg > 4 || (g.e_nrg > 0 && !g.e_part) ||
      (g.NOUT & 31) != 0)
    return hipErrorInvalidValue;
  if (g.nlr != 0 && g.nlr != 2 && g.nlr != 4) return hipErrorInvalidValue;
  const int cus = cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  const uint32_t grid = n < static_cast<uint32_t>(cus) ? n : static_cast<uint32_t>(cus);
#define FT_GE(NL, E) hipLaunchKernelGGL((k_gemm_pipe<NL, (E > 5 ? 3 : 0), E>), dim3(grid), dim3(256), 0, st, g)
#define FT_GEN(E) do { if (g.nlr == 4) FT_GE(4, E); else if (g.nlr > 0) FT_GE(2, E); else FT_GE(0, E); } while (0)
  const int e = (mirror ? 6 : 1) + g.e_nrg;
  switch (e) {
    case 1: FT_GEN(1); break;
    case 2: FT_GEN(2); break;
    case 3: FT_GEN(3); break;
    case 4: FT_GEN(4); break;
    case 5: FT_GEN(5); break;
    case 6: FT_GEN(6); break;
    case 7: FT_GEN(7); break;
    case 8: FT_GEN(8); break;
    case 9: FT_GEN(9); break;
    default: FT_GEN(10); break;
  }
#undef FT_GEN
#undef FT_GE
  return hipGetLastError();
}

}  // namespace ft
