// Standalone elementwise activation around the MLP's GELU, the same device
// functions the fused kernels apply as they load their inputs (FourTune,
// "3.3 Kernel Fusion for Efficiency / MLP Fusion": GeLU between the two
// linears of an MLP block):
//   act 1: out = bf16(gelu(h))              (the second linear's input)
//   act 2: out = bf16(g * gelu'(h))         (the first linear's incoming gradient)
// Memory bound; 8 elements per lane, 16-byte loads and stores.
#include "ft_device.hpp"
#include "ft_kernels.h"

namespace ft {

namespace {

template <int ACT>
__global__ __launch_bounds__(256) void k_act(const uint16_t* __restrict__ h,
                                             const uint16_t* __restrict__ g, int64_t n,
                                             uint16_t* __restrict__ out) {
  const int64_t nv = n / 8;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < nv; i += stride) {
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(h) + i);
    u32x4 o;
    if constexpr (ACT == 2) o = act_bf16x8<2>(__builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g) + i), x);
    else o = act_bf16x8<1>(x, x);
    reinterpret_cast<u32x4*>(out)[i] = o;
  }
  // tail (n % 8 elements), one thread
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (int64_t e = nv * 8; e < n; ++e) {
      const float hv = bf16_to_f32(h[e]);
      const float r = ACT == 2 ? gelu_tanh_grad_f32(hv, bf16_to_f32(g[e])) : gelu_tanh_f32(hv);
      out[e] = static_cast<uint16_t>(cvt_pk_bf16(r, 0.0f));
    }
  }
}

}  // namespace

hipError_t launch_act(int act, const uint16_t* h, const uint16_t* g, int64_t n, uint16_t* out,
                      hipStream_t st) {
  int64_t grid = (n / 8 + 255) / 256;
  if (grid < 1) grid = 1;
  if (grid > 8192) grid = 8192;
  if (act == 2) hipLaunchKernelGGL(k_act<2>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, h, g, n, out);
  else hipLaunchKernelGGL(k_act<1>, dim3(static_cast<uint32_t>(grid)), dim3(256), 0, st, h, g, n, out);
  return hipGetLastError();
}

}  // namespace ft
