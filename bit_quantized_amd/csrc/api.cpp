// libfourtune C ABI (include/fourtune.h): argument checks, workspace layout
// and kernel dispatch.  Every check runs before the first launch, so a call
// that fails has enqueued nothing.
#include "../../include/fourtune.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "ft_kernels.h"

namespace ft {

int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      return 0;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

}  // namespace ft

namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
constexpr int64_t kMaxDim = int64_t(1) << 30;
// Kernels address tensors with 32-bit buffer offsets.
constexpr int64_t kMaxBytes = (int64_t(1) << 31) - 1;

// 1 = current device is gfx950, 0 = not, -1 = unknown yet.  Cached per device.
int g_arch_ok[64];
std::once_flag g_arch_once;

ft_status device_check() {
  std::call_once(g_arch_once, [] {
    for (int& v : g_arch_ok) v = -1;
  });
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FT_EUNSUPPORTED;
  if (dev < 0 || dev >= 64) return FT_EUNSUPPORTED;
  if (g_arch_ok[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FT_EUNSUPPORTED;
    g_arch_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  }
  return g_arch_ok[dev] == 1 ? FT_OK : FT_EUNSUPPORTED;
}

ft_status launched(hipError_t e) { return e == hipSuccess ? FT_OK : FT_EDEVICE; }

// ---- optional per-kernel timing (benchmarks): hipEvents around each launch
struct TimingState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  struct Pending { int slot; hipEvent_t a, b; };
  std::vector<Pending> pending;
  std::vector<std::string> names;
  std::vector<double> total_ms;
  std::vector<int64_t> counts;
  int slot(const char* n) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == n) return static_cast<int>(i);
    names.emplace_back(n);
    total_ms.push_back(0.0);
    counts.push_back(0);
    return static_cast<int>(names.size() - 1);
  }
  hipEvent_t take() {
    if (pool.empty()) {
      hipEvent_t e = nullptr;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      return e;
    }
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  void drain() {  // caller holds mu
    for (auto& p : pending) {
      float ms = 0.f;
      if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
        total_ms[p.slot] += ms;
        counts[p.slot] += 1;
      }
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
};
TimingState g_tm;

// Brackets one launch with events when timing is on.
struct Timed {
  hipEvent_t a = nullptr, b = nullptr;
  int slot = -1;
  hipStream_t st;
  Timed(const char* name, hipStream_t s) : st(s) {
    if (!g_tm.on) return;
    std::lock_guard<std::mutex> lk(g_tm.mu);
    slot = g_tm.slot(name);
    a = g_tm.take();
    b = g_tm.take();
    if (a && b) hipEventRecord(a, st);
  }
  hipError_t done(hipError_t e) {
    if (a && b) {
      hipEventRecord(b, st);
      std::lock_guard<std::mutex> lk(g_tm.mu);
      g_tm.pending.push_back({slot, a, b});
    }
    return e;
  }
};

// Checks shared by forward and backward.
ft_status check_linear(const ft_linear* L) {
  if (!L) return FT_EINVAL;
  if (L->M < 1 || L->K < 32 || L->N < 32) return FT_ESHAPE;
  if (L->M > kMaxDim || L->K > kMaxDim || L->N > kMaxDim) return FT_ESHAPE;
  if ((L->K & 31) || (L->N & 31)) return FT_ESHAPE;
  if (L->M * L->K * 2 > kMaxBytes || L->M * L->N * 2 > kMaxBytes || L->N * L->K / 2 > kMaxBytes)
    return FT_ESHAPE;
  // the fused quantizer and the GEMM address whole 64-row blocks and
  // 256-row tiles with 32-bit offsets: the padded activations and outputs
  // must stay below 2^31 bytes as well
  if ((L->M + 256) * std::max(L->K, L->N) * 2 > kMaxBytes) return FT_ESHAPE;
  if (L->r_stab < 0 || L->r_lora < 0 || L->r_stab + L->r_lora > FT_MAX_RANK) return FT_ESHAPE;
  if (L->M * (L->r_stab + L->r_lora) * 2 > kMaxBytes) return FT_ESHAPE;
  if (!L->w_codes || !L->w_scales) return FT_EINVAL;
  if ((L->act_in != FT_ACT_NONE && L->act_in != FT_ACT_GELU_TANH) ||
      (L->act_out != FT_ACT_NONE && L->act_out != FT_ACT_GELU_TANH))
    return FT_EINVAL;
  if ((L->wt_codes == nullptr) != (L->wt_scales == nullptr)) return FT_EINVAL;
  if (L->precision < FT_W4A4G4 || L->precision > FT_W4A16G16) return FT_EINVAL;
  if (L->w_block != FT_WBLOCK_TILE32 && L->w_block != FT_WBLOCK_ROW32) return FT_EINVAL;
  // group-wise weights: 4-bit products only (the dequantizer reads tiles)
  if (L->w_block == FT_WBLOCK_ROW32 && L->precision != FT_W4A4G4) return FT_EINVAL;
  // a 16-bit product reads the weight dequantized to bf16, with 32-bit
  // offsets over its padded rows
  if (L->precision != FT_W4A4G4 &&
      (std::max(L->K, L->N) + 256) * std::min(L->K, L->N) * 2 > kMaxBytes)
    return FT_ESHAPE;
  if (L->r_stab > 0 && (!L->L1t || !L->L2)) return FT_EINVAL;
  if (L->r_lora > 0 && (!L->At || !L->B)) return FT_EINVAL;
  const void* ptrs[] = {L->w_codes, L->w_scales, L->wt_codes, L->wt_scales, L->L1t, L->L2, L->At, L->B};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  return FT_OK;
}

inline bool a16(const ft_linear* L) { return (L->precision & FT_W4A16G4) != 0; }
inline bool g16(const ft_linear* L) { return (L->precision & FT_W4A4G16) != 0; }

struct FwdLayout {
  size_t xq_codes, xq_scales, u_pad, v_pad, part, w16, x16, total;
};
FwdLayout fwd_layout(const ft_linear* L) {
  const int R = L->r_stab + L->r_lora;
  const size_t rp = static_cast<size_t>(ft::rank_pad(R));
  const bool bf = a16(L);
  FwdLayout o;
  size_t off = 0;
  o.xq_codes = off; off += bf ? 0 : align_up(static_cast<size_t>(L->M) * (L->K / 2));
  o.xq_scales = off; off += bf ? 0 : align_up(static_cast<size_t>(L->M) * (L->K / 32));
  // A16: the weight in bf16 [N, K], and act_in(X) when there is an act_in
  o.w16 = off; off += bf ? align_up(static_cast<size_t>(L->N) * L->K * 2) : 0;
  o.x16 = off; off += bf && L->act_in != FT_ACT_NONE ? align_up(static_cast<size_t>(L->M) * L->K * 2) : 0;
  o.u_pad = off; off += align_up(static_cast<size_t>(L->M) * rp * 2);     // U, zero-padded ranks
  o.v_pad = off; off += align_up(static_cast<size_t>(L->N) * rp * 2);     // [L2^T | B^T], padded
  o.part = off; off += align_up(ft::quant_down_part_bytes(L->M, L->K, R, 0));
  o.total = off;
  return o;
}

// dB's partial sums come out of the backward quantize kernel (which reads
// dY anyway) for adapter ranks up to 32; above that the adapter-gradient
// kernel reads dY again.
bool db_fused_in_quant(const ft_linear* L) {
  return L->r_lora > 0 && ft::quant_down_db_chunks(L->M, L->N, L->r_lora) > 0;
}

struct BwdLayout {
  size_t gq_codes, gq_scales, P, p_pad, d_pad, part, dA_part, dB_part, w16, g16, total;
};
BwdLayout bwd_layout(const ft_linear* L) {
  const int R = L->r_stab + L->r_lora;
  const int rl = L->r_lora;
  const size_t rp = static_cast<size_t>(ft::rank_pad(R));
  const bool bf = g16(L);
  BwdLayout o;
  size_t off = 0;
  o.gq_codes = off; off += bf ? 0 : align_up(static_cast<size_t>(L->M) * (L->N / 2));
  o.gq_scales = off; off += bf ? 0 : align_up(static_cast<size_t>(L->M) * (L->N / 32));
  // G16: the transposed weight in bf16 [K, N], and dY * act_out'(H) when
  // there is an act_out
  o.w16 = off; off += bf ? align_up(static_cast<size_t>(L->K) * L->N * 2) : 0;
  o.g16 = off; off += bf && L->act_out != FT_ACT_NONE ? align_up(static_cast<size_t>(L->M) * L->N * 2) : 0;
  o.P = off; off += align_up(static_cast<size_t>(L->M) * R * 2);
  o.p_pad = off; off += align_up(static_cast<size_t>(L->M) * rp * 2);     // P, zero-padded ranks
  o.d_pad = off; off += align_up(static_cast<size_t>(L->K) * rp * 2);     // [L1 | A], padded
  const bool db_fused = db_fused_in_quant(L);
  o.part = off; off += align_up(ft::quant_down_part_bytes(L->M, L->N, R, db_fused ? rl : 0));
  o.dA_part = off; off += align_up(rl ? ft::lora_grad_part_bytes(L->M, L->K, rl) : 0);
  o.dB_part = off;
  off += align_up(db_fused ? ft::quant_down_db_bytes(L->M, L->N, rl)
                           : (rl ? ft::lora_grad_part_bytes(L->M, L->N, rl) : 0));
  o.total = off;
  return o;
}

// The factors rank-major: D^T = [L1^T ; A^T] (rows of K values) and
// V = [L2 ; B] (rows of N values).
ft::RankRows rows_Dt(const ft_linear* L) {
  return ft::RankRows{L->L1t, L->At, L->r_stab, L->r_lora, L->K};
}
ft::RankRows rows_V(const ft_linear* L) {
  return ft::RankRows{L->L2, L->B, L->r_stab, L->r_lora, L->N};
}

}  // namespace

extern "C" {

const char* fourtune_status_string(ft_status s) {
  switch (s) {
    case FT_OK: return "ok";
    case FT_EINVAL: return "invalid argument (null pointer or bad enum value)";
    case FT_ESHAPE: return "unsupported shape";
    case FT_EALIGN: return "misaligned pointer or row stride";
    case FT_EWORKSPACE: return "workspace too small";
    case FT_EDEVICE: return "HIP launch failed";
    case FT_EUNSUPPORTED: return "no supported GPU (gfx950) is current";
  }
  return "unknown status";
}

ft_status fourtune_quantize(int mode, const uint16_t* in, int64_t rows, int64_t cols,
                            int64_t ld_in, uint8_t* codes, uint8_t* scales, uint8_t* codes_t,
                            uint8_t* scales_t, void* stream) {
  if (mode != FT_Q_ROW32 && mode != FT_Q_ROW32_T && mode != FT_Q_TILE32) return FT_EINVAL;
  if (!in || !codes || !scales) return FT_EINVAL;
  if (mode == FT_Q_ROW32_T) {
    if (!codes_t || !scales_t) return FT_EINVAL;
  } else if (mode == FT_Q_TILE32) {
    if ((codes_t == nullptr) != (scales_t == nullptr)) return FT_EINVAL;
  } else if (codes_t || scales_t) {
    return FT_EINVAL;
  }
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return FT_ESHAPE;
  if (rows * ld_in * 2 > kMaxBytes) return FT_ESHAPE;
  if (cols & 31) return FT_ESHAPE;
  if (mode != FT_Q_ROW32 && (rows & 31)) return FT_ESHAPE;
  if (ld_in < cols || (ld_in & 7)) return FT_EALIGN;
  if (!aligned16(in) || !aligned16(codes) || !aligned16(scales)) return FT_EALIGN;
  if (codes_t && !aligned16(codes_t)) return FT_EALIGN;
  if (scales_t && !aligned16(scales_t)) return FT_EALIGN;
  if (rows == 0 || cols == 0) return FT_OK;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (mode) {
    case FT_Q_ROW32:
      { Timed tm("quant_row32", st); return launched(tm.done(ft::launch_quant_row32(in, nullptr, 0, rows, cols, ld_in, codes, scales, st, true))); }
    case FT_Q_TILE32:
      { Timed tm("quant_tile32", st); return launched(tm.done(ft::launch_quant_tile32(in, rows, cols, ld_in, codes, scales, codes_t, scales_t, st))); }
    default:
    {
      Timed tm("quant_row32_t", st);
      return launched(tm.done(
          ft::launch_quant_row32_t(in, rows, cols, ld_in, codes, scales, codes_t, scales_t, st)));
    }
  }
}

ft_status fourtune_dequantize(int mode, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t cols, uint16_t* out, void* stream) {
  if (mode != FT_Q_TILE32) return FT_EINVAL;
  if (!codes || !scales || !out) return FT_EINVAL;
  if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return FT_ESHAPE;
  if ((rows & 31) || (cols & 31)) return FT_ESHAPE;
  if (rows * cols * 2 > kMaxBytes) return FT_ESHAPE;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(out)) return FT_EALIGN;
  if (rows == 0 || cols == 0) return FT_OK;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Timed tm("dequant_tile32", st);
  return launched(tm.done(ft::launch_dequant_tile32(codes, scales, rows, cols, out, st)));
}

size_t fourtune_workspace_bytes(const ft_linear* L, int is_bwd) {
  if (!L || L->M < 1 || L->K < 32 || L->N < 32 || (L->K & 31) || (L->N & 31)) return 0;
  if (L->M > kMaxDim || L->K > kMaxDim || L->N > kMaxDim) return 0;
  if (L->r_stab < 0 || L->r_lora < 0 || L->r_stab + L->r_lora > FT_MAX_RANK) return 0;
  if (L->precision < FT_W4A4G4 || L->precision > FT_W4A16G16) return 0;
  if (L->w_block != FT_WBLOCK_TILE32 && L->w_block != FT_WBLOCK_ROW32) return 0;
  return is_bwd ? bwd_layout(L).total : fwd_layout(L).total;
}

ft_status fourtune_linear_fwd(const ft_linear* L, const uint16_t* X, uint16_t* Y,
                              uint16_t* U_save, uint8_t* xq_codes, uint8_t* xq_scales,
                              void* workspace, size_t ws_bytes, void* stream) {
  if (ft_status s = check_linear(L); s != FT_OK) return s;
  const int R = L->r_stab + L->r_lora;
  if (!X || !Y) return FT_EINVAL;
  if (R > 0 && !U_save) return FT_EINVAL;
  if ((xq_codes == nullptr) != (xq_scales == nullptr)) return FT_EINVAL;
  if (a16(L) && xq_codes) return FT_EINVAL;
  const void* ptrs[] = {X, Y, U_save, xq_codes, xq_scales, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const FwdLayout lay = fwd_layout(L);
  if (ws_bytes < lay.total) return FT_EWORKSPACE;
  if (!workspace) return FT_EINVAL;
  if (ft_status s = device_check(); s != FT_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool bf = a16(L);
  // A16: no codes; the quantize stores of kernel 1 are dropped
  uint8_t* qc = bf ? nullptr : xq_codes ? xq_codes : ws + lay.xq_codes;
  uint8_t* qs = bf ? nullptr : xq_scales ? xq_scales : ws + lay.xq_scales;
  uint16_t* u_pad = reinterpret_cast<uint16_t*>(ws + lay.u_pad);
  uint16_t* v_pad = reinterpret_cast<uint16_t*>(ws + lay.v_pad);
  hipError_t e = hipSuccess;
  // act_in: X is the pre-activation h; the layer's input is gelu(h)
  const int act = L->act_in == FT_ACT_GELU_TANH ? 1 : 0;
  if (R > 0) {
    Timed tm("fwd_quant_down", st);
    e = tm.done(ft::launch_quant_down(X, nullptr, act, L->M, L->K, L->K, qc, qs, rows_Dt(L), U_save,
                                      u_pad, rows_V(L), L->N, v_pad,
                                      reinterpret_cast<float*>(ws + lay.part), nullptr, st));
  } else if (!bf) {
    Timed tm("fwd_quant_down", st);
    e = tm.done(ft::launch_quant_row32(X, nullptr, act, L->M, L->K, L->K, qc, qs, st));
  }
  if (e != hipSuccess) return FT_EDEVICE;
  ft::GemmArgs g{};
  g.M = L->M; g.RED = L->K; g.NOUT = L->N;
  g.a_codes = qc; g.a_scales = qs;
  g.b_codes = L->w_codes; g.b_scales = L->w_scales;
  g.b_row_scales = L->w_block == FT_WBLOCK_ROW32;
  g.lm = u_pad; g.lo = v_pad; g.nlr = ft::rank_pad(R) / 32; g.out = Y;
  if (bf) {
    uint16_t* w16 = reinterpret_cast<uint16_t*>(ws + lay.w16);
    {
      Timed tm("fwd_dequant_w", st);
      if (tm.done(ft::launch_dequant_tile32(L->w_codes, L->w_scales, L->N, L->K, w16, st)) != hipSuccess)
        return FT_EDEVICE;
    }
    const uint16_t* x16 = X;
    if (act) {
      uint16_t* xa = reinterpret_cast<uint16_t*>(ws + lay.x16);
      Timed tm("fwd_act", st);
      if (tm.done(ft::launch_act(1, X, nullptr, L->M * L->K, xa, st)) != hipSuccess) return FT_EDEVICE;
      x16 = xa;
    }
    g.a16 = x16; g.b16 = w16;
  }
  Timed tm("fwd_gemm", st);
  return launched(tm.done(ft::launch_gemm(g, st)));
}

ft_status fourtune_linear_bwd(const ft_linear* L, const uint16_t* dY, const uint16_t* X,
                              const uint16_t* U_save, const uint16_t* H, uint16_t* dX, void* dA, void* dB,
                              ft_dtype grad_dtype, uint16_t* P_save, uint8_t* gq_codes,
                              uint8_t* gq_scales, void* workspace, size_t ws_bytes,
                              void* stream) {
  if (ft_status s = check_linear(L); s != FT_OK) return s;
  const int R = L->r_stab + L->r_lora;
  const int rl = L->r_lora;
  if (!dY) return FT_EINVAL;
  if (dX && !L->wt_codes) return FT_EINVAL;
  if (grad_dtype != FT_BF16 && grad_dtype != FT_F32) return FT_EINVAL;
  if (rl > 0 && (!X || !U_save || !dA || !dB)) return FT_EINVAL;
  if (L->act_out != FT_ACT_NONE && !H) return FT_EINVAL;
  if ((gq_codes == nullptr) != (gq_scales == nullptr)) return FT_EINVAL;
  if (g16(L) && gq_codes) return FT_EINVAL;
  const void* ptrs[] = {dY, X, U_save, H, dX, dA, dB, P_save, gq_codes, gq_scales, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const BwdLayout lay = bwd_layout(L);
  if (ws_bytes < lay.total) return FT_EWORKSPACE;
  if (!workspace) return FT_EINVAL;
  if (ft_status s = device_check(); s != FT_OK) return s;

  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool bf = g16(L);
  // G16: no codes; the quantize stores of kernel 1 are dropped
  uint8_t* qc = bf ? nullptr : gq_codes ? gq_codes : ws + lay.gq_codes;
  uint8_t* qs = bf ? nullptr : gq_scales ? gq_scales : ws + lay.gq_scales;
  uint16_t* P = P_save ? P_save : reinterpret_cast<uint16_t*>(ws + lay.P);
  uint16_t* p_pad = reinterpret_cast<uint16_t*>(ws + lay.p_pad);
  uint16_t* d_pad = reinterpret_cast<uint16_t*>(ws + lay.d_pad);
  hipError_t e = hipSuccess;
  const bool db_fused = db_fused_in_quant(L);
  ft::DbFuse db{U_save, R, L->r_stab, rl, reinterpret_cast<float*>(ws + lay.dB_part)};
  // act_out: dY is the gradient of gelu(Y) and H the saved Y; the incoming
  // gradient of this layer is dY * gelu'(H)
  const int act = L->act_out == FT_ACT_GELU_TANH ? 2 : 0;
  const uint16_t* h2 = act ? H : nullptr;
  if (R > 0) {
    Timed tm("bwd_quant_down", st);
    e = tm.done(ft::launch_quant_down(dY, h2, act, L->M, L->N, L->N, qc, qs, rows_V(L), P, p_pad,
                                      rows_Dt(L), dX ? L->K : 0, d_pad,
                                      reinterpret_cast<float*>(ws + lay.part),
                                      db_fused ? &db : nullptr, st));
  } else if (!bf) {
    Timed tm("bwd_quant_down", st);
    e = tm.done(ft::launch_quant_row32(dY, h2, act, L->M, L->N, L->N, qc, qs, st));
  }
  if (e != hipSuccess) return FT_EDEVICE;
  if (dX) {
    ft::GemmArgs g{};
    g.M = L->M; g.RED = L->N; g.NOUT = L->K;
    g.a_codes = qc; g.a_scales = qs;
    g.b_codes = L->wt_codes; g.b_scales = L->wt_scales;
    g.b_row_scales = L->w_block == FT_WBLOCK_ROW32;
    g.lm = p_pad; g.lo = d_pad; g.nlr = ft::rank_pad(R) / 32; g.out = dX;
    if (bf) {
      uint16_t* w16 = reinterpret_cast<uint16_t*>(ws + lay.w16);
      {
        Timed tm("bwd_dequant_w", st);
        if (tm.done(ft::launch_dequant_tile32(L->wt_codes, L->wt_scales, L->K, L->N, w16, st)) != hipSuccess)
          return FT_EDEVICE;
      }
      const uint16_t* g16p = dY;
      if (act) {
        uint16_t* ga = reinterpret_cast<uint16_t*>(ws + lay.g16);
        Timed tm("bwd_act", st);
        if (tm.done(ft::launch_act(2, H, dY, L->M * L->N, ga, st)) != hipSuccess) return FT_EDEVICE;
        g16p = ga;
      }
      g.a16 = g16p; g.b16 = w16;
    }
    Timed tm("bwd_gemm_dgrad", st);
    if (tm.done(ft::launch_gemm(g, st)) != hipSuccess) return FT_EDEVICE;
  }
  if (rl > 0) {
    const int f32 = grad_dtype == FT_F32 ? 1 : 0;
    ft::LoraGradArgs a{};
    a.M = L->M; a.I = L->K; a.big = X; a.small = P; a.ld_small = R; a.r0 = L->r_stab; a.rl = rl;
    a.big2 = nullptr; a.act = L->act_in == FT_ACT_GELU_TANH ? 1 : 0;
    a.out = dA; a.out_f32 = f32;
    a.part = reinterpret_cast<float*>(ws + lay.dA_part);
    ft::LoraGradArgs b = a;
    b.I = L->N; b.big = dY; b.small = U_save;
    b.big2 = L->act_out == FT_ACT_GELU_TANH ? H : nullptr;
    b.act = L->act_out == FT_ACT_GELU_TANH ? 2 : 0;
    b.out = dB;
    b.part = reinterpret_cast<float*>(ws + lay.dB_part);
    b.nchunk = db_fused ? ft::quant_down_db_chunks(L->M, L->N, rl) : 0;
    Timed tm("bwd_lora_grads", st);
    if (tm.done(ft::launch_lora_grads(a, b, db_fused, st)) != hipSuccess) return FT_EDEVICE;
  }
  return FT_OK;
}

ft_status fourtune_act_fwd(int act, const uint16_t* h, int64_t n, uint16_t* out, void* stream) {
  if (act != FT_ACT_GELU_TANH) return FT_EINVAL;
  if (!h || !out) return FT_EINVAL;
  if (n < 0 || n * 2 > kMaxBytes) return FT_ESHAPE;
  if (!aligned16(h) || !aligned16(out)) return FT_EALIGN;
  if (n == 0) return FT_OK;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Timed tm("act_fwd", st);
  return launched(tm.done(ft::launch_act(1, h, nullptr, n, out, st)));
}

ft_status fourtune_act_bwd(int act, const uint16_t* h, const uint16_t* g, int64_t n, uint16_t* out,
                           void* stream) {
  if (act != FT_ACT_GELU_TANH) return FT_EINVAL;
  if (!h || !g || !out) return FT_EINVAL;
  if (n < 0 || n * 2 > kMaxBytes) return FT_ESHAPE;
  if (!aligned16(h) || !aligned16(g) || !aligned16(out)) return FT_EALIGN;
  if (n == 0) return FT_OK;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Timed tm("act_bwd", st);
  return launched(tm.done(ft::launch_act(2, h, g, n, out, st)));
}

void fourtune_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tm.mu);
  g_tm.on = on != 0;
}

void fourtune_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_tm.mu);
  g_tm.drain();
  for (auto& v : g_tm.total_ms) v = 0.0;
  for (auto& c : g_tm.counts) c = 0;
}

int fourtune_timing_read(const char** names, double* total_ms, int64_t* counts, int max_entries) {
  std::lock_guard<std::mutex> lk(g_tm.mu);
  g_tm.drain();
  const int n = static_cast<int>(g_tm.names.size());
  for (int i = 0; i < n && i < max_entries; ++i) {
    if (names) names[i] = g_tm.names[i].c_str();
    if (total_ms) total_ms[i] = g_tm.total_ms[i];
    if (counts) counts[i] = g_tm.counts[i];
  }
  return n;
}

}  // extern "C"
