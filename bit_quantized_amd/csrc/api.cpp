// libfourtune C ABI (include/fourtune.h): argument checks, workspace layout
// and kernel dispatch.  Every check runs before the first launch, so a call
// that fails has enqueued nothing.
#include "../../include/fourtune.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
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

// 1 = current device is gfx950, 0 = not, 0 also before the first query
// (then the query runs; racing first calls both store the same answer).
// Cached per device.
std::atomic<int> g_arch_ok[64];

ft_status device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FT_EUNSUPPORTED;
  if (dev < 0 || dev >= 64) return FT_EUNSUPPORTED;
  int ok = g_arch_ok[dev].load(std::memory_order_acquire);
  if (ok == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FT_EUNSUPPORTED;
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(ok, std::memory_order_release);
  }
  return ok == 1 ? FT_OK : FT_EUNSUPPORTED;
}

ft_status launched(hipError_t e) { return e == hipSuccess ? FT_OK : FT_EDEVICE; }

// ---- optional per-kernel timing (benchmarks): hipEvents around each launch
// Kernel names are string literals (static storage), so the pointers handed
// out by fourtune_timing_read stay valid for the life of the process.
struct TimingState {
  std::mutex mu;
  std::atomic<bool> on{false};
  std::vector<hipEvent_t> pool;
  struct Pending { int slot; hipEvent_t a, b; };
  std::vector<Pending> pending;
  std::vector<const char*> names;
  std::vector<double> total_ms;
  std::vector<int64_t> counts;
  int slot(const char* n) {
    for (size_t i = 0; i < names.size(); ++i)
      if (std::strcmp(names[i], n) == 0) return static_cast<int>(i);
    names.push_back(n);
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
// Set by the entry point that allocates nothing while it runs: no timing
// events are created for its launches (creating one allocates).
thread_local bool t_no_timing = false;

// Brackets one launch with events when timing is on.
struct Timed {
  hipEvent_t a = nullptr, b = nullptr;
  int slot = -1;
  hipStream_t st;
  Timed(const char* name, hipStream_t s) : st(s) {
    if (t_no_timing || !g_tm.on.load(std::memory_order_relaxed)) return;
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

// The backward's dgrad computes the adapter gradients on the CUs its tiles
// leave free when at least this many are free.
constexpr int kSideMinFreeCUs = 16;

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
  if (L->w_block != FT_WBLOCK_TILE32 && L->w_block != FT_WBLOCK_ROW32 &&
      L->w_block != FT_WBLOCK_TILE32_T)
    return FT_EINVAL;
  // the method's tiles serve the dgrad as they are: no second weight
  if (L->w_block == FT_WBLOCK_TILE32 && L->wt_codes) return FT_EINVAL;
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
  size_t xq_codes, xq_scales, u_pad, v_pad, part, w16, x16, sk_part, total;
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
  // the GEMM's split sums when the output has few tiles (a few rows)
  o.sk_part = off; off += bf ? 0 : align_up(ft::gemm_split_bytes(L->M, L->K, L->N));
  o.total = off;
  return o;
}

// dB's partial sums come out of the backward quantize kernel (which reads
// dY anyway) for adapter ranks up to 32; above that the adapter-gradient
// kernel reads dY again.
bool db_fused_in_quant(const ft_linear* L) {
  return L->r_lora > 0 && ft::quant_down_db_chunks(L->M, L->N, L->r_stab + L->r_lora, L->r_lora) > 0;
}

struct BwdLayout {
  size_t gq_codes, gq_scales, P, p_pad, d_pad, part, dA_part, dB_part, w16, g16, sk_part, total;
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
  off += align_up(db_fused ? ft::quant_down_db_bytes(L->M, L->N, R, rl)
                           : (rl ? ft::lora_grad_part_bytes(L->M, L->N, rl) : 0));
  o.sk_part = off; off += bf ? 0 : align_up(ft::gemm_split_bytes(L->M, L->N, L->K));
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

// The second linear's input and down-projection partials that the first
// linear's GEMM of a fused MLP forward writes (fourtune_mlp_fwd).
struct MlpEpi {
  uint8_t* codes;
  uint8_t* scales;
  float* part;
  ft::RankRows pr;
  int R, nrg;
};

// The forward's kernels after the checks.  k1 = false: kernel 1's results
// (the quantized input and the padded rank operands) are already in place;
// epi: the GEMM also makes the next linear's input (MLP fusion).
ft_status fwd_run(const ft_linear* L, const uint16_t* X, uint16_t* Y, uint16_t* U_save,
                  uint8_t* xq_codes, uint8_t* xq_scales, uint8_t* ws, const FwdLayout& lay,
                  hipStream_t st, bool k1, const MlpEpi* epi) {
  const int R = L->r_stab + L->r_lora;
  const bool bf = a16(L);
  // A16: no codes; the quantize stores of kernel 1 are dropped
  uint8_t* qc = bf ? nullptr : xq_codes ? xq_codes : ws + lay.xq_codes;
  uint8_t* qs = bf ? nullptr : xq_scales ? xq_scales : ws + lay.xq_scales;
  uint16_t* u_pad = reinterpret_cast<uint16_t*>(ws + lay.u_pad);
  uint16_t* v_pad = reinterpret_cast<uint16_t*>(ws + lay.v_pad);
  hipError_t e = hipSuccess;
  // act_in: X is the pre-activation h; the layer's input is gelu(h)
  const int act = L->act_in == FT_ACT_GELU_TANH ? 1 : 0;
  if (!k1) {
    // (the second linear of a fused MLP: made by the first one's GEMM)
  } else if (R > 0) {
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
  if (!bf) {
    const ft::SplitPlan sp = ft::gemm_split_plan(L->M, L->K, L->N);
    g.splits = sp.splits; g.split_pairs = sp.pairs;
    g.part = reinterpret_cast<float*>(ws + lay.sk_part);
  }
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
  if (epi) {
    g.e_codes = epi->codes; g.e_scales = epi->scales; g.e_part = epi->part;
    g.e_pr = epi->pr; g.e_R = epi->R; g.e_nrg = epi->nrg;
  }
  Timed tm(epi ? "fwd_gemm_mlp" : "fwd_gemm", st);
  return launched(tm.done(ft::launch_gemm(g, st)));
}

// Hooks of the MLP block's fused backward (fourtune_mlp_bwd).
// On the second linear: epi and h: its dgrad's epilogue writes dY1 (to dX)
// and makes the first linear's quantized dY1 and P1 partial sums.
// On the first linear: k1_done: those are in place; dB is formed from
// db_big = dY1 by the adapter-gradient kernel, its partials in db_part.
struct BwdHook {
  const MlpEpi* epi;
  const uint16_t* h;
  bool k1_done;
  const uint16_t* db_big;
  float* db_part;
};

// The backward's kernels after the checks.
ft_status bwd_run(const ft_linear* L, const uint16_t* dY, const uint16_t* X,
                  const uint16_t* U_save, const uint16_t* H, uint16_t* dX, void* dA, void* dB,
                  ft_dtype grad_dtype, uint16_t* P_save, uint8_t* gq_codes, uint8_t* gq_scales,
                  uint8_t* ws, const BwdLayout& lay, hipStream_t st, const BwdHook* hook) {
  const int R = L->r_stab + L->r_lora;
  const int rl = L->r_lora;
  const bool bf = g16(L);
  // G16: no codes; the quantize stores of kernel 1 are dropped
  uint8_t* qc = bf ? nullptr : gq_codes ? gq_codes : ws + lay.gq_codes;
  uint8_t* qs = bf ? nullptr : gq_scales ? gq_scales : ws + lay.gq_scales;
  uint16_t* P = P_save ? P_save : reinterpret_cast<uint16_t*>(ws + lay.P);
  uint16_t* p_pad = reinterpret_cast<uint16_t*>(ws + lay.p_pad);
  uint16_t* d_pad = reinterpret_cast<uint16_t*>(ws + lay.d_pad);
  hipError_t e = hipSuccess;
  // the first linear of a fused MLP backward: kernel 1's results come from
  // the second linear's dgrad and the partial sums' kernel, and dB is
  // formed by the adapter-gradient kernel from dY1
  const bool k1 = !(hook && hook->k1_done);
  const bool db_fused = k1 && db_fused_in_quant(L);
  ft::DbFuse db{U_save, R, L->r_stab, rl, reinterpret_cast<float*>(ws + lay.dB_part)};
  // act_out: dY is the gradient of gelu(Y) and H the saved Y; the incoming
  // gradient of this layer is dY * gelu'(H)
  const int act = L->act_out == FT_ACT_GELU_TANH ? 2 : 0;
  const uint16_t* h2 = act ? H : nullptr;
  if (!k1) {
    // (made by the second linear's dgrad epilogue and the partial sums' kernel)
  } else if (R > 0) {
    Timed tm("bwd_quant_down", st);
    // the pipelined dgrad on the forward's tiles (N % 128 == 0, 4-bit)
    // reads [L1 | A] as nibble planes through its transposing b read
    // (not when the dgrad splits its reduction: the split sums' kernel
    // reads the plain [K, ranks] copy)
    const bool planes = L->w_block == FT_WBLOCK_TILE32 && !bf && (L->N % 128) == 0 &&
                        ft::gemm_split_plan(L->M, L->N, L->K).splits <= 1;
    e = tm.done(ft::launch_quant_down(dY, h2, act, L->M, L->N, L->N, qc, qs, rows_V(L), P, p_pad,
                                      rows_Dt(L), dX ? L->K : 0, d_pad,
                                      reinterpret_cast<float*>(ws + lay.part),
                                      db_fused ? &db : nullptr, st, planes));
  } else if (!bf) {
    Timed tm("bwd_quant_down", st);
    e = tm.done(ft::launch_quant_row32(dY, h2, act, L->M, L->N, L->N, qc, qs, st));
  }
  if (e != hipSuccess) return FT_EDEVICE;
  // the adapter gradients: dA = P[:, r_s:]^T X and dB = U[:, r_s:]^T dY
  ft::LoraGradArgs la{}, lb{};
  if (rl > 0) {
    const int f32 = grad_dtype == FT_F32 ? 1 : 0;
    la.M = L->M; la.I = L->K; la.big = X; la.small = P; la.ld_small = R; la.r0 = L->r_stab; la.rl = rl;
    la.big2 = nullptr; la.act = L->act_in == FT_ACT_GELU_TANH ? 1 : 0;
    la.out = dA; la.out_f32 = f32;
    la.part = reinterpret_cast<float*>(ws + lay.dA_part);
    lb = la;
    lb.I = L->N; lb.big = dY; lb.small = U_save;
    lb.big2 = L->act_out == FT_ACT_GELU_TANH ? H : nullptr;
    lb.act = L->act_out == FT_ACT_GELU_TANH ? 2 : 0;
    lb.out = dB;
    lb.part = reinterpret_cast<float*>(ws + lay.dB_part);
    if (!k1) {
      // dY1 = dY * gelu'(H) is already formed
      lb.big = hook->db_big; lb.big2 = nullptr; lb.act = 0;
      lb.part = hook->db_part;
    }
    lb.nchunk = db_fused ? ft::quant_down_db_chunks(L->M, L->N, R, rl) : 0;
  }
  // the adapter gradients made by the dgrad's launch on the CUs its tiles
  // leave free
  bool da_side = false;
  if (dX) {
    ft::GemmArgs g{};
    g.M = L->M; g.RED = L->N; g.NOUT = L->K;
    g.a_codes = qc; g.a_scales = qs;
    if (L->w_block == FT_WBLOCK_TILE32) {
      // the forward's tiles [N, K/2], read transposed (section 3.2)
      g.b_codes = L->w_codes; g.b_scales = L->w_scales;
      g.b_transposed = 1;
    } else {
      g.b_codes = L->wt_codes; g.b_scales = L->wt_scales;
      g.b_row_scales = L->w_block == FT_WBLOCK_ROW32;
    }
    g.lm = p_pad; g.lo = d_pad; g.nlr = ft::rank_pad(R) / 32; g.out = dX;
    if (!bf) {
      const ft::SplitPlan sp = ft::gemm_split_plan(L->M, L->N, L->K);
      g.splits = sp.splits; g.split_pairs = sp.pairs;
      g.part = reinterpret_cast<float*>(ws + lay.sk_part);
    }
    if (bf) {
      uint16_t* w16 = reinterpret_cast<uint16_t*>(ws + lay.w16);
      {
        Timed tm("bwd_dequant_w", st);
        const hipError_t de =
            L->w_block == FT_WBLOCK_TILE32
                ? ft::launch_dequant_tile32_t(L->w_codes, L->w_scales, L->N, L->K, w16, st)
                : ft::launch_dequant_tile32(L->wt_codes, L->wt_scales, L->K, L->N, w16, st);
        if (tm.done(de) != hipSuccess) return FT_EDEVICE;
      }
      g.b_transposed = 0;
      const uint16_t* g16p = dY;
      if (act) {
        uint16_t* ga = reinterpret_cast<uint16_t*>(ws + lay.g16);
        Timed tm("bwd_act", st);
        if (tm.done(ft::launch_act(2, H, dY, L->M * L->N, ga, st)) != hipSuccess) return FT_EDEVICE;
        g16p = ga;
      }
      g.a16 = g16p; g.b16 = w16;
    }
    if (hook && hook->epi) {
      // the second linear of a fused MLP backward: dX here is dY1
      const MlpEpi* ep = hook->epi;
      g.e_codes = ep->codes; g.e_scales = ep->scales; g.e_part = ep->part;
      g.e_pr = ep->pr; g.e_R = ep->R; g.e_nrg = ep->nrg; g.e_h = hook->h;
    }
    // the transposed-weight dgrad whose tiles leave CUs free computes the
    // adapter gradients there (dB's partials made by the quantizer, ranks
    // in one pass, X without an activation): its launch gets one workgroup
    // more per CU that is free from the start (fewer tiles than CUs) or
    // that finishes a round early (a partial last round: the extra
    // workgroups are dispatched as those CUs free up), when the side
    // work's estimate (about 2.5 us per 512-token chunk of a 64-column
    // block of dA on one CU) stays within 0.8 of the time those CUs are
    // free (about 1 us per 128-deep step of a tile).  The adapter-gradient
    // launch then does not run.
    if (rl > 0 && rl <= 64 && db_fused && la.act == 0 && g.b_transposed && !bf &&
        !(hook && hook->epi) && (L->N & 127) == 0) {
      const int64_t cus = ft::cu_count();
      const int64_t wgs = ft::gemm_workgroups(g);
      const int64_t tiles = ((L->M + 255) / 256) * ((L->K + 255) / 256);
      const int64_t units = tiles * std::max(g.splits, 1);
      const int64_t steps = g.splits > 1 ? 2 * g.split_pairs
                                         : (L->N / 128 + (L->N / 128) % 2) + ft::rank_pad(R) / 32;
      int64_t side = 0, free_rounds = 0;
      if (wgs > 0 && wgs + kSideMinFreeCUs <= cus) {
        side = cus - wgs;                                  // free from the start
        free_rounds = (units + wgs - 1) / wgs;
      } else if (wgs == cus && units % cus != 0 && cus - units % cus >= kSideMinFreeCUs) {
        side = cus - units % cus;                          // free for the last round
        free_rounds = 1;
      }
      if (side > 0) {
        const double side_us = 2.5 * ((ft::lora_col_blocks(L->K) + side - 1) / side) * ft::lora_chunks(L->M);
        if (side_us <= 0.8 * static_cast<double>(free_rounds * steps)) {
          g.lora_a = la;
          g.lora_b = lb;
          g.gemm_wgs = static_cast<uint32_t>(wgs);
          g.side_wgs = static_cast<uint32_t>(side);
          da_side = true;
        }
      }
    }
    Timed tm(hook && hook->epi ? "bwd_gemm_dgrad_mlp" : "bwd_gemm_dgrad", st);
    if (tm.done(ft::launch_gemm(g, st)) != hipSuccess) return FT_EDEVICE;
  }
  if (rl > 0 && !da_side) {
    Timed tm("bwd_lora_grads", st);
    if (tm.done(ft::launch_lora_grads(la, lb, db_fused, st)) != hipSuccess) return FT_EDEVICE;
  }
  return FT_OK;
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
  if (ld_in < 0 || ld_in > kMaxDim) return FT_ESHAPE;
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
  if (L->w_block != FT_WBLOCK_TILE32 && L->w_block != FT_WBLOCK_ROW32 &&
      L->w_block != FT_WBLOCK_TILE32_T)
    return 0;
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
  return fwd_run(L, X, Y, U_save, xq_codes, xq_scales, static_cast<uint8_t*>(workspace), lay,
                 static_cast<hipStream_t>(stream), true, nullptr);
}

size_t fourtune_mlp_workspace_bytes(const ft_linear* fc1, const ft_linear* fc2) {
  const size_t a = fourtune_workspace_bytes(fc1, 0), b = fourtune_workspace_bytes(fc2, 0);
  return a && b ? a + b : 0;
}

ft_status fourtune_mlp_fwd(const ft_linear* fc1, const ft_linear* fc2, const uint16_t* X,
                           uint16_t* H, uint16_t* Y, uint16_t* U1_save, uint16_t* U2_save,
                           uint8_t* aq_codes, uint8_t* aq_scales, void* workspace,
                           size_t ws_bytes, void* stream) {
  if (ft_status s = check_linear(fc1); s != FT_OK) return s;
  if (ft_status s = check_linear(fc2); s != FT_OK) return s;
  if (fc2->M != fc1->M || fc2->K != fc1->N) return FT_ESHAPE;
  if (fc2->act_in != FT_ACT_GELU_TANH) return FT_EINVAL;
  const int R1 = fc1->r_stab + fc1->r_lora, R2 = fc2->r_stab + fc2->r_lora;
  if (!X || !H || !Y) return FT_EINVAL;
  if ((R1 > 0 && !U1_save) || (R2 > 0 && !U2_save)) return FT_EINVAL;
  if ((aq_codes == nullptr) != (aq_scales == nullptr)) return FT_EINVAL;
  if (a16(fc2) && aq_codes) return FT_EINVAL;
  const void* ptrs[] = {X, H, Y, U1_save, U2_save, aq_codes, aq_scales, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const FwdLayout l1 = fwd_layout(fc1), l2 = fwd_layout(fc2);
  if (ws_bytes < l1.total + l2.total) return FT_EWORKSPACE;
  if (!workspace) return FT_EINVAL;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws1 = static_cast<uint8_t*>(workspace);
  uint8_t* ws2 = ws1 + l1.total;
  const int64_t M = fc1->M, N1 = fc1->N;
  // the down-projection partials per 256-column split of h, 32-bit offsets
  const int64_t nsplit = (N1 + 255) / 256;
  const int nrg = ft::rank_reduce_nrg(R2);
  const bool fused = !a16(fc1) && !a16(fc2) && fc1->w_block != FT_WBLOCK_ROW32 &&
                     ft::gemm_mlp_ok(M, fc1->K, N1, R2) &&
                     nsplit * ((M + 63) / 64) * 4 * nrg * 1024 <= kMaxBytes;
  if (!fused) {
    if (ft_status s = fwd_run(fc1, X, H, U1_save, nullptr, nullptr, ws1, l1, st, true, nullptr);
        s != FT_OK)
      return s;
    return fwd_run(fc2, H, Y, U2_save, aq_codes, aq_scales, ws2, l2, st, true, nullptr);
  }
  uint8_t* qc2 = aq_codes ? aq_codes : ws2 + l2.xq_codes;
  uint8_t* qs2 = aq_scales ? aq_scales : ws2 + l2.xq_scales;
  float* part2 = reinterpret_cast<float*>(ws2 + l2.part);
  const MlpEpi epi{qc2, qs2, part2, rows_Dt(fc2), R2, nrg};
  if (ft_status s = fwd_run(fc1, X, H, U1_save, nullptr, nullptr, ws1, l1, st, true, &epi); s != FT_OK)
    return s;
  if (R2 > 0) {
    Timed tm("fwd_rank_reduce", st);
    if (tm.done(ft::launch_rank_reduce(part2, M, static_cast<int>(nsplit), R2, U2_save,
                                       reinterpret_cast<uint16_t*>(ws2 + l2.u_pad), rows_V(fc2),
                                       fc2->N, reinterpret_cast<uint16_t*>(ws2 + l2.v_pad), st)) !=
        hipSuccess)
      return FT_EDEVICE;
  }
  return fwd_run(fc2, H, Y, U2_save, qc2, qs2, ws2, l2, st, false, nullptr);
}

size_t fourtune_mlp_bwd_workspace_bytes(const ft_linear* fc1, const ft_linear* fc2) {
  const size_t a = fourtune_workspace_bytes(fc1, 1), b = fourtune_workspace_bytes(fc2, 1);
  if (!a || !b) return 0;
  // dY1 (or, unfused, dX2) [M, N1] bf16 and the first linear's dB partials
  // when the adapter-gradient kernel forms dB
  const size_t dy = align_up(static_cast<size_t>(fc1->M) * fc1->N * 2);
  const size_t dbp = fc1->r_lora ? align_up(ft::lora_grad_part_bytes(fc1->M, fc1->N, fc1->r_lora)) : 0;
  return a + b + dy + dbp;
}

ft_status fourtune_mlp_bwd(const ft_linear* fc1, const ft_linear* fc2, const uint16_t* dY,
                           const uint16_t* X, const uint16_t* H, const uint16_t* U1_save,
                           const uint16_t* U2_save, uint16_t* dX, void* dA1, void* dB1, void* dA2,
                           void* dB2, ft_dtype grad_dtype, void* workspace, size_t ws_bytes,
                           void* stream) {
  if (ft_status s = check_linear(fc1); s != FT_OK) return s;
  if (ft_status s = check_linear(fc2); s != FT_OK) return s;
  if (fc2->M != fc1->M || fc2->K != fc1->N) return FT_ESHAPE;
  if (fc2->act_in != FT_ACT_GELU_TANH || fc1->act_out != FT_ACT_GELU_TANH) return FT_EINVAL;
  if (grad_dtype != FT_BF16 && grad_dtype != FT_F32) return FT_EINVAL;
  if (!dY || !X || !H || !dX) return FT_EINVAL;
  if (fc1->w_block != FT_WBLOCK_TILE32 && !fc1->wt_codes) return FT_EINVAL;
  if (fc2->w_block != FT_WBLOCK_TILE32 && !fc2->wt_codes) return FT_EINVAL;
  const int R1 = fc1->r_stab + fc1->r_lora, R2 = fc2->r_stab + fc2->r_lora;
  if ((R1 > 0 && !U1_save) || (R2 > 0 && !U2_save)) return FT_EINVAL;
  if ((fc1->r_lora > 0 && (!dA1 || !dB1)) || (fc2->r_lora > 0 && (!dA2 || !dB2))) return FT_EINVAL;
  const void* ptrs[] = {dY, X, H, U1_save, U2_save, dX, dA1, dB1, dA2, dB2, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return FT_EALIGN;
  const BwdLayout l1 = bwd_layout(fc1), l2 = bwd_layout(fc2);
  const int64_t M = fc1->M, F = fc1->N;
  const size_t dy_bytes = align_up(static_cast<size_t>(M) * F * 2);
  const size_t dbp_bytes = fc1->r_lora ? align_up(ft::lora_grad_part_bytes(M, F, fc1->r_lora)) : 0;
  if (ws_bytes < l1.total + l2.total + dy_bytes + dbp_bytes) return FT_EWORKSPACE;
  if (!workspace) return FT_EINVAL;
  if (ft_status s = device_check(); s != FT_OK) return s;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws1 = static_cast<uint8_t*>(workspace);
  uint8_t* ws2 = ws1 + l1.total;
  uint16_t* dy1 = reinterpret_cast<uint16_t*>(ws2 + l2.total);
  float* dbp = reinterpret_cast<float*>(ws2 + l2.total + dy_bytes);
  // the first linear's P1 partial sums per 256-column split of dY1
  const int64_t nsplit = (F + 255) / 256;
  const int nrg = ft::rank_reduce_nrg(R1);
  const bool fused = !a16(fc1) && !g16(fc1) && !a16(fc2) && !g16(fc2) &&
                     fc2->w_block == FT_WBLOCK_TILE32 && (fc2->N % 128) == 0 && M > 16 && R1 <= 64 &&
                     ft::gemm_split_plan(M, fc2->N, F).splits <= 1 &&
                     nsplit * ((M + 63) / 64) * 4 * nrg * 1024 <= kMaxBytes;
  if (!fused) {
    // the two backwards one after the other, through dX2 [M, N1]
    if (ft_status s = bwd_run(fc2, dY, H, U2_save, nullptr, dy1, dA2, dB2, grad_dtype, nullptr,
                              nullptr, nullptr, ws2, l2, st, nullptr);
        s != FT_OK)
      return s;
    return bwd_run(fc1, dy1, X, U1_save, H, dX, dA1, dB1, grad_dtype, nullptr, nullptr, nullptr,
                   ws1, l1, st, nullptr);
  }
  // the second linear, its dgrad making dY1, Qrow(dY1) and the P1 partials
  const MlpEpi epi{ws1 + l1.gq_codes, ws1 + l1.gq_scales, reinterpret_cast<float*>(ws1 + l1.part),
                   rows_V(fc1), R1, nrg};
  const BwdHook h2{&epi, H, false, nullptr, nullptr};
  if (ft_status s = bwd_run(fc2, dY, H, U2_save, nullptr, dy1, dA2, dB2, grad_dtype, nullptr,
                            nullptr, nullptr, ws2, l2, st, &h2);
      s != FT_OK)
    return s;
  if (R1 > 0) {
    // P1 and its padded copy, and the first linear's [L1 | A] for its dgrad
    // (as nibble planes where that dgrad reads its b transposed in one pass)
    const bool planes = fc1->w_block == FT_WBLOCK_TILE32 && (F % 128) == 0 &&
                        ft::gemm_split_plan(M, F, fc1->K).splits <= 1;
    Timed tm("bwd_rank_reduce", st);
    if (tm.done(ft::launch_rank_reduce(reinterpret_cast<float*>(ws1 + l1.part), M,
                                       static_cast<int>(nsplit), R1,
                                       reinterpret_cast<uint16_t*>(ws1 + l1.P),
                                       reinterpret_cast<uint16_t*>(ws1 + l1.p_pad), rows_Dt(fc1),
                                       fc1->K, reinterpret_cast<uint16_t*>(ws1 + l1.d_pad), st,
                                       planes)) != hipSuccess)
      return FT_EDEVICE;
  }
  const BwdHook h1{nullptr, nullptr, true, dy1, dbp};
  return bwd_run(fc1, dy1, X, U1_save, H, dX, dA1, dB1, grad_dtype, nullptr, nullptr, nullptr, ws1,
                 l1, st, &h1);
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
  // a separately stored dgrad weight (group-wise blocks, or the tiles'
  // transposed layout copy) is needed only for dX
  if (dX && L->w_block != FT_WBLOCK_TILE32 && !L->wt_codes) return FT_EINVAL;
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

  return bwd_run(L, dY, X, U_save, H, dX, dA, dB, grad_dtype, P_save, gq_codes, gq_scales,
                 static_cast<uint8_t*>(workspace), lay, static_cast<hipStream_t>(stream), nullptr);
}

ft_status fourtune_linear_fwd_noalloc(const ft_linear* L, const uint16_t* X, uint16_t* Y,
                                      uint16_t* U_save, uint8_t* xq_codes, uint8_t* xq_scales,
                                      void* stream) {
  if (ft_status s = check_linear(L); s != FT_OK) return s;
  if (fwd_layout(L).total > ft::kNoAllocScratchBytes) return FT_EWORKSPACE;
  if (ft_status s = device_check(); s != FT_OK) return s;
  void* ws = ft::noalloc_scratch();
  if (!ws) return FT_EDEVICE;
  struct Quiet {
    Quiet() { t_no_timing = true; }
    ~Quiet() { t_no_timing = false; }
  } quiet;
  return fourtune_linear_fwd(L, X, Y, U_save, xq_codes, xq_scales, ws, ft::kNoAllocScratchBytes,
                             stream);
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
  g_tm.on.store(on != 0, std::memory_order_relaxed);
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
    if (names) names[i] = g_tm.names[i];
    if (total_ms) total_ms[i] = g_tm.total_ms[i];
    if (counts) counts[i] = g_tm.counts[i];
  }
  return n;
}

}  // extern "C"
