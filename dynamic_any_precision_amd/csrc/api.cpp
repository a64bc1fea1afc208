// C ABI of libmoe_anyprec: argument validation, workspace plans and launches.
// Validation runs on the host before any HIP call, so it works without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "moe_anyprec.h"
#include "kernels.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int num_cu_cached() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cache[dev] = v;
  }
  return cache[dev];
}

moe_status check_bank(const moe_expert_bank* b, bool need_ptrs) {
  if (!b) return MOE_ERR_NULL;
  if (need_ptrs && (!b->w13_planes || !b->w13_sz || !b->w2_planes || !b->w2_sz)) return MOE_ERR_NULL;
  if (b->n_experts < 1 || b->b_max < 1 || b->b_max > 4) return MOE_ERR_RANGE;
  if (b->group != 64 && b->group != 128) return MOE_ERR_UNSUPPORTED;
  if (b->d_model < 128 || b->d_ff < 128 || b->d_model % 128 || b->d_ff % 128) return MOE_ERR_SHAPE;
  if (need_ptrs && (!aligned(b->w13_planes, 16) || !aligned(b->w2_planes, 16) || !aligned(b->w13_sz, 16) ||
                    !aligned(b->w2_sz, 16)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

// floor(P * (target - b_lo) / (b_max - b_lo)) with exact arithmetic on the
// float value of target (a dyadic rational), clamped to [0, P].
int32_t exact_budget(int32_t P, int32_t b_lo, int32_t b_max, float target) {
  if (P <= 0 || b_max <= b_lo) return 0;
  int e = 0;
  const double fr = std::frexp((double)target, &e);
  const int64_t m = (int64_t)std::ldexp(fr, 24);
  const int ex = e - 24;
  __int128 num, den;
  if (ex >= 0) {
    num = (__int128)P * (((__int128)m << ex) - b_lo);
    den = (__int128)(b_max - b_lo);
  } else {
    num = (__int128)P * ((__int128)m - ((__int128)b_lo << (-ex)));
    den = (__int128)(b_max - b_lo) << (-ex);
  }
  __int128 q = num / den;
  if ((num % den != 0) && ((num < 0) != (den < 0))) q -= 1;
  if (q < 0) q = 0;
  if (q > P) q = P;
  return (int32_t)q;
}

moe::MatrixDev w13_of(const moe_expert_bank* b) {
  moe::MatrixDev m;
  m.planes = b->w13_planes;
  m.sz = b->w13_sz;
  m.N = 2 * b->d_ff;
  m.K = b->d_model;
  return m;
}

moe::MatrixDev w2_of(const moe_expert_bank* b) {
  moe::MatrixDev m;
  m.planes = b->w2_planes;
  m.sz = b->w2_sz;
  m.N = b->d_model;
  m.K = b->d_ff;
  return m;
}

moe_status ffn_shape(const moe_expert_bank* routed, const moe_expert_bank* shared, int32_t T, int32_t top_k,
                     bool need_ptrs, moe::FfnShape* out) {
  moe_status st = check_bank(routed, need_ptrs);
  if (st != MOE_OK) return st;
  if (shared) {
    st = check_bank(shared, need_ptrs);
    if (st != MOE_OK) return st;
    if (shared->d_model != routed->d_model || shared->group != routed->group || shared->b_max != routed->b_max)
      return MOE_ERR_SHAPE;
    if (shared->n_experts > 16) return MOE_ERR_RANGE;
  }
  if (T < 0 || top_k < 1 || top_k > 8 || top_k > routed->n_experts || routed->n_experts > 256) return MOE_ERR_RANGE;
  if ((int64_t)T * top_k + (shared ? (int64_t)shared->n_experts * T : 0) >= (1 << 24)) return MOE_ERR_RANGE;
  if (shared && shared->plane_prefix) return MOE_ERR_UNSUPPORTED;  // shared banks are uniform
  *out = moe::make_shape(T, top_k, routed->n_experts, routed->b_max, routed->group, routed->d_model, routed->d_ff,
                         shared ? shared->n_experts : 0, shared ? shared->d_ff : 0);
  out->bprefix = routed->plane_prefix;
  return MOE_OK;
}

// Measurement hook: events recorded around the gate/up and down kernels.
thread_local hipEvent_t g_kernel_events[4] = {nullptr, nullptr, nullptr, nullptr};

hipError_t mark(int i, hipStream_t strm) {
  return g_kernel_events[i] ? hipEventRecord(g_kernel_events[i], strm) : hipSuccess;
}

// The FFN after the plan: activation gather, gate/up + SwiGLU, down, combine.
hipError_t ffn_after_plan(const moe::FfnShape& s, const moe::FfnLayout& L, char* ws, const moe_expert_bank* routed,
                          const moe_expert_bank* shared, const uint16_t* x, const float* topk_gate, float* y,
                          int32_t accumulate, hipStream_t strm) {
  const int ncu = num_cu_cached();
  moe::MatrixDev none;
  std::memset(&none, 0, sizeof(none));
  none.N = 16;
  none.K = 128;
  // one token: the plan kernel wrote the token's fragment, which every chunk reads
  hipError_t e = s.act_shared ? hipSuccess : moe::launch_gather(s, L, ws, x, strm);
  if (e == hipSuccess) e = mark(0, strm);
  if (e == hipSuccess)
    e = moe::launch_ffn_w13(s, L, ws, w13_of(routed), shared ? w13_of(shared) : none, ncu, strm);
  if (e == hipSuccess) e = mark(1, strm);
  if (e == hipSuccess) e = mark(2, strm);
  if (e == hipSuccess) e = moe::launch_ffn_w2(s, L, ws, w2_of(routed), shared ? w2_of(shared) : none, ncu, strm);
  if (e == hipSuccess) e = mark(3, strm);
  if (e == hipSuccess) e = moe::launch_combine(s, L, ws, topk_gate, y, accumulate, strm);
  return e;
}

size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

namespace moe {
int record_hip_error(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return MOE_ERR_HIP;
}
}  // namespace moe

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "required pointer is NULL";
    case MOE_ERR_SHAPE: return "inconsistent or unsupported shape";
    case MOE_ERR_ALIGN: return "buffer not aligned";
    case MOE_ERR_RANGE: return "argument out of range";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

void moe_set_kernel_events(void* w13_begin, void* w13_end, void* w2_begin, void* w2_end) {
  g_kernel_events[0] = static_cast<hipEvent_t>(w13_begin);
  g_kernel_events[1] = static_cast<hipEvent_t>(w13_end);
  g_kernel_events[2] = static_cast<hipEvent_t>(w2_begin);
  g_kernel_events[3] = static_cast<hipEvent_t>(w2_end);
}

size_t moe_route_workspace_bytes(int32_t T, int32_t E) {
  if (T < 0 || E < 1) return 0;
  return moe::route_workspace_bytes(T, E);
}

moe_status moe_route(const uint16_t* x, int32_t T, int32_t d, const float* w_router, int32_t E,
                     const float* logit_bias, int32_t top_k, int32_t renorm_topk, int32_t* topk_idx,
                     float* topk_gate, void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > 256 || top_k < 1 || top_k > 8 || top_k > E) return MOE_ERR_RANGE;
  if (d < 128 || d % 128) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(workspace, 16)) return MOE_ERR_ALIGN;
  if (ws_bytes < moe::route_workspace_bytes(T, E)) return MOE_ERR_WORKSPACE;
  return hip_status(moe::launch_route(x, T, d, w_router, E, logit_bias, top_k, renorm_topk, topk_idx, topk_gate,
                                      workspace, static_cast<hipStream_t>(stream)));
}

int32_t moe_budget_pairs(int32_t P, int32_t b_lo, int32_t b_max, float target_avg_bits) {
  return exact_budget(P, b_lo, b_max, target_avg_bits);
}

moe_status moe_alloc_bits(const float* gate, int32_t P, int32_t b_lo, int32_t b_max, float target_avg_bits,
                          uint8_t* bits, float* tau_out, int32_t* n_hi_out, void* stream) {
  if (P < 0 || b_lo < 1 || b_max > 4 || b_lo > b_max) return MOE_ERR_RANGE;
  if (!(target_avg_bits >= (float)b_lo && target_avg_bits <= (float)b_max)) return MOE_ERR_RANGE;
  if (P == 0) return MOE_OK;
  if (!gate || !bits) return MOE_ERR_NULL;
  const int32_t ns = exact_budget(P, b_lo, b_max, target_avg_bits);
  return hip_status(moe::launch_alloc(gate, P, ns, b_lo, b_max, bits, tau_out, n_hi_out,
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_bits_from_threshold(const float* gate, int32_t P, float tau, int32_t b_lo, int32_t b_max,
                                   uint8_t* bits, void* stream) {
  if (P < 0 || b_lo < 1 || b_max > 4 || b_lo > b_max || tau != tau) return MOE_ERR_RANGE;
  if (P == 0) return MOE_OK;
  if (!gate || !bits) return MOE_ERR_NULL;
  return hip_status(moe::launch_bits_threshold(gate, P, tau, b_lo, b_max, bits, static_cast<hipStream_t>(stream)));
}

moe_status moe_bits_from_threshold_device(const float* gate, int32_t P, const float* tau, int32_t b_lo,
                                          int32_t b_max, uint8_t* bits, void* stream) {
  if (P < 0 || b_lo < 1 || b_max > 4 || b_lo > b_max) return MOE_ERR_RANGE;
  if (P == 0) return MOE_OK;
  if (!gate || !tau || !bits) return MOE_ERR_NULL;
  return hip_status(moe::launch_bits_threshold_dev(gate, P, tau, b_lo, b_max, bits, static_cast<hipStream_t>(stream)));
}

size_t moe_ffn_workspace_bytes(const moe_expert_bank* routed, const moe_expert_bank* shared, int32_t T,
                               int32_t top_k) {
  moe::FfnShape s;
  if (ffn_shape(routed, shared, T, top_k, false, &s) != MOE_OK) return 0;
  return moe::make_layout(s).total;
}

moe_status moe_anyprec_ffn(const moe_expert_bank* routed, const moe_expert_bank* shared, const uint16_t* x,
                           int32_t T, int32_t top_k, const int32_t* topk_idx, const float* topk_gate,
                           const uint8_t* bits, float* y, int32_t accumulate, void* workspace, size_t ws_bytes,
                           void* stream) {
  moe::FfnShape s;
  moe_status st = ffn_shape(routed, shared, T, top_k, true, &s);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !topk_idx || !topk_gate || !bits || !y || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  const moe::FfnLayout L = moe::make_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (moe::one_token_fits(s)) {
    s.act_shared = 1;
    e = moe::launch_one(s, L, ws, x, nullptr, 0, 0, 0, 0, const_cast<int32_t*>(topk_idx), nullptr,
                        const_cast<uint8_t*>(bits), strm);
  } else {
    e = moe::launch_plan(s, L, ws, topk_idx, bits, strm);
  }
  if (e == hipSuccess) e = ffn_after_plan(s, L, ws, routed, shared, x, topk_gate, y, accumulate, strm);
  return hip_status(e);
}

size_t moe_layer_workspace_bytes(const moe_expert_bank* routed, const moe_expert_bank* shared, int32_t T,
                                 int32_t top_k) {
  moe::FfnShape s;
  if (ffn_shape(routed, shared, T, top_k, false, &s) != MOE_OK) return 0;
  return al256(moe::make_layout(s).total) + moe::route_workspace_bytes(T, routed->n_experts);
}

moe_status moe_layer(const moe_expert_bank* routed, const moe_expert_bank* shared, const uint16_t* x, int32_t T,
                     int32_t top_k, const float* w_router, const float* logit_bias, int32_t renorm_topk,
                     int32_t b_lo, float target_avg_bits, int32_t* topk_idx, float* topk_gate, uint8_t* bits,
                     float* y, int32_t accumulate, void* workspace, size_t ws_bytes, void* stream) {
  moe::FfnShape s;
  moe_status st = ffn_shape(routed, shared, T, top_k, true, &s);
  if (st != MOE_OK) return st;
  const int32_t b_max = routed->b_max;
  if (b_lo < 1 || b_lo > b_max) return MOE_ERR_RANGE;
  if (!(target_avg_bits >= (float)b_lo && target_avg_bits <= (float)b_max)) return MOE_ERR_RANGE;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !topk_idx || !topk_gate || !bits || !y || !workspace) return MOE_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_router, 16) || !aligned(y, 16) || !aligned(workspace, 256))
    return MOE_ERR_ALIGN;
  const moe::FfnLayout L = moe::make_layout(s);
  const size_t route_off = al256(L.total);
  if (ws_bytes < route_off + moe::route_workspace_bytes(T, s.E)) return MOE_ERR_WORKSPACE;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  double* logits = reinterpret_cast<double*>(ws + route_off);
  const int32_t n_star = exact_budget(s.P, b_lo, b_max, target_avg_bits);
  hipError_t e = moe::launch_route_logits(x, T, s.d, w_router, s.E, logit_bias, logits, strm);
  if (e == hipSuccess) {
    if (moe::one_token_fits(s)) {
      s.act_shared = 1;
      e = moe::launch_one(s, L, ws, x, logits, renorm_topk, n_star, b_lo, b_max, topk_idx, topk_gate, bits, strm);
    } else if (moe::control_fits(s)) {
      if (!moe::control_does_topk(s))
        e = moe::launch_route_topk(logits, T, s.E, top_k, renorm_topk, topk_idx, topk_gate, strm);
      if (e == hipSuccess)
        e = moe::launch_control(s, L, ws, logits, renorm_topk, n_star, b_lo, b_max, topk_idx, topk_gate, bits,
                                strm);
    } else {
      e = moe::launch_route_topk(logits, T, s.E, top_k, renorm_topk, topk_idx, topk_gate, strm);
      if (e == hipSuccess) e = moe::launch_alloc(topk_gate, s.P, n_star, b_lo, b_max, bits, nullptr, nullptr, strm);
      if (e == hipSuccess) e = moe::launch_plan(s, L, ws, topk_idx, bits, strm);
    }
  }
  if (e == hipSuccess) e = ffn_after_plan(s, L, ws, routed, shared, x, topk_gate, y, accumulate, strm);
  return hip_status(e);
}

moe_status moe_permute(const int32_t* topk_idx, const uint8_t* bits, int32_t T, int32_t top_k, int32_t E,
                       int32_t b_max, int32_t* slot_pair, int32_t* expert_offsets, int32_t* expert_maxbits,
                       void* workspace, size_t ws_bytes, void* stream) {
  if (T < 0 || E < 1 || E > 256 || top_k < 1 || top_k > 8 || top_k > E || b_max < 1 || b_max > 4)
    return MOE_ERR_RANGE;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !bits || !slot_pair || !expert_offsets || !expert_maxbits || !workspace) return MOE_ERR_NULL;
  if (!aligned(workspace, 256)) return MOE_ERR_ALIGN;
  const moe::FfnShape s = moe::make_shape(T, top_k, E, b_max, 128, 128, 128, 0, 0);
  const moe::FfnLayout L = moe::make_layout(s);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  hipError_t e = moe::launch_plan(s, L, ws, topk_idx, bits, strm);
  if (e == hipSuccess)
    e = hipMemcpyAsync(slot_pair, ws + L.slot_pair, (size_t)s.P * 4, hipMemcpyDeviceToDevice, strm);
  if (e == hipSuccess)
    e = hipMemcpyAsync(expert_offsets, ws + L.expert_off, (size_t)(E + 1) * 4, hipMemcpyDeviceToDevice, strm);
  if (e == hipSuccess)
    e = hipMemcpyAsync(expert_maxbits, ws + L.expert_maxbits, (size_t)E * 4, hipMemcpyDeviceToDevice, strm);
  return hip_status(e);
}

moe_status moe_dequant(const moe_expert_bank* bank, int32_t expert, int32_t matrix, int32_t bits, float* out,
                       void* stream) {
  moe_status st = check_bank(bank, true);
  if (st != MOE_OK) return st;
  if (expert < 0 || expert >= bank->n_experts || matrix < 0 || matrix > 1 || bits < 1 || bits > bank->b_max)
    return MOE_ERR_RANGE;
  if (!out) return MOE_ERR_NULL;
  const moe::MatrixDev m = matrix == 0 ? w13_of(bank) : w2_of(bank);
  return hip_status(moe::launch_dequant(m, bank->b_max, bank->group, expert, bits, bank->plane_prefix, out,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_residual_to_bf16(const float* h, uint16_t* x, int64_t n, void* stream) {
  if (n < 0) return MOE_ERR_RANGE;
  if (n == 0) return MOE_OK;
  if (!h || !x) return MOE_ERR_NULL;
  return hip_status(moe::launch_residual_to_bf16(h, x, n, static_cast<hipStream_t>(stream)));
}

moe_status moe_rmsnorm_to_bf16(const float* h, uint16_t* x, int32_t rows, int32_t d, float eps, void* stream) {
  if (rows < 0 || d < 1 || !(eps >= 0.0f) || eps > 3.0e38f) return MOE_ERR_RANGE;
  if (rows == 0) return MOE_OK;
  if (!h || !x) return MOE_ERR_NULL;
  return hip_status(moe::launch_rmsnorm_to_bf16(h, x, rows, d, eps, static_cast<hipStream_t>(stream)));
}

moe_status moe_duorate_bake(const moe_expert_bank* bank, double* delta, void* stream) {
  moe_status st = check_bank(bank, true);
  if (st != MOE_OK) return st;
  if (bank->plane_prefix) return MOE_ERR_UNSUPPORTED;
  if (!delta) return MOE_ERR_NULL;
  if (!aligned(delta, 8)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_duo_bake(w13_of(bank), bank->b_max, bank->group, bank->n_experts, delta,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_duorate_profile(const uint16_t* x, int32_t T, int32_t d, const int32_t* topk_idx, int32_t top_k,
                               int32_t E, double* act_energy, int32_t* pair_count, void* stream) {
  if (T < 0 || d < 1 || top_k < 1 || E < 1 || E > 1024) return MOE_ERR_RANGE;
  if ((int64_t)T * top_k >= (1 << 30)) return MOE_ERR_RANGE;
  if (!act_energy || !pair_count || (T > 0 && (!x || !topk_idx))) return MOE_ERR_NULL;
  if (!aligned(act_energy, 8)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_duo_profile(x, T, d, topk_idx, top_k, E, act_energy, pair_count,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_duorate_solve(const double* delta, const double* act_energy, const int32_t* pair_count, int32_t E,
                             int32_t d, int32_t b_lo, int32_t b_max, float target_rate, double* distortion,
                             uint8_t* expert_bits, double* lambda_out, void* stream) {
  if (E < 1 || E > 1024 || d < 1 || b_lo < 1 || b_max > 4 || b_lo > b_max) return MOE_ERR_RANGE;
  if (!(target_rate >= (float)b_lo && target_rate <= (float)b_max)) return MOE_ERR_RANGE;
  if (!delta || !act_energy || !pair_count || !distortion || !expert_bits) return MOE_ERR_NULL;
  if (!aligned(delta, 8) || !aligned(act_energy, 8) || !aligned(distortion, 8)) return MOE_ERR_ALIGN;
  // target = m * 2^-shift exactly (m a 24-bit integer)
  int ex = 0;
  const double fr = std::frexp((double)target_rate, &ex);
  const long long m = (long long)std::ldexp(fr, 24);
  const int shift = 24 - ex;
  return hip_status(moe::launch_duo_solve(delta, act_energy, pair_count, E, d, b_max, b_lo, b_max, m, shift,
                                          distortion, expert_bits, lambda_out, static_cast<hipStream_t>(stream)));
}

moe_status moe_bits_from_expert_widths(const int32_t* topk_idx, int32_t P, const uint8_t* expert_bits, int32_t E,
                                       uint8_t* bits, void* stream) {
  if (P < 0 || E < 1) return MOE_ERR_RANGE;
  if (P == 0) return MOE_OK;
  if (!topk_idx || !expert_bits || !bits) return MOE_ERR_NULL;
  return hip_status(moe::launch_bits_from_expert(topk_idx, P, expert_bits, E, bits, static_cast<hipStream_t>(stream)));
}

size_t moe_dpa_residuals_workspace_bytes(const moe_expert_bank* bank) {
  if (check_bank(bank, false) != MOE_OK) return 0;
  return al256((size_t)bank->n_experts * bank->b_max * bank->d_model * 8) +
         al256((size_t)bank->n_experts * bank->b_max * bank->d_ff * 8);
}

moe_status moe_dpa_residuals(const moe_expert_bank* bank, double* resid, void* workspace, size_t ws_bytes,
                             void* stream) {
  moe_status st = check_bank(bank, true);
  if (st != MOE_OK) return st;
  if (bank->plane_prefix) return MOE_ERR_UNSUPPORTED;
  if (!resid || !workspace) return MOE_ERR_NULL;
  if (!aligned(resid, 8) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  if (ws_bytes < moe_dpa_residuals_workspace_bytes(bank)) return MOE_ERR_WORKSPACE;
  hipStream_t strm = static_cast<hipStream_t>(stream);
  const int E = bank->n_experts, B = bank->b_max;
  double* d13 = static_cast<double*>(workspace);
  double* d2 = reinterpret_cast<double*>(static_cast<char*>(workspace) + al256((size_t)E * B * bank->d_model * 8));
  hipError_t e = moe::launch_duo_bake(w13_of(bank), B, bank->group, E, d13, strm);
  if (e == hipSuccess) e = moe::launch_duo_bake(w2_of(bank), B, bank->group, E, d2, strm);
  if (e == hipSuccess) e = moe::launch_resid_sum(d13, d2, E, B, bank->d_model, bank->d_ff, resid, strm);
  return hip_status(e);
}

// floor(P * (target - b_lo)) exactly on the float value of target, clamped to [0, P * (b_max - b_lo)]
static int64_t exact_chunk_budget(int32_t P, int32_t b_lo, int32_t b_max, float target) {
  int ex = 0;
  const double fr = std::frexp((double)target, &ex);
  const __int128 m = (__int128)std::ldexp(fr, 24);
  const int sh = 24 - ex;  // target = m / 2^sh, sh > 0 for targets below 2^24
  __int128 num = (__int128)P * (m - ((__int128)b_lo << sh));
  __int128 q = num >= 0 ? (num >> sh) : -((-num + ((__int128)1 << sh) - 1) >> sh);
  if (q < 0) q = 0;
  const __int128 cap = (__int128)P * (b_max - b_lo);
  if (q > cap) q = cap;
  return (int64_t)q;
}

size_t moe_dpa_alloc_workspace_bytes(int32_t P, int32_t b_lo, int32_t b_max) {
  if (P < 0 || b_lo < 1 || b_max > 4 || b_lo > b_max) return 0;
  const size_t n = (size_t)P * (b_max - b_lo);
  return al256(n * 4) + al256(n) + 256;
}

moe_status moe_dpa_alloc(const float* gate, const int32_t* topk_idx, int32_t P, const double* resid, int32_t E,
                         int32_t b_lo, int32_t b_max, float target_avg_bits, uint8_t* bits, int32_t* n_chunks_out,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (P < 0 || E < 1 || b_lo < 1 || b_max > 4 || b_lo > b_max) return MOE_ERR_RANGE;
  if (!(target_avg_bits >= (float)b_lo && target_avg_bits <= (float)b_max)) return MOE_ERR_RANGE;
  if ((int64_t)P * (b_max - b_lo) >= (1 << 30)) return MOE_ERR_RANGE;
  if (P == 0) return MOE_OK;
  if (!gate || !topk_idx || !resid || !bits || !workspace) return MOE_ERR_NULL;
  if (!aligned(resid, 8) || !aligned(workspace, 256)) return MOE_ERR_ALIGN;
  if (ws_bytes < moe_dpa_alloc_workspace_bytes(P, b_lo, b_max)) return MOE_ERR_WORKSPACE;
  const size_t n = (size_t)P * (b_max - b_lo);
  float* scores = static_cast<float*>(workspace);
  uint8_t* chosen = static_cast<uint8_t*>(workspace) + al256(n * 4);
  const int64_t nc = exact_chunk_budget(P, b_lo, b_max, target_avg_bits);
  return hip_status(moe::launch_dpa_alloc(gate, topk_idx, P, resid, E, b_max, b_lo, (int)nc, scores, chosen, bits,
                                          n_chunks_out, static_cast<hipStream_t>(stream)));
}

moe_status moe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return MOE_ERR_RANGE;
  if (bytes == 0) return MOE_OK;
  if (!buf || !sink) return MOE_ERR_NULL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_stream_read(buf, bytes, sink, MOE_STREAM_SINK, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
