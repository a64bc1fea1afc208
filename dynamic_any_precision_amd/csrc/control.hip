// Fused decode control: softmax + top-k of every token, the bit allocation and
// the execution plan in one block, for batches of at most 1024 pairs whose
// plan fits the one-block plan.  Same results as the three separate steps
// (route_dev.hpp, alloc.hip, plan_dev.hpp); it saves launches and round trips
// through memory between them.  With more tokens than the block has waves
// the top-k runs as its own kernel (one wave per token across the chip) and
// this kernel takes its output: allocation and plan only.
//
// Allocation by ranks: with n* the budget, the threshold tau of the
// bisection (the smallest key whose strict upper set holds at most n*
// pairs; MatMoE abstract item (3) and review, Core Contribution: binary
// search for the threshold that meets the target average) gives a pair of
// key v the high width exactly when #{keys >= v} <= n*: if that count fits,
// a value just below v is a candidate threshold, so tau < v; if v > tau, the
// pairs at or above v are among those above tau.  Each thread counts its
// pair's rank against the P keys in LDS.
#include "common.hpp"
#include "kernels.hpp"
#include "plan_dev.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

constexpr int CTL_MAX_PAIRS = PM_NT;

__device__ __forceinline__ uint32_t gate_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool TOPK>
__global__ __launch_bounds__(PM_NT) void k_control(FfnShape s, PlanPtrs pp, const double* __restrict__ logits,
                                                   int renorm, int n_star, int b_lo, int b_max,
                                                   int* __restrict__ idx_out, float* __restrict__ gate_out,
                                                   uint8_t* __restrict__ bits_out) {
  __shared__ PlanSmallLds L;
  // gate keys live in the plan's prefix array until the plan's scan
  uint32_t* skey = reinterpret_cast<uint32_t*>(L.pre);
  static_assert(CTL_MAX_PAIRS <= PM_SMALL_WORDS, "gate keys fit the prefix array");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  plan_small_clear(s, L);

  if (!TOPK) {
    // top-k done: take its experts and gates
    for (int i = tid; i < s.P; i += PM_NT) {
      L.sexp[i] = (short)idx_out[i];
      skey[i] = gate_key(gate_out[i]);
    }
  }
  // softmax + top-k: one wave per token, tokens dealt round-robin
  for (int t = wave; TOPK && t < s.T; t += PM_NT / WAVE) {
    const int base = t * s.k;
    topk_token(logits + (size_t)t * s.E, s.E, s.k, renorm,
               [&](int j, int e, float g) {
                 idx_out[base + j] = e;
                 gate_out[base + j] = g;
                 L.sexp[base + j] = (short)e;
                 skey[base + j] = gate_key(g);
               },
               lane);
  }
  __syncthreads();

  // allocation: high width iff #{keys >= own key} <= n*
  if (tid < s.P) {
    const uint32_t v = skey[tid];
    int ge = 0;
    for (int j = 0; j < s.P; ++j) ge += skey[j] >= v ? 1 : 0;
    const int b = ge <= n_star ? b_max : b_lo;
    bits_out[tid] = (uint8_t)b;
    L.sbits[tid] = (uint8_t)b;
  }
  __syncthreads();

  // top-k never repeats an expert and allocation widths lie in [b_lo, b_max]
  plan_small_core(s, pp, L, 0);
}

}  // namespace

bool control_fits(const FfnShape& s) {
  return s.P <= CTL_MAX_PAIRS && (long)s.E * s.B * s.W <= PM_SMALL_WORDS && s.E <= 256;
}

// the top-k inside the control kernel while every token has a wave of its own
bool control_does_topk(const FfnShape& s) { return s.T <= PM_NT / WAVE; }

hipError_t launch_control(const FfnShape& s, const FfnLayout& L, char* ws, const double* logits, int renorm,
                          int n_star, int b_lo, int b_max, int* idx, float* gate, uint8_t* bits,
                          hipStream_t stream) {
  if (control_does_topk(s))
    hipLaunchKernelGGL(k_control<true>, dim3(1), dim3(PM_NT), 0, stream, s, plan_ptrs(L, ws), logits, renorm, n_star,
                       b_lo, b_max, idx, gate, bits);
  else
    hipLaunchKernelGGL(k_control<false>, dim3(1), dim3(PM_NT), 0, stream, s, plan_ptrs(L, ws), logits, renorm,
                       n_star, b_lo, b_max, idx, gate, bits);
  return hipGetLastError();
}

}  // namespace moe
