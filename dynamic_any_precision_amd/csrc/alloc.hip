// Bit allocation by threshold bisection (MatMoE abstract item (3) and review,
// Core Contribution: a routing-score threshold found by binary search so the
// batch meets a target average bit-width; DPA-MoE abstract: allocation after
// routing from live gate scores), and the widths from a fixed threshold
// (the same review: the threshold set on a calibration distribution of
// routing scores and then applied as is).
//
// One block (one wave when P <= 2048).  Gate scores are mapped to
// order-preserving 32-bit keys and held in registers; tau is built from its
// most significant bit down: bit b of the answer is 0 iff
// #{key > prefix | (2^b - 1)} <= n*, which makes tau the smallest key whose
// strict upper set fits the budget.  32 steps, each one count reduced with
// DPP lane moves (plus one LDS exchange between waves for large P).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {


__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

template <int NT>
__device__ __forceinline__ int block_count(int c, int* red) {
  c = wave_sum_i_dpp(c);
  if constexpr (NT == WAVE) {
    return c;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NT / WAVE; ++w) tot += red[w];
    return tot;
  }
}

template <int NT, int AL_VPT>
__global__ __launch_bounds__(NT) void k_alloc(const float* __restrict__ gate, int P, int n_star, int b_lo,
                                              int b_max, uint8_t* __restrict__ bits, float* __restrict__ tau_out,
                                              int* __restrict__ n_hi_out) {
  __shared__ int red[NT / WAVE];
  const int tid = threadIdx.x;
  uint32_t keys[AL_VPT];
#pragma unroll
  for (int i = 0; i < AL_VPT; ++i) {
    const int idx = tid + i * NT;
    keys[i] = idx < P ? order_key(gate[idx]) : 0u;  // key 0 is below every real score
  }
  const int in_regs = NT * AL_VPT;

  auto count_above = [&](uint32_t cand) -> int {
    int c = 0;
#pragma unroll
    for (int i = 0; i < AL_VPT; ++i) c += (keys[i] > cand) ? 1 : 0;
    for (int idx = in_regs + tid; idx < P; idx += NT) c += (order_key(gate[idx]) > cand) ? 1 : 0;
    return block_count<NT>(c, red);
  };

  uint32_t prefix = 0u;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = prefix | ((1u << b) - 1u);
    if (count_above(cand) > n_star) prefix |= (1u << b);
  }
  const int n_hi = count_above(prefix);

#pragma unroll
  for (int i = 0; i < AL_VPT; ++i) {
    const int idx = tid + i * NT;
    if (idx < P) bits[idx] = (uint8_t)(keys[i] > prefix ? b_max : b_lo);
  }
  for (int idx = in_regs + tid; idx < P; idx += NT)
    bits[idx] = (uint8_t)(order_key(gate[idx]) > prefix ? b_max : b_lo);
  if (tid == 0) {
    if (tau_out) *tau_out = (n_star >= P) ? -INFINITY : key_to_float(prefix);
    if (n_hi_out) *n_hi_out = n_hi;
  }
}

// Fixed-threshold widths (calibration-threshold mode): one thread per pair.
__global__ __launch_bounds__(256) void k_bits_threshold(const float* __restrict__ gate, int P, float tau, int b_lo,
                                                        int b_max, uint8_t* __restrict__ bits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < P) bits[i] = (uint8_t)(gate[i] > tau ? b_max : b_lo);
}

}  // namespace

hipError_t launch_bits_threshold(const float* gate, int P, float tau, int b_lo, int b_max, uint8_t* bits,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(k_bits_threshold, dim3((P + 255) / 256), dim3(256), 0, stream, gate, P, tau, b_lo, b_max, bits);
  return hipGetLastError();
}

hipError_t launch_alloc(const float* gate, int P, int n_star, int b_lo, int b_max, uint8_t* bits, float* tau_out,
                        int* n_hi_out, hipStream_t stream) {
  if (P <= WAVE * 4) {
    hipLaunchKernelGGL((k_alloc<WAVE, 4>), dim3(1), dim3(WAVE), 0, stream, gate, P, n_star, b_lo, b_max, bits,
                       tau_out, n_hi_out);
  } else if (P <= WAVE * 32) {
    hipLaunchKernelGGL((k_alloc<WAVE, 32>), dim3(1), dim3(WAVE), 0, stream, gate, P, n_star, b_lo, b_max, bits,
                       tau_out, n_hi_out);
  } else {
    hipLaunchKernelGGL((k_alloc<1024, 32>), dim3(1), dim3(1024), 0, stream, gate, P, n_star, b_lo, b_max, bits,
                       tau_out, n_hi_out);
  }
  return hipGetLastError();
}

}  // namespace moe
