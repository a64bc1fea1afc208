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
// DPP lane moves.  Larger batches take four radix passes instead (below).
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

// Block-wide sum of one count per thread.  Successive calls alternate
// between two halves of `red` (2 x NT/64 ints), so one barrier per call
// suffices: a half is written again only two calls later, after every thread
// has passed the barrier of the call in between.
template <int NT>
__device__ __forceinline__ int block_count(int c, int* red, int& parity) {
  c = wave_sum_i_dpp(c);
  if constexpr (NT == WAVE) {
    return c;
  } else {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    int* r = red + parity * (NT / WAVE);
    parity ^= 1;
    if (lane == 0) r[wave] = c;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NT / WAVE; ++w) tot += r[w];
    return tot;
  }
}

template <int NT, int AL_VPT>
__global__ __launch_bounds__(NT) void k_alloc(const float* __restrict__ gate, int P, int n_star, int b_lo,
                                              int b_max, uint8_t* __restrict__ bits, float* __restrict__ tau_out,
                                              int* __restrict__ n_hi_out) {
  __shared__ int red[2 * (NT / WAVE)];
  int parity = 0;
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
    return block_count<NT>(c, red, parity);
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

// Large batches: the same tau by a radix descent over 8-bit digits instead of
// 32 bisection steps.  In each of four passes the keys that share the prefix
// found so far are histogrammed by their next digit, and the digit becomes
// the smallest d for which the keys above the prefix plus the prefix's keys
// with a digit above d number at most n*.  This is the smallest 32-bit value
// whose strict upper set fits the budget, the bisection's answer.
template <int NT, int AL_VPT>
__global__ __launch_bounds__(NT) void k_alloc_radix(const float* __restrict__ gate, int P, int n_star, int b_lo,
                                                    int b_max, uint8_t* __restrict__ bits, float* __restrict__ tau_out,
                                                    int* __restrict__ n_hi_out) {
  __shared__ int hist[256];
  __shared__ uint32_t s_prefix;
  __shared__ int s_above;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t keys[AL_VPT];
#pragma unroll
  for (int i = 0; i < AL_VPT; ++i) {
    const int idx = tid + i * NT;
    keys[i] = idx < P ? order_key(gate[idx]) : 0u;
  }
  const int in_regs = NT * AL_VPT;
  // The keys' common leading bits (from their minimum and maximum) are the
  // answer's leading bits already; the first digit is the 8 bits below them,
  // so its histogram spreads over many bins (gates share their top key bits,
  // and a first digit of the top 8 bits put them all on a few bins, where
  // the atomics serialise).  Then 8-bit digits down to bit 0.
  __shared__ uint32_t s_mm[2 * (NT / WAVE)];
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < AL_VPT; ++i)
    if (tid + i * NT < P) {
      kmin = min(kmin, keys[i]);
      kmax = max(kmax, keys[i]);
    }
  for (int idx = in_regs + tid; idx < P; idx += NT) {
    const uint32_t k = order_key(gate[idx]);
    kmin = min(kmin, k);
    kmax = max(kmax, k);
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, m, WAVE));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, WAVE));
  }
  if (lane == 0) {
    s_mm[2 * wave] = kmin;
    s_mm[2 * wave + 1] = kmax;
  }
  __syncthreads();
  kmin = 0xFFFFFFFFu;
  kmax = 0u;
#pragma unroll
  for (int w = 0; w < NT / WAVE; ++w) {
    kmin = min(kmin, s_mm[2 * w]);
    kmax = max(kmax, s_mm[2 * w + 1]);
  }
  // With n* < P the answer lies in [kmin, kmax] (at least one key is at or
  // below it, none above kmax is needed), so it carries the keys' common
  // leading bits; with n* >= P it is 0 and the descent starts from the top.
  const uint32_t diff = kmin ^ kmax;
  const int hb = (diff && n_star < P) ? 31 - __clz((int)diff) : 31;  // highest bit where the keys differ
  uint32_t prefix = hb >= 31 ? 0u : (kmin & ~((2u << hb) - 1u));
  int above = 0;
  int shift = hb >= 7 ? hb - 7 : 0;
  int width = hb - shift + 1;
  for (;;) {
    for (int j = tid; j < 256; j += NT) hist[j] = 0;
    __syncthreads();
    const uint32_t top = (uint32_t)(shift + width);
    const uint32_t hmask = top >= 32 ? 0u : (0xFFFFFFFFu << top);
    const uint32_t dmask = (1u << width) - 1u;
#pragma unroll
    for (int i = 0; i < AL_VPT; ++i)
      if (tid + i * NT < P && (keys[i] & hmask) == prefix) atomicAdd(&hist[(keys[i] >> shift) & dmask], 1);
    for (int idx = in_regs + tid; idx < P; idx += NT) {
      const uint32_t k = order_key(gate[idx]);
      if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1);
    }
    __syncthreads();
    if (wave == 0) {
      const int h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
      const int ls = h0 + h1 + h2 + h3;
      int suf = ls;  // sum over lanes >= this one
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) {
        const int o = __shfl_down(suf, m, WAVE);
        if (lane + m < 64) suf += o;
      }
      // the prefix's keys with a digit above 4 lane + i
      int sd[4];
      sd[3] = suf - ls;
      sd[2] = sd[3] + h3;
      sd[1] = sd[2] + h2;
      sd[0] = sd[1] + h1;
      int dmin = 256;
#pragma unroll
      for (int i = 3; i >= 0; --i)
        if (above + sd[i] <= n_star) dmin = 4 * lane + i;
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) dmin = min(dmin, __shfl_xor(dmin, m, WAVE));
      if (lane == (dmin >> 2)) {
        s_prefix = prefix | ((uint32_t)dmin << shift);
        s_above = above + sd[dmin & 3];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    above = s_above;
    if (shift == 0) break;
    width = shift < 8 ? shift : 8;
    shift -= width;
  }
#pragma unroll
  for (int i = 0; i < AL_VPT; ++i) {
    const int idx = tid + i * NT;
    if (idx < P) bits[idx] = (uint8_t)(keys[i] > prefix ? b_max : b_lo);
  }
  for (int idx = in_regs + tid; idx < P; idx += NT)
    bits[idx] = (uint8_t)(order_key(gate[idx]) > prefix ? b_max : b_lo);
  if (tid == 0) {
    if (tau_out) *tau_out = (n_star >= P) ? -INFINITY : key_to_float(prefix);
    if (n_hi_out) *n_hi_out = above;
  }
}

// Fixed-threshold widths (calibration-threshold mode): one thread per pair.
__global__ __launch_bounds__(256) void k_bits_threshold(const float* __restrict__ gate, int P, float tau, int b_lo,
                                                        int b_max, uint8_t* __restrict__ bits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < P) bits[i] = (uint8_t)(gate[i] > tau ? b_max : b_lo);
}

// The same with tau read from device memory (written there by the allocation
// kernel's tau output, so a changed target needs no host round trip).
__global__ __launch_bounds__(256) void k_bits_threshold_dev(const float* __restrict__ gate, int P,
                                                            const float* __restrict__ tau, int b_lo, int b_max,
                                                            uint8_t* __restrict__ bits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const float t = *tau;
  if (i < P) bits[i] = (uint8_t)(gate[i] > t ? b_max : b_lo);
}

}  // namespace

hipError_t launch_bits_threshold_dev(const float* gate, int P, const float* tau, int b_lo, int b_max, uint8_t* bits,
                                     hipStream_t stream) {
  hipLaunchKernelGGL(k_bits_threshold_dev, dim3((P + 255) / 256), dim3(256), 0, stream, gate, P, tau, b_lo, b_max,
                     bits);
  return hipGetLastError();
}

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
    hipLaunchKernelGGL((k_alloc_radix<1024, 32>), dim3(1), dim3(1024), 0, stream, gate, P, n_star, b_lo, b_max, bits,
                       tau_out, n_hi_out);
  }
  return hipGetLastError();
}

}  // namespace moe
