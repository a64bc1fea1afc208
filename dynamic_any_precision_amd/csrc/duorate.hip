// DuoRate two-rate per-expert allocation ("DuoRate: Two-Rate Per-Expert
// Precision Allocation for Mixture-of-Experts Serving", abstract): the store
// is one uniform tier of a prefix-readable bitplane stream; offline a
// distortion tensor is baked from it; online a prefill is profiled without
// labels, and a Lagrangian rate-distortion problem under the decode rate is
// solved per expert (routing frequency cancels from each decision) with one
// dot product per expert and width plus a bisection on the multiplier.
//
//   bake:     Delta[e][b-1][c] = sum_n (s(n, c) (q(n, c) - qhat_b(n, c)))^2
//             over the rows of W13, qhat_b the floor-and-compensation code
//             of the first b planes (the -z s terms of both reads cancel);
//   profile:  n[e] = routed pairs of expert e, a[e][c] = sum of x[t][c]^2
//             over them, in token order;
//   distort:  Dbar[e][b-1] = <Delta[e][b-1], a[e]> / n[e]  (0 if n[e] = 0);
//   solve:    b_e(lam) = argmin_b fl(Dbar + fl(lam b)), ties to the smaller
//             b; lam* = the smallest non-negative double with
//             sum_e n[e] b_e(lam) <= floor(target * sum_e n[e]), by
//             bisection over the bit patterns of doubles in
//             [0, 2 max_e Dbar[e][b_lo-1] + 1].
#include "common.hpp"
#include "kernels.hpp"

// Every floating-point operation of this file is rounded on its own: no
// multiply-add contraction, so decisions taken on these values are the ones
// any IEEE double (or float) evaluation of the same expressions takes.
#pragma clang fp contract(off)

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// bake: one block per (expert, 128-column block of W13's input); thread =
// (column c of the block, half h of the rows).  Each thread rebuilds the
// code q of every row of its half in its column from the planes, and
// accumulates the squared F&C error of every width.

constexpr int BAKE_THREADS = 256;

__global__ __launch_bounds__(BAKE_THREADS) void k_duo_bake(const uint32_t* __restrict__ planes,
                                                           const float* __restrict__ sz, int N, int K, int B, int g,
                                                           double* __restrict__ delta) {
  const int e = blockIdx.x, kb = blockIdx.y;
  const int c = threadIdx.x & 127, h = threadIdx.x >> 7;
  const int j = c >> 5, i = c & 31;
  const size_t plane_words = (size_t)N * K / 32;
  const uint32_t* pe = planes + (size_t)e * B * plane_words;
  const int NQG = K / g;
  const float* se = sz + (size_t)e * (N / 16) * NQG * 32;
  const int G = (128 * kb + c) / g;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int n = h; n < N; n += 2) {
    const int tile = n >> 4, r = n & 15;
    const size_t w = (size_t)tile * (16 * K / 32) + 64 * kb + 16 * j + r;
    int q = 0;
    for (int p = 0; p < B; ++p) q = (q << 1) | ((pe[p * plane_words + w] >> i) & 1u);
    const double s = (double)se[((size_t)tile * NQG + G) * 32 + r];
    for (int b = 1; b <= B; ++b) {
      const int dl = B - b;
      const double qh = (double)((q >> dl) << dl) + 0.5 * (double)((1 << dl) - 1);
      const double err = ((double)q - qh) * s;
      acc[b - 1] += err * err;
    }
  }
  __shared__ double part[4][128];
  if (h == 1)
    for (int b = 0; b < B; ++b) part[b][c] = acc[b];
  __syncthreads();
  if (h == 0)
    for (int b = 0; b < B; ++b) delta[((size_t)e * B + b) * K + 128 * kb + c] = acc[b] + part[b][c];
}

// ---------------------------------------------------------------------------
// profile: one block per (expert, 256-column slice).  The block walks the
// pairs in order in steps of 256, marks those routed to its expert in four
// wave ballots, and adds x^2 of the marked tokens, in pair order, to one
// fp64 accumulator per column.

constexpr int PROF_THREADS = 256;

__global__ __launch_bounds__(PROF_THREADS) void k_duo_profile(const uint16_t* __restrict__ x, int T, int d,
                                                              const int* __restrict__ idx, int k, int E,
                                                              double* __restrict__ a, int* __restrict__ n) {
  const int e = blockIdx.x;
  const int col = blockIdx.y * PROF_THREADS + threadIdx.x;
  const int P = T * k;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __shared__ unsigned long long mask[4];
  double acc = 0.0;
  int cnt = 0;
  for (int p0 = 0; p0 < P; p0 += PROF_THREADS) {
    const int p = p0 + threadIdx.x;
    const bool hit = p < P && idx[p] == e;
    const unsigned long long m = __ballot(hit);
    if (lane == 0) mask[wv] = m;
    __syncthreads();
    for (int w = 0; w < 4; ++w) {
      unsigned long long mm = mask[w];
      while (mm) {
        const int b = __ffsll((long long)mm) - 1;
        mm &= mm - 1;
        const int t = (p0 + 64 * w + b) / k;
        if (col < d) {
          const double v = (double)bf16_to_f32(x[(size_t)t * d + col]);
          acc += v * v;
        }
        ++cnt;
      }
    }
    __syncthreads();
  }
  if (col < d) a[(size_t)e * d + col] = acc;
  if (blockIdx.y == 0 && threadIdx.x == 0) n[e] = cnt;
}

// ---------------------------------------------------------------------------
// per-token distortion: one block per (expert, width); fixed-order reduction.

__global__ __launch_bounds__(256) void k_duo_distortion(const double* __restrict__ delta, const double* __restrict__ a,
                                                        const int* __restrict__ n, int d, int B,
                                                        double* __restrict__ D) {
  const int e = blockIdx.x, b = blockIdx.y;
  const double* dl = delta + ((size_t)e * B + b) * d;
  const double* ae = a + (size_t)e * d;
  double s = 0.0;
  for (int c = threadIdx.x; c < d; c += 256) s += dl[c] * ae[c];
  s = wave_sum_d(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = ((part[0] + part[1]) + part[2]) + part[3];
    const int ne = n[e];
    D[(size_t)e * B + b] = ne > 0 ? tot / (double)ne : 0.0;
  }
}

// ---------------------------------------------------------------------------
// solve: one block, one thread per expert (E <= 1024).

// The cost fl(D + fl(lam b)): a rounded product and a rounded sum.
__device__ __forceinline__ int lag_width(const double* De, double lam, int b_lo, int b_max) {
  double best = 0.0;
  int bw = b_lo;
  for (int b = b_lo; b <= b_max; ++b) {
    const double c = De[b - 1] + lam * (double)b;
    if (b == b_lo || c < best) {
      best = c;
      bw = b;
    }
  }
  return bw;
}

__device__ long long block_sum_ll(long long v, long long* red) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  const int nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

__device__ double block_max_d(double v, double* red) {
  v = wave_max_d(v);
  const int nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = red[0];
  for (int w = 1; w < nw; ++w) t = fmax(t, red[w]);
  return t;
}

__global__ __launch_bounds__(1024) void k_duo_solve(const double* __restrict__ D, const int* __restrict__ n, int E,
                                                    int B, int b_lo, int b_max, long long tmant, int tshift,
                                                    uint8_t* __restrict__ widths, double* __restrict__ lam_out) {
  __shared__ long long red_ll[16];
  __shared__ double red_d[16];
  const int e = threadIdx.x;
  const bool live = e < E;
  double De[4] = {0.0, 0.0, 0.0, 0.0};
  long long ne = 0;
  if (live) {
    for (int b = 0; b < B; ++b) De[b] = D[(size_t)e * B + b];
    ne = n[e];
  }
  // budget floor(target * N): target = tmant * 2^-tshift exactly
  const long long N = block_sum_ll(ne, red_ll);
  const long long budget = (tmant * N) >> tshift;
  const double dmax = block_max_d(live ? De[b_lo - 1] : 0.0, red_d);
  const double lam_hi = 2.0 * dmax + 1.0;
  unsigned long long lo = 0, hi = (unsigned long long)__double_as_longlong(lam_hi);
  while (lo < hi) {
    const unsigned long long mid = lo + (hi - lo) / 2;
    const double lam = __longlong_as_double((long long)mid);
    const long long s = block_sum_ll(live ? ne * lag_width(De, lam, b_lo, b_max) : 0, red_ll);
    if (s <= budget)
      hi = mid;
    else
      lo = mid + 1;
  }
  const double lam = __longlong_as_double((long long)lo);
  if (live) widths[e] = (uint8_t)lag_width(De, lam, b_lo, b_max);
  if (e == 0 && lam_out) *lam_out = lam;
}

// per-pair widths of a batch from the per-expert widths (0 for an index
// outside [0, E), which the FFN drops)
__global__ void k_bits_from_expert(const int* __restrict__ idx, int P, const uint8_t* __restrict__ w, int E,
                                   uint8_t* __restrict__ bits) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P) return;
  const int e = idx[i];
  bits[i] = (e >= 0 && e < E) ? w[e] : (uint8_t)0;
}

}  // namespace

hipError_t launch_duo_bake(MatrixDev m, int B, int g, int E, double* delta, hipStream_t stream) {
  hipLaunchKernelGGL(k_duo_bake, dim3(E, m.K / 128), dim3(BAKE_THREADS), 0, stream, m.planes, m.sz, m.N, m.K, B, g,
                     delta);
  return hipGetLastError();
}

hipError_t launch_duo_profile(const uint16_t* x, int T, int d, const int* idx, int k, int E, double* a, int* n,
                              hipStream_t stream) {
  hipLaunchKernelGGL(k_duo_profile, dim3(E, (d + PROF_THREADS - 1) / PROF_THREADS), dim3(PROF_THREADS), 0, stream, x,
                     T, d, idx, k, E, a, n);
  return hipGetLastError();
}

hipError_t launch_duo_solve(const double* delta, const double* a, const int* n, int E, int d, int B, int b_lo,
                            int b_max, long long tmant, int tshift, double* D, uint8_t* widths, double* lam_out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_duo_distortion, dim3(E, B), dim3(256), 0, stream, delta, a, n, d, B, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int threads = ((E + 63) / 64) * 64;
  hipLaunchKernelGGL(k_duo_solve, dim3(1), dim3(threads), 0, stream, D, n, E, B, b_lo, b_max, tmant, tshift, widths,
                     lam_out);
  return hipGetLastError();
}

hipError_t launch_bits_from_expert(const int* idx, int P, const uint8_t* w, int E, uint8_t* bits, hipStream_t stream) {
  hipLaunchKernelGGL(k_bits_from_expert, dim3((P + 255) / 256), dim3(256), 0, stream, idx, P, w, E, bits);
  return hipGetLastError();
}

}  // namespace moe
