// Residual-aware chunk allocation ("DPA-MoE: A Runtime Precision Control
// Framework for MoE Inference", abstract: per-expert reconstruction
// residuals profiled offline, chunks allocated at inference time from live
// router gate scores), over widths b_lo..b_max:
//   resid[e][b-1] = ||W_hat^(B) - W_hat^(b)||_F^2 over both matrices of
//                   expert e (from the per-column bakes of both matrices);
//   score(p, k)   = fp32(fp64(g_p)^2 * (resid[e][k-2] - resid[e][k-1])),
//                   the gate-weighted residual plane k of pair p removes,
//                   k = b_lo+1 .. b_max;
//   the extra planes go to the floor(P (target - b_lo)) candidates of
//   highest score without splitting equal scores (the threshold bisection
//   of the allocation kernel, run over the candidates), and a pair's width
//   is b_lo plus its chosen candidates.
#include "common.hpp"
#include "kernels.hpp"

// Every floating-point operation of this file is rounded on its own: no
// multiply-add contraction, so decisions taken on these values are the ones
// any IEEE double (or float) evaluation of the same expressions takes.
#pragma clang fp contract(off)

namespace moe {
namespace {

// per-expert residual: one block per (expert, width), fixed-order sums
__global__ __launch_bounds__(256) void k_resid_sum(const double* __restrict__ d13, const double* __restrict__ d2,
                                                   int B, int d, int f, double* __restrict__ resid) {
  const int e = blockIdx.x, b = blockIdx.y;
  const double* p13 = d13 + ((size_t)e * B + b) * d;
  const double* p2 = d2 + ((size_t)e * B + b) * f;
  double s = 0.0;
  for (int c = threadIdx.x; c < d; c += 256) s += p13[c];
  for (int c = threadIdx.x; c < f; c += 256) s += p2[c];
  s = wave_sum_d(s);
  __shared__ double part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) resid[(size_t)e * B + b] = ((part[0] + part[1]) + part[2]) + part[3];
}

// candidate scores, one thread per (pair, extra plane)
__global__ void k_dpa_scores(const float* __restrict__ gate, const int* __restrict__ idx, int P,
                             const double* __restrict__ resid, int E, int B, int b_lo, int nk,
                             float* __restrict__ scores) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P * nk) return;
  const int p = i / nk, k = b_lo + 1 + (i - p * nk);
  const int e = idx[p];
  float s = 0.0f;
  if (e >= 0 && e < E) {
    const double g = (double)gate[p];
    const double gain = resid[(size_t)e * B + k - 2] - resid[(size_t)e * B + k - 1];
    s = (float)((g * g) * gain);
  }
  scores[i] = s;
}

// widths: b_lo plus the chosen candidates of each pair
__global__ void k_dpa_count(const uint8_t* __restrict__ chosen, int P, int nk, int b_lo, uint8_t* __restrict__ bits) {
  const int p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= P) return;
  int b = b_lo;
  for (int k = 0; k < nk; ++k) b += chosen[(size_t)p * nk + k];
  bits[p] = (uint8_t)b;
}

}  // namespace

hipError_t launch_resid_sum(const double* d13, const double* d2, int E, int B, int d, int f, double* resid,
                            hipStream_t stream) {
  hipLaunchKernelGGL(k_resid_sum, dim3(E, B), dim3(256), 0, stream, d13, d2, B, d, f, resid);
  return hipGetLastError();
}

hipError_t launch_dpa_alloc(const float* gate, const int* idx, int P, const double* resid, int E, int B, int b_lo,
                            int n_chunks, float* scores, uint8_t* chosen, uint8_t* bits, int* n_chosen_out,
                            hipStream_t stream) {
  const int nk = B - b_lo;
  if (nk == 0) {
    hipLaunchKernelGGL(k_dpa_count, dim3((P + 255) / 256), dim3(256), 0, stream, chosen, P, 0, b_lo, bits);
    return hipGetLastError();
  }
  const long n = (long)P * nk;
  hipLaunchKernelGGL(k_dpa_scores, dim3((n + 255) / 256), dim3(256), 0, stream, gate, idx, P, resid, E, B, b_lo, nk,
                     scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_alloc(scores, (int)n, n_chunks, 0, 1, chosen, nullptr, n_chosen_out, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_dpa_count, dim3((P + 255) / 256), dim3(256), 0, stream, chosen, P, nk, b_lo, bits);
  return hipGetLastError();
}

}  // namespace moe
