// Router: fp64-accumulated logits GEMV, then softmax over all experts and
// top-k.  ("routing each token to a small set of experts", DPA-MoE abstract;
// "routing scores", MatMoE abstract.)
//
// Logits: grid (E/2 expert tiles, T/2 or T/4 token tiles), 512 threads.  The
// eight waves of a block split the hidden dimension; each accumulates the
// (expert, token) dot products of its tile and slice in float64 from exact
// bf16 / fp32 inputs, a butterfly reduce-scatter leaves lane l with the slice
// sum of pair l mod (tile size), and wave 0 adds the eight slices in a fixed
// order.  Small
// tiles give many blocks: the kernel is latency-bound at decode sizes.
// Prefill-sized batches (T >= 256) take the logits on the fp64 matrix cores
// instead: one wave per 16-token x 16-expert tile, v_mfma_f64_16x16x4f64 over
// the hidden dimension (the same exact products, accumulated in fp64).
// Top-k: one wave per token, k rounds of a wave-wide arg-max over (logit
// desc, index asc) through DPP lane moves.
#include "common.hpp"
#include "kernels.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

// logits tiles (tokens x experts per block): about a thousand blocks at
// decode sizes -- 2 x 2 up to 32 tokens, 4 x 2 above
constexpr int RT_ET = 2;
constexpr int RT_WAVES = 8;
#ifndef RT_TOPK_WAVES
#define RT_TOPK_WAVES 1  // waves (tokens) per top-k block: one, so the tokens spread over the CUs
#endif

template <int M, int N>
__device__ __forceinline__ void butterfly_step(double (&v)[N], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const double send = up ? v[i] : v[i + M];
    const double keep = up ? v[i + M] : v[i];
    v[i] = keep + __shfl_xor(send, M, WAVE);
  }
  if constexpr (M > 1) butterfly_step<M / 2, N>(v, lane);
}

// Reduce-scatter of N values per lane (N a power of two <= 32): after the
// step with mask M, v[0 .. M-1] hold partial sums of the indices selected by
// the lane's bits below N; the xor steps from N up then fold the wave's
// groups of N lanes, so v[0] is the wave total of index lane % N.
template <int N>
__device__ __forceinline__ void butterfly(double (&v)[N], int lane) {
  butterfly_step<N / 2, N>(v, lane);
#pragma unroll
  for (int m = N; m < WAVE; m <<= 1) v[0] += __shfl_xor(v[0], m, WAVE);
}

// One wave per token.
__global__ __launch_bounds__(256) void k_route_topk(const double* __restrict__ logits, int T, int E, int k, int renorm,
                                                    int* __restrict__ idx_out, float* __restrict__ gate_out) {
  const int t = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  if (t >= T) return;
  int* io = idx_out + (size_t)t * k;
  float* go = gate_out + (size_t)t * k;
  topk_token(logits + (size_t)t * E, E, k, renorm, [&](int j, int e, float g) { io[j] = e; go[j] = g; },
             threadIdx.x & 63);
}

template <int RT_TT>
__global__ __launch_bounds__(RT_WAVES * 64) void k_route_logits(const uint16_t* __restrict__ x, int T, int d,
                                                      const float* __restrict__ W, int E,
                                                      const float* __restrict__ bias, double* __restrict__ logits) {
  __shared__ double part[RT_WAVES][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * RT_TT;
  const int nt = min(RT_TT, T - t0);
  const int e0 = blockIdx.x * RT_ET;
  const int slice = ((d / RT_WAVES) + 3) & ~3;
  const int c_beg = wave * slice;
  const int c_end = min(d, c_beg + slice);

  double acc[RT_ET * RT_TT];
#pragma unroll
  for (int i = 0; i < RT_ET * RT_TT; ++i) acc[i] = 0.0;

#pragma unroll 2
  for (int c = c_beg + lane * 4; c < c_end; c += 256) {
    float4 wv[RT_ET];
#pragma unroll
    for (int ee = 0; ee < RT_ET; ++ee)
      wv[ee] = (e0 + ee < E) ? *reinterpret_cast<const float4*>(W + (size_t)(e0 + ee) * d + c)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
    uint2 xv[RT_TT];
#pragma unroll
    for (int tt = 0; tt < RT_TT; ++tt)
      xv[tt] = (tt < nt) ? *reinterpret_cast<const uint2*>(x + (size_t)(t0 + tt) * d + c) : make_uint2(0, 0);
#pragma unroll
    for (int tt = 0; tt < RT_TT; ++tt) {
      const double x0 = bf16_to_f32(xv[tt].x & 0xFFFFu), x1 = bf16_to_f32(xv[tt].x >> 16);
      const double x2 = bf16_to_f32(xv[tt].y & 0xFFFFu), x3 = bf16_to_f32(xv[tt].y >> 16);
#pragma unroll
      for (int ee = 0; ee < RT_ET; ++ee) {
        double a = acc[ee * RT_TT + tt];
        a = fma((double)wv[ee].x, x0, a);
        a = fma((double)wv[ee].y, x1, a);
        a = fma((double)wv[ee].z, x2, a);
        a = fma((double)wv[ee].w, x3, a);
        acc[ee * RT_TT + tt] = a;
      }
    }
  }
  static_assert(RT_ET * RT_TT <= 32 && (RT_ET * RT_TT & (RT_ET * RT_TT - 1)) == 0, "reduce-scatter width");
  butterfly<RT_ET * RT_TT>(acc, lane);
  part[wave][lane] = acc[0];
  __syncthreads();
  if (wave == 0 && lane < RT_ET * RT_TT) {
    const int ee = lane / RT_TT, tt = lane % RT_TT;
    const int e = e0 + ee, t = t0 + tt;
    if (e < E && tt < nt) {
      double l = part[0][lane];
#pragma unroll
      for (int w = 1; w < RT_WAVES; ++w) l += part[w][lane];
      if (bias) l += (double)bias[e];
      logits[(size_t)t * E + e] = l;
    }
  }

}

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// One wave per 16 x 16 (token, expert) tile, four expert tiles per block.
// Matrix-core operand layouts (16x16x4, fp64): lane l supplies A[l%16][l/16]
// and B[l/16][l%16] and holds D[l/16 + 4r][l%16], r = 0..3 (rows interleaved,
// unlike the fp32 16x16 layouts).  The hidden
// dimension is walked in steps of 16 in which lane l owns columns
// k0 + 4(l/16) + s, s = 0..3 (A and B share this order of k, which a sum does
// not depend on): one 8-byte x load and one 16-byte W load per lane and step.
__global__ __launch_bounds__(256) void k_route_logits_mfma(const uint16_t* __restrict__ x, int T, int d,
                                                           const float* __restrict__ W, int E,
                                                           const float* __restrict__ bias,
                                                           double* __restrict__ logits) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * 16;
  const int e0 = (blockIdx.x * 4 + wave) * 16;
  if (e0 >= E) return;
  const int r16 = lane & 15, q = lane >> 4;
  const int t = t0 + r16, e = e0 + r16;
  const uint16_t* xr = x + (size_t)(t < T ? t : 0) * d + 4 * q;
  const float* wr = W + (size_t)(e < E ? e : 0) * d + 4 * q;
  // RING steps of 16 columns in flight (each wave's loads are a chain of
  // dependent round trips otherwise); two accumulators alternate by step.
  constexpr int RING = 4;
  f64x4_t acc[2] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  uint2 xq[RING];
  float4 wq[RING];
#pragma unroll
  for (int r = 0; r < RING; ++r) {
    const int kk = 16 * r;
    xq[r] = (t < T && kk < d) ? *reinterpret_cast<const uint2*>(xr + kk) : make_uint2(0u, 0u);
    wq[r] = (e < E && kk < d) ? *reinterpret_cast<const float4*>(wr + kk) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int k0 = 0; k0 < d; k0 += 16 * RING) {
#pragma unroll
    for (int r = 0; r < RING; ++r) {
      const uint2 xc = xq[r];
      const float4 wc = wq[r];
      const int kn = k0 + 16 * (r + RING);
      if (kn < d) {
        xq[r] = t < T ? *reinterpret_cast<const uint2*>(xr + kn) : make_uint2(0u, 0u);
        wq[r] = e < E ? *reinterpret_cast<const float4*>(wr + kn) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (k0 + 16 * r < d) {
        f64x4_t& a = acc[r & 1];
        a = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(xc.x & 0xFFFFu), (double)wc.x, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(xc.x >> 16), (double)wc.y, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(xc.y & 0xFFFFu), (double)wc.z, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f64_16x16x4f64((double)bf16_to_f32(xc.y >> 16), (double)wc.w, a, 0, 0, 0);
      }
    }
  }
  if (e < E) {
    const double b = bias ? (double)bias[e] : 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tt = t0 + q + 4 * r;
      if (tt < T) logits[(size_t)tt * E + e] = (acc[0][r] + acc[1][r]) + b;
    }
  }
}

}  // namespace

size_t route_workspace_bytes(int T, int E) {
  return ((size_t)T * E * sizeof(double) + 255) & ~size_t(255);
}

hipError_t launch_route_logits(const uint16_t* x, int T, int d, const float* W, int E, const float* bias,
                               double* logits, hipStream_t stream) {
  if (T >= 256) {
    dim3 grid((E + 63) / 64, (T + 15) / 16);
    hipLaunchKernelGGL(k_route_logits_mfma, grid, dim3(256), 0, stream, x, T, d, W, E, bias, logits);
    return hipGetLastError();
  }
  if (T <= 32) {
    dim3 grid((E + RT_ET - 1) / RT_ET, (T + 1) / 2);
    hipLaunchKernelGGL(k_route_logits<2>, grid, dim3(RT_WAVES * 64), 0, stream, x, T, d, W, E, bias, logits);
  } else {
    dim3 grid((E + RT_ET - 1) / RT_ET, (T + 3) / 4);
    hipLaunchKernelGGL(k_route_logits<4>, grid, dim3(RT_WAVES * 64), 0, stream, x, T, d, W, E, bias, logits);
  }
  return hipGetLastError();
}

hipError_t launch_route_topk(const double* logits, int T, int E, int k, int renorm, int* idx, float* gate,
                             hipStream_t stream) {
  hipLaunchKernelGGL(k_route_topk, dim3((T + RT_TOPK_WAVES - 1) / RT_TOPK_WAVES), dim3(64 * RT_TOPK_WAVES), 0, stream,
                     logits, T, E, k, renorm, idx, gate);
  return hipGetLastError();
}

hipError_t launch_route(const uint16_t* x, int T, int d, const float* W, int E, const float* bias, int k,
                        int renorm, int* idx, float* gate, void* ws, hipStream_t stream) {
  double* logits = static_cast<double*>(ws);
  hipError_t e = launch_route_logits(x, T, d, W, E, bias, logits, stream);
  if (e == hipSuccess) e = launch_route_topk(logits, T, E, k, renorm, idx, gate, stream);
  return e;
}

}  // namespace moe
