// Router: fp64-accumulated logits GEMV, softmax over all experts and top-k,
// in one launch.  ("routing each token to a small set of experts",
// DPA-MoE abstract; "routing scores", MatMoE abstract.)
//
// Grid (E/16 expert tiles, T/8 token tiles), 256 threads.  Each wave owns 4
// experts of the tile and accumulates 4 x 8 (expert, token) dot products in
// float64 over its slice of the hidden dimension; a butterfly
// reduce-scatter leaves lane l with the full sum of pair l mod 32.  The last block
// of a token tile to finish (atomic counter, reset afterwards) runs softmax
// and top-k for the tile's tokens, one wave per token.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int RT_TT = 8;   // tokens per block
constexpr int RT_EW = 4;   // experts per wave
constexpr int RT_ET = 16;  // experts per block

template <int M>
__device__ __forceinline__ void butterfly_step(double (&v)[32], int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    const double send = up ? v[i] : v[i + M];
    const double keep = up ? v[i + M] : v[i];
    v[i] = keep + __shfl_xor(send, M, WAVE);
  }
  if constexpr (M > 1) butterfly_step<M / 2>(v, lane);
}

// Full sum across the two wave halves, then a reduce-scatter: after the step
// with mask M, v[0 .. M-1] hold partial sums of the indices selected by the
// lane's higher bits; finally v[0] = total of index lane % 32.
__device__ __forceinline__ void butterfly32(double (&v)[32], int lane) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] += __shfl_xor(v[i], 32, WAVE);
  butterfly_step<16>(v, lane);
}

__global__ __launch_bounds__(256) void k_route(const uint16_t* __restrict__ x, int T, int d,
                                               const float* __restrict__ W, int E,
                                               const float* __restrict__ bias, int k, int renorm,
                                               int* __restrict__ idx_out, float* __restrict__ gate_out,
                                               double* __restrict__ logits, unsigned* __restrict__ counters) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.y * RT_TT;
  const int nt = min(RT_TT, T - t0);
  const int e0 = blockIdx.x * RT_ET + wave * RT_EW;

  double acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.0;

  for (int c = lane * 4; c < d; c += 256) {
    double w[RT_EW][4];
#pragma unroll
    for (int ee = 0; ee < RT_EW; ++ee) {
      float4 wv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e0 + ee < E) wv = *reinterpret_cast<const float4*>(W + (size_t)(e0 + ee) * d + c);
      w[ee][0] = wv.x; w[ee][1] = wv.y; w[ee][2] = wv.z; w[ee][3] = wv.w;
    }
#pragma unroll
    for (int tt = 0; tt < RT_TT; ++tt) {
      if (tt < nt) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + tt) * d + c);
        const double x0 = bf16_to_f32(xv.x & 0xFFFFu), x1 = bf16_to_f32(xv.x >> 16);
        const double x2 = bf16_to_f32(xv.y & 0xFFFFu), x3 = bf16_to_f32(xv.y >> 16);
#pragma unroll
        for (int ee = 0; ee < RT_EW; ++ee) {
          double a = acc[ee * RT_TT + tt];
          a = fma(w[ee][0], x0, a);
          a = fma(w[ee][1], x1, a);
          a = fma(w[ee][2], x2, a);
          a = fma(w[ee][3], x3, a);
          acc[ee * RT_TT + tt] = a;
        }
      }
    }
  }
  butterfly32(acc, lane);
  if (lane < 32) {
    const int ee = lane / RT_TT, tt = lane % RT_TT;
    const int e = e0 + ee, t = t0 + tt;
    if (e < E && tt < nt) {
      double l = acc[0];
      if (bias) l += (double)bias[e];
      logits[(size_t)t * E + e] = l;
    }
  }

  // ---- last block of this token tile: softmax + top-k ----
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = atomicAdd(&counters[blockIdx.y], 1u);
    s_last = (prev == gridDim.x - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  for (int tt = wave; tt < nt; tt += 4) {
    const int t = t0 + tt;
    const volatile double* lrow = logits + (size_t)t * E;
    double lv[4];
    double m = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      lv[i] = (e < E) ? lrow[e] : -INFINITY;
      m = fmax(m, lv[i]);
    }
    m = wave_max_d(m);
    double ps = 0.0;
    double pv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      pv[i] = (e < E) ? exp(lv[i] - m) : 0.0;
      ps += pv[i];
    }
    ps = wave_sum_d(ps);
    // top-k by (logit desc, index asc); lane r keeps the r-th choice
    bool taken[4] = {false, false, false, false};
    double my_g = 0.0;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
      double bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        if (e < E && !taken[i] && (lv[i] > bv || (lv[i] == bv && e < be))) { bv = lv[i]; be = e; }
      }
#pragma unroll
      for (int msk = 32; msk >= 1; msk >>= 1) {
        const double ov = __shfl_xor(bv, msk, WAVE);
        const int oe = __shfl_xor(be, msk, WAVE);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      // probability of the winner, broadcast from its owner lane
      double p = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (lane + 64 * i == be) {
          taken[i] = true;
          p = pv[i];
        }
      }
      p = wave_sum_d(p) / ps;
      if (lane == r) {
        my_g = p;
        my_i = be;
      }
    }
    const double gsum = wave_sum_d(lane < k ? my_g : 0.0);
    if (lane < k) {
      idx_out[(size_t)t * k + lane] = my_i;
      gate_out[(size_t)t * k + lane] = (float)(renorm ? my_g / gsum : my_g);
    }
  }
  if (threadIdx.x == 0) counters[blockIdx.y] = 0u;
}

}  // namespace

size_t route_workspace_bytes(int T, int E) {
  const size_t nt = (size_t)(T + RT_TT - 1) / RT_TT;
  const size_t logits = ((size_t)T * E * sizeof(double) + 255) & ~size_t(255);
  return logits + ((nt * sizeof(unsigned) + 255) & ~size_t(255));
}

hipError_t launch_route(const uint16_t* x, int T, int d, const float* W, int E, const float* bias, int k,
                        int renorm, int* idx, float* gate, void* ws, hipStream_t stream) {
  const size_t logits_bytes = ((size_t)T * E * sizeof(double) + 255) & ~size_t(255);
  double* logits = static_cast<double*>(ws);
  unsigned* counters = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + logits_bytes);
  dim3 grid((E + RT_ET - 1) / RT_ET, (T + RT_TT - 1) / RT_TT);
  hipLaunchKernelGGL(k_route, grid, dim3(256), 0, stream, x, T, d, W, E, bias, k, renorm, idx, gate, logits,
                     counters);
  return hipGetLastError();
}

}  // namespace moe
