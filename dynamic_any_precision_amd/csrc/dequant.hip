// Floor-and-compensation dequantisation of one stored matrix (MatMoE review,
// Core Contribution, F&C paragraph), and the bf16 layer input of a residual
// stream (plain cast, or RMS-normalised rows).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// out[n][c] = fp32(((q >> delta) << delta) + (2^delta - 1)/2 - z) * s, one rounding:
// the bracket is exact in fp32 (a multiple of 1/2 below 16 in size).
__global__ __launch_bounds__(256) void k_dequant(const uint32_t* __restrict__ planes, const float* __restrict__ sz,
                                                 int N, int K, int B, int g, int expert, int bits,
                                                 const int* __restrict__ bprefix, float* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)N * K) return;
  const int n = (int)(idx / K), c = (int)(idx % K);
  const size_t plane_words = (size_t)N * K / 32;
  const int tile = n >> 4, r = n & 15;
  const int kb = c >> 7, j = (c >> 5) & 3, bit = c & 31;
  const size_t word = (size_t)tile * (K / 2) + 64 * kb + 16 * j + r;
  // a ragged bank: the expert's own first plane and width, read at most that wide
  size_t first = (size_t)expert * B;
  if (bprefix) {
    first = (size_t)bprefix[expert];
    B = bprefix[expert + 1] - bprefix[expert];
    bits = bits < B ? bits : B;
  }
  const uint32_t* base = planes + first * plane_words;
  uint32_t q = 0;
  for (int p = 0; p < bits; ++p) q = (q << 1) | ((base[p * plane_words + word] >> bit) & 1u);
  const int delta = B - bits;
  const float code = (float)(q << delta);
  const float comp = 0.5f * (float)((1 << delta) - 1);
  const int NQG = K / g;
  const float* s = sz + (((size_t)expert * (N >> 4) + tile) * NQG + c / g) * 32;
  const float scale = s[r], zero = s[16 + r];
  const float tval = __fadd_rn(__fadd_rn(code, comp), -zero);
  out[idx] = __fmul_rn(tval, scale);
}

__global__ __launch_bounds__(256) void k_residual_to_bf16(const float* __restrict__ h, uint16_t* __restrict__ x,
                                                          int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] = (uint16_t)f32_to_bf16(h[i]);
}

// One block per row of d values: r = fp32(1 / sqrt(sum(h^2) / d + eps)) with
// the squares and their sum in fp64 (each square exact; the sum's order
// moves only its last fp64 bits), then x = bf16_rne(fp32(h * r)).
__global__ __launch_bounds__(256) void k_rmsnorm_to_bf16(const float* __restrict__ h, uint16_t* __restrict__ x,
                                                         int d, float eps) {
  __shared__ double part[4];
  const float* hr = h + (size_t)blockIdx.x * d;
  uint16_t* xr = x + (size_t)blockIdx.x * d;
  double ss = 0.0;
  for (int i = threadIdx.x; i < d; i += 256) {
    const double v = (double)hr[i];
    ss = fma(v, v, ss);
  }
  ss = wave_sum_d(ss);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float r = (float)(1.0 / sqrt(tot / (double)d + (double)eps));
  for (int i = threadIdx.x; i < d; i += 256) xr[i] = (uint16_t)f32_to_bf16(__fmul_rn(hr[i], r));
}

// Streaming read: blocks of 256 threads, 8 loads of 16 B in flight per thread
// per round, grid-stride.  One XOR-folded word per wave goes to sink.
constexpr int SR_UNROLL = 8;

__global__ __launch_bounds__(256) void k_stream_read(const uint4* __restrict__ p, int64_t n16,
                                                     uint32_t* __restrict__ sink) {
  uint32_t acc = 0u;
  const int64_t step = (int64_t)gridDim.x * 256 * SR_UNROLL;
  for (int64_t base = (int64_t)blockIdx.x * 256 * SR_UNROLL + threadIdx.x; base < n16; base += step) {
    uint4 v[SR_UNROLL];
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n16 ? p[i] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < SR_UNROLL; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m, WAVE);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int sink_len, hipStream_t stream) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  int64_t blocks = (n16 + 256 * SR_UNROLL - 1) / (256 * SR_UNROLL);
  if (blocks > sink_len / 4) blocks = sink_len / 4;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const uint4*>(buf), n16,
                     sink);
  return hipGetLastError();
}

hipError_t launch_dequant(MatrixDev m, int B, int g, int expert, int bits, const int* bprefix, float* out,
                          hipStream_t stream) {
  const size_t total = (size_t)m.N * m.K;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  hipLaunchKernelGGL(k_dequant, dim3(blocks), dim3(256), 0, stream, m.planes, m.sz, m.N, m.K, B, g, expert, bits,
                     bprefix, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_to_bf16(const float* h, uint16_t* x, int rows, int d, float eps, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rmsnorm_to_bf16, dim3(rows), dim3(256), 0, stream, h, x, d, eps);
  return hipGetLastError();
}

hipError_t launch_residual_to_bf16(const float* h, uint16_t* x, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n + 255) / 256);
  hipLaunchKernelGGL(k_residual_to_bf16, dim3(blocks), dim3(256), 0, stream, h, x, n);
  return hipGetLastError();
}

}  // namespace moe
