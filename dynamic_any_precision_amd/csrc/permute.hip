// Token-to-expert permutation and histogram.
//
// One block of 1024 threads builds the execution plan of the FFN:
//   - a histogram of pairs per key (expert, 4 - bits) and its exclusive scan;
//   - a stable order of pairs by (expert asc, bits desc, pair id asc).  Each
//     expert appears at most once per token, so the rank of a pair among the
//     pairs of its key is the number of earlier tokens carrying that key:
//     one bit per (key, token) set with atomicOr, then per-key prefix
//     popcounts.  The order is deterministic;
//   - chunks of at most 16 (64 for prefill-sized batches) consecutive pairs
//     of one expert, each with the set
//     of bit-widths it holds (the planes it must stream are those of its
//     widest pair, "reads the maximum bits any token of an expert needs");
//   - chunks for the always-on shared experts.
// Pairs with an expert index out of range, a width outside [1, b_max] or a
// repeated expert within one token are dropped (never indexed).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int PM_NT = 1024;

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Exclusive scan of one int per thread over the block; returns the thread's
// exclusive prefix and writes the block total to *total.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int o = __shfl_up(incl, m, WAVE);
    if (lane >= m) incl += o;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < PM_NT / WAVE; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  *total = tot;
  return base + incl - v;
}

struct PlanPtrs {
  int* pair_key;
  uint32_t* bitmap;
  int* prefix;
  int* slot_pair;
  int* pair_slot;
  int* slot_info;
  int4* chunks;
  int* meta;
  int* expert_off;
  int* expert_maxbits;
};

__device__ void permute_body(const FfnShape& s, const PlanPtrs& pp, const int* __restrict__ idx,
                             const uint8_t* __restrict__ bits) {
  __shared__ int cnt[1024];
  __shared__ int off[1025];
  __shared__ int wsum[PM_NT / WAVE];
  const int tid = threadIdx.x;
  const int B = s.B, E = s.E, k = s.k, P = s.P, W = s.W;
  const int NK = E * B;

  // phase 0: clear
  for (int i = tid; i < NK; i += PM_NT) cnt[i] = 0;
  for (int i = tid; i < NK * W; i += PM_NT) pp.bitmap[i] = 0u;
  for (int i = tid; i < P; i += PM_NT) pp.slot_pair[i] = -1;
  if (tid < 16) pp.meta[tid] = 0;
  __syncthreads();

  // phase 1: histogram and token bitmaps
  int err = 0;
  for (int i = tid; i < P; i += PM_NT) {
    const int t = i / k;
    const int e = idx[i];
    const int b = bits[i];
    int key = -1;
    if (e >= 0 && e < E && b >= 1 && b <= B) {
      const int kk = e * B + (B - b);
      const uint32_t bit = 1u << (t & 31);
      const uint32_t old = atomicOr(&pp.bitmap[(size_t)kk * W + (t >> 5)], bit);
      if (!(old & bit)) {
        atomicAdd(&cnt[kk], 1);
        key = kk;
      } else {
        err |= 2;
      }
    } else {
      err |= 1;
    }
    pp.pair_key[i] = key;
  }
  if (err) atomicOr(&pp.meta[1], err);
  __syncthreads();

  // phase 2: scan over keys, per-key bitmap prefixes, expert summaries
  {
    const int v = tid < NK ? cnt[tid] : 0;
    int total;
    const int ex = block_exclusive_scan(v, wsum, &total);
    if (tid < NK) off[tid] = ex;
    if (tid == 0) off[NK] = total;
  }
  for (int kk = tid; kk < NK; kk += PM_NT) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      pp.prefix[(size_t)kk * W + w] = run;
      run += __popc(load_coherent(&pp.bitmap[(size_t)kk * W + w]));
    }
  }
  __syncthreads();
  for (int e = tid; e <= E; e += PM_NT) {
    pp.expert_off[e] = off[e * B];
    if (e < E) {
      int mb = 0;
      for (int L = B - 1; L >= 0; --L)
        if (cnt[e * B + L] > 0) mb = B - L;
      pp.expert_maxbits[e] = mb;
    }
  }

  // phase 3: stable slots
  for (int i = tid; i < P; i += PM_NT) {
    const int kk = pp.pair_key[i];
    if (kk < 0) {
      pp.pair_slot[i] = -1;
      continue;
    }
    const int t = i / k;
    const size_t wi = (size_t)kk * W + (t >> 5);
    const uint32_t below = load_coherent(&pp.bitmap[wi]) & ((1u << (t & 31)) - 1u);
    const int slot = off[kk] + pp.prefix[wi] + __popc(below);
    const int b = B - (kk % B);
    pp.slot_pair[slot] = i;
    pp.pair_slot[i] = slot;
    pp.slot_info[slot] = t | (b << 24);
  }

  // phase 4: routed chunks
  {
    const int e = tid;
    int m = 0, nch = 0;
    if (e < E) {
      m = off[(e + 1) * B] - off[e * B];
      nch = (m + s.cs - 1) / s.cs;
    }
    int total;
    const int cbase = block_exclusive_scan(nch, wsum, &total);
    if (e < E) {
      for (int c = 0; c < nch; ++c) {
        const int s0 = off[e * B] + s.cs * c;
        const int mm = min(s.cs, m - s.cs * c);
        int mask = 0;
        for (int L = 0; L < B; ++L) {
          const int lo = off[e * B + L], hi = off[e * B + L + 1];
          if (hi > lo && hi > s0 && lo < s0 + mm) mask |= 1 << (B - L - 1);  // bit (b-1) for width b
        }
        pp.chunks[cbase + c] = make_int4(e, s0, mm, mask);
      }
    }
    if (tid == 0) pp.meta[0] = total;
  }

  // shared experts: every token, full width
  const int ncs = (s.T + s.cs - 1) / s.cs;
  for (int i = tid; i < s.n_shared * ncs; i += PM_NT) {
    const int sh = i / ncs, c = i % ncs;
    pp.chunks[s.max_rchunks + i] =
        make_int4(sh, P + sh * s.T + s.cs * c, min(s.cs, s.T - s.cs * c), (1 << (B - 1)) | (1 << 16));
  }
  for (int i = tid; i < s.n_shared * s.T; i += PM_NT) pp.slot_info[P + i] = (i % s.T) | (B << 24);
}

__global__ __launch_bounds__(PM_NT) void k_plan(FfnShape s, PlanPtrs pp, const int* __restrict__ idx,
                                                const uint8_t* __restrict__ bits) {
  permute_body(s, pp, idx, bits);
}

}  // namespace

hipError_t launch_plan(const FfnShape& s, const FfnLayout& L, char* ws, const int* idx, const uint8_t* bits,
                       hipStream_t stream) {
  PlanPtrs pp;
  pp.pair_key = reinterpret_cast<int*>(ws + L.pair_key);
  pp.bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  pp.prefix = reinterpret_cast<int*>(ws + L.prefix);
  pp.slot_pair = reinterpret_cast<int*>(ws + L.slot_pair);
  pp.pair_slot = reinterpret_cast<int*>(ws + L.pair_slot);
  pp.slot_info = reinterpret_cast<int*>(ws + L.slot_info);
  pp.chunks = reinterpret_cast<int4*>(ws + L.chunks);
  pp.meta = reinterpret_cast<int*>(ws + L.meta);
  pp.expert_off = reinterpret_cast<int*>(ws + L.expert_off);
  pp.expert_maxbits = reinterpret_cast<int*>(ws + L.expert_maxbits);
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(PM_NT), 0, stream, s, pp, idx, bits);
  return hipGetLastError();
}

}  // namespace moe
