// Token-to-expert permutation and histogram.
//
// Builds the execution plan of the FFN:
//   - a stable order of pairs by (expert asc, bits desc, pair id asc).  Pairs
//     are keyed by (expert, 4 - bits).  Each expert appears at most once per
//     token, so the rank of a pair among the pairs of its key is the number
//     of earlier tokens carrying that key: one bit per (key, token) in
//     32-token words, then one exclusive scan of the word popcounts over the
//     key-major word array gives, at word (key, w), the pairs of all smaller
//     keys plus those of this key in earlier words.  The order is
//     deterministic;
//   - per-expert offsets and widest width, "reads the maximum bits any token
//     of an expert needs";
//   - chunks of at most 16 (64 for prefill-sized batches) consecutive pairs
//     of one expert, each with the set of bit-widths it holds (the planes it
//     streams are those of its widest pair) and the number of its pairs of
//     width >= b for b = 1..4 (pairs are sorted by width, so these counts give
//     every pair's width);
//   - chunks for the always-on shared experts.
// A pair is dropped (never indexed) when its expert index is out of range,
// its width is outside [1, b_max], or an earlier pair of its token already
// holds the same expert with a valid width.
//
// Small batches: one block of 1024 threads with the word array in LDS.
// Large batches: three launches over the chip: the words of one 32-token
// column per block; one wave per key for the scan along its row (and the
// key's pair count); slots per block of 1024 pairs, each block scanning the
// key counts itself (block 0 also writes the chunks).
#include "plan_dev.hpp"

namespace moe {

namespace {

// ---------------------------------------------------------------------------
// one block: NK * W <= PM_SMALL_WORDS and P <= PM_NT * PM_SMALL_PER_T

__global__ __launch_bounds__(PM_NT) void k_plan_small(FfnShape s, PlanPtrs pp, const int* __restrict__ idx,
                                                      const uint8_t* __restrict__ bits) {
  __shared__ PlanSmallLds L;
  const int tid = threadIdx.x;
  plan_small_clear(s, L);
  int err = 0;
  for (int i = tid; i < s.P; i += PM_NT) {
    const int e = idx[i], b = bits[i];
    const bool ok = e >= 0 && e < s.E && b >= 1 && b <= s.B;
    if (!ok) err |= 1;
    L.sexp[i] = (short)(ok ? e : -1);
    L.sbits[i] = (uint8_t)b;
  }
  __syncthreads();
  plan_small_core(s, pp, L, err);
}

// ---------------------------------------------------------------------------
// large batches

// One block per 32-token word w: the word of every key, pair keys, error bits.
__global__ __launch_bounds__(PM_COL_NT) void k_plan_cols(FfnShape s, PlanPtrs pp, const int* __restrict__ idx,
                                                         const uint8_t* __restrict__ bits) {
  __shared__ uint32_t colw[1024];
  __shared__ int errs;
  const int w = blockIdx.x, tid = threadIdx.x;
  const int NK = s.E * s.B;
  for (int j = tid; j < NK; j += PM_COL_NT) colw[j] = 0u;
  if (tid == 0) errs = 0;
  __syncthreads();
  const int p0 = 32 * w * s.k, p1 = min(s.P, 32 * (w + 1) * s.k);
  int err = 0;
  for (int i = p0 + tid; i < p1; i += PM_COL_NT) {
    const int kk = pair_key(s, idx, bits, i, err);
    if (kk >= 0) atomicOr(&colw[kk], 1u << ((i / s.k) & 31));
    pp.pair_key[i] = kk;
  }
  if (err) atomicOr(&errs, err);
  __syncthreads();
  for (int j = tid; j < NK; j += PM_COL_NT) pp.bitmap[(size_t)j * s.W + w] = colw[j];
  if (tid == 0) pp.colerr[w] = errs;
}

// One wave per key: exclusive scan of the popcounts along the key's row of
// words (prefix within the key) and the key's pair count.
__global__ __launch_bounds__(256) void k_plan_keys(FfnShape s, PlanPtrs pp) {
  const int kk = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (kk >= s.E * s.B) return;
  const uint32_t* row = pp.bitmap + (size_t)kk * s.W;
  int* prow = pp.prefix + (size_t)kk * s.W;
  int run = 0;
  for (int w0 = 0; w0 < s.W; w0 += 64) {
    const int w = w0 + lane;
    const int v = w < s.W ? __popc(row[w]) : 0;
    int incl = v;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m, WAVE);
      if (lane >= m) incl += o;
    }
    if (w < s.W) prow[w] = run + incl - v;
    run += __shfl(incl, 63, WAVE);
  }
  if (lane == 0) pp.keycnt[kk] = run;
}

// Blocks of PM_NT pairs: key offsets from the key counts (every block), the
// slot of every pair; block 0 also the expert summaries, chunks and errors.
__global__ __launch_bounds__(PM_NT) void k_plan_slots(FfnShape s, PlanPtrs pp) {
  __shared__ int off[1025];
  __shared__ int wsum[PM_NT / WAVE];
  __shared__ int errs;
  const int tid = threadIdx.x;
  const int NK = s.E * s.B;
  {
    const int v = tid < NK ? pp.keycnt[tid] : 0;
    int total;
    const int ex = block_exclusive_scan(v, wsum, &total);
    if (tid < NK) off[tid] = ex;
    if (tid == 0) off[NK] = total;
  }
  __syncthreads();
  const int i = blockIdx.x * PM_NT + tid;
  if (i < s.P) {
    if (i >= off[NK]) pp.slot_pair[i] = -1;
    const int kk = pp.pair_key[i];
    if (kk < 0) {
      pp.pair_slot[i] = -1;
    } else {
      const int t = i / s.k;
      const size_t wi = (size_t)kk * s.W + (t >> 5);
      put_slot(s, pp, i, kk, off[kk] + pp.prefix[wi] + __popc(pp.bitmap[wi] & ((1u << (t & 31)) - 1u)));
    }
  }
  if (blockIdx.x != 0) return;
  if (tid == 0) errs = 0;
  __syncthreads();
  int err = 0;
  for (int w = tid; w < s.W; w += PM_NT) err |= pp.colerr[w];
  if (err) atomicOr(&errs, err);
  plan_chunks(s, pp, off, wsum);
  if (tid == 0) pp.meta[1] = errs;
}

}  // namespace

hipError_t launch_plan(const FfnShape& s, const FfnLayout& L, char* ws, const int* idx, const uint8_t* bits,
                       hipStream_t stream) {
  const PlanPtrs pp = plan_ptrs(L, ws);
  if ((long)s.E * s.B * s.W <= PM_SMALL_WORDS && s.P <= PM_NT * PM_SMALL_PER_T) {
    hipLaunchKernelGGL(k_plan_small, dim3(1), dim3(PM_NT), 0, stream, s, pp, idx, bits);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_plan_cols, dim3(s.W), dim3(PM_COL_NT), 0, stream, s, pp, idx, bits);
  hipLaunchKernelGGL(k_plan_keys, dim3((s.E * s.B + 3) / 4), dim3(256), 0, stream, s, pp);
  hipLaunchKernelGGL(k_plan_slots, dim3((s.P + PM_NT - 1) / PM_NT), dim3(PM_NT), 0, stream, s, pp);
  return hipGetLastError();
}

}  // namespace moe
