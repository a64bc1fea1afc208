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
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int PM_NT = 1024;
constexpr int PM_SMALL_WORDS = 4096;  // key x token-word entries the one-block plan keeps in LDS
constexpr int PM_SMALL_PER_T = 8;     // pairs per thread of the one-block plan
constexpr int PM_COL_NT = 256;

// Exclusive scan of one int per thread over a block of PM_NT threads; returns
// the thread's exclusive prefix and writes the block total to *total.
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
  int* colerr;
  int* keycnt;
  int* slot_pair;
  int* pair_slot;
  int* slot_info;
  int4* chunks;
  int* chunk_cnt;
  int* meta;
  int* expert_off;
  int* expert_maxbits;
};

// Key e*B + (B - b) of pair i, or -1 for a dropped pair (err: bit 0 invalid
// expert or width, bit 1 repeated expert).
__device__ int pair_key(const FfnShape& s, const int* __restrict__ idx, const uint8_t* __restrict__ bits, int i,
                        int& err) {
  const int e = idx[i], b = bits[i];
  if (e < 0 || e >= s.E || b < 1 || b > s.B) {
    err |= 1;
    return -1;
  }
  for (int j = (i / s.k) * s.k; j < i; ++j) {
    const int bj = bits[j];
    if (idx[j] == e && bj >= 1 && bj <= s.B) {
      err |= 2;
      return -1;
    }
  }
  return e * s.B + (s.B - b);
}

// Flat exclusive scan of the popcounts of n LDS words (block of PM_NT
// threads, contiguous segment per thread).  pre[j] receives the prefix of
// word j; off[kk] the prefix at word kk*W (the first pairs of key kk) and
// off[n/W] the total.
__device__ void scan_words(const uint32_t* words, int* pre, int n, int W, int* off, int* wsum) {
  const int tid = threadIdx.x;
  const int seg = (n + PM_NT - 1) / PM_NT;
  const int j0 = min(n, tid * seg), j1 = min(n, j0 + seg);
  int v = 0;
  for (int j = j0; j < j1; ++j) v += __popc(words[j]);
  int total;
  int run = block_exclusive_scan(v, wsum, &total);
  for (int j = j0; j < j1; ++j) {
    pre[j] = run;
    if (j % W == 0) off[j / W] = run;
    run += __popc(words[j]);
  }
  if (tid == 0) off[n / W] = total;
}

// Expert offsets and widest widths, routed chunks, shared chunks and slots.
// off: LDS key offsets (NK + 1 entries).  Block of PM_NT threads.
__device__ void plan_chunks(const FfnShape& s, const PlanPtrs& pp, const int* off, int* wsum) {
  const int tid = threadIdx.x;
  const int B = s.B, E = s.E;
  for (int e = tid; e <= E; e += PM_NT) {
    pp.expert_off[e] = off[e * B];
    if (e < E) {
      int mb = 0;
      for (int L = B - 1; L >= 0; --L)
        if (off[e * B + L + 1] > off[e * B + L]) mb = B - L;
      pp.expert_maxbits[e] = mb;
    }
  }
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
        int mask = 0, cnt = 0;
        for (int L = 0; L < B; ++L) {
          const int lo = off[e * B + L], hi = off[e * B + L + 1];
          if (hi > lo && hi > s0 && lo < s0 + mm) mask |= 1 << (B - L - 1);  // bit (b-1) for width b
          // pairs of the chunk with width >= B - L
          cnt |= min(max(hi - s0, 0), mm) << (8 * (B - L - 1));
        }
        pp.chunks[cbase + c] = make_int4(e, s0, mm, mask);
        pp.chunk_cnt[cbase + c] = cnt;
      }
    }
    if (tid == 0) pp.meta[0] = total;
  }
  // shared experts: every token, full width
  const int ncs = (s.T + s.cs - 1) / s.cs;
  for (int i = tid; i < s.n_shared * ncs; i += PM_NT) {
    const int sh = i / ncs, c = i % ncs;
    const int mm = min(s.cs, s.T - s.cs * c);
    pp.chunks[s.max_rchunks + i] = make_int4(sh, s.P + sh * s.T + s.cs * c, mm, (1 << (B - 1)) | (1 << 16));
    int cnt = 0;
    for (int b = 1; b <= B; ++b) cnt |= mm << (8 * (b - 1));
    pp.chunk_cnt[s.max_rchunks + i] = cnt;
  }
  for (int i = tid; i < s.n_shared * s.T; i += PM_NT) pp.slot_info[s.P + i] = (i % s.T) | (B << 24);
}

__device__ __forceinline__ void put_slot(const FfnShape& s, const PlanPtrs& pp, int i, int kk, int slot) {
  pp.slot_pair[slot] = i;
  pp.pair_slot[i] = slot;
  pp.slot_info[slot] = (i / s.k) | ((s.B - kk % s.B) << 24);
}

// ---------------------------------------------------------------------------
// one block: NK * W <= PM_SMALL_WORDS and P <= PM_NT * PM_SMALL_PER_T

__global__ __launch_bounds__(PM_NT) void k_plan_small(FfnShape s, PlanPtrs pp, const int* __restrict__ idx,
                                                      const uint8_t* __restrict__ bits) {
  __shared__ uint32_t bm[PM_SMALL_WORDS];
  __shared__ int pre[PM_SMALL_WORDS];
  __shared__ int off[1025];
  __shared__ int wsum[PM_NT / WAVE];
  __shared__ short sexp[PM_NT * PM_SMALL_PER_T];  // expert of a valid pair, else -1
  __shared__ int errs;
  const int tid = threadIdx.x;
  const int W = s.W, P = s.P, NW = s.E * s.B * W;
  for (int j = tid; j < NW; j += PM_NT) bm[j] = 0u;
  if (tid == 0) errs = 0;
  int err = 0;
  int bw[PM_SMALL_PER_T];
#pragma unroll
  for (int r = 0; r < PM_SMALL_PER_T; ++r) {
    const int i = tid + r * PM_NT;
    bw[r] = 0;
    if (i < P) {
      const int e = idx[i], b = bits[i];
      const bool ok = e >= 0 && e < s.E && b >= 1 && b <= s.B;
      if (!ok) err |= 1;
      sexp[i] = (short)(ok ? e : -1);
      bw[r] = b;
    }
  }
  __syncthreads();

  // key of each pair; an earlier valid pair of the token with the same
  // expert drops it
  int keys[PM_SMALL_PER_T];
#pragma unroll
  for (int r = 0; r < PM_SMALL_PER_T; ++r) {
    const int i = tid + r * PM_NT;
    keys[r] = -1;
    if (i < P) {
      const int e = sexp[i];
      if (e >= 0) {
        bool dup = false;
        for (int j = (i / s.k) * s.k; j < i; ++j) dup |= sexp[j] == e;
        if (dup) {
          err |= 2;
        } else {
          keys[r] = e * s.B + (s.B - bw[r]);
          const int t = i / s.k;
          atomicOr(&bm[keys[r] * W + (t >> 5)], 1u << (t & 31));
        }
      }
    }
  }
  if (err) atomicOr(&errs, err);
  __syncthreads();

  scan_words(bm, pre, NW, W, off, wsum);
  __syncthreads();

  const int nvalid = off[s.E * s.B];
#pragma unroll
  for (int r = 0; r < PM_SMALL_PER_T; ++r) {
    const int i = tid + r * PM_NT;
    if (i >= P) continue;
    if (i >= nvalid) pp.slot_pair[i] = -1;
    const int kk = keys[r];
    if (kk < 0) {
      pp.pair_slot[i] = -1;
      continue;
    }
    const int t = i / s.k;
    const int wi = kk * W + (t >> 5);
    put_slot(s, pp, i, kk, pre[wi] + __popc(bm[wi] & ((1u << (t & 31)) - 1u)));
  }
  plan_chunks(s, pp, off, wsum);
  if (tid == 0) pp.meta[1] = errs;
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
  PlanPtrs pp;
  pp.pair_key = reinterpret_cast<int*>(ws + L.pair_key);
  pp.bitmap = reinterpret_cast<uint32_t*>(ws + L.bitmap);
  pp.prefix = reinterpret_cast<int*>(ws + L.prefix);
  pp.colerr = reinterpret_cast<int*>(ws + L.colerr);
  pp.keycnt = reinterpret_cast<int*>(ws + L.keycnt);
  pp.slot_pair = reinterpret_cast<int*>(ws + L.slot_pair);
  pp.pair_slot = reinterpret_cast<int*>(ws + L.pair_slot);
  pp.slot_info = reinterpret_cast<int*>(ws + L.slot_info);
  pp.chunks = reinterpret_cast<int4*>(ws + L.chunks);
  pp.chunk_cnt = reinterpret_cast<int*>(ws + L.chunk_cnt);
  pp.meta = reinterpret_cast<int*>(ws + L.meta);
  pp.expert_off = reinterpret_cast<int*>(ws + L.expert_off);
  pp.expert_maxbits = reinterpret_cast<int*>(ws + L.expert_maxbits);
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
