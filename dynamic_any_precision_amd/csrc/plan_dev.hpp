// Device code of the execution plan shared by the plan kernels and the fused
// decode control kernel: scans, chunk records, slots, and the one-block plan
// over a key x token-word array held in LDS (see permute.hip for the method).
#pragma once

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

// A pair of expert e at width b reads min(b, B_e) planes (B_e the expert's
// stored width; B for a uniform bank).
__device__ __forceinline__ int clamp_width(const FfnShape& s, int e, int b) {
  if (!s.bprefix) return b;
  const int be = s.bprefix[e + 1] - s.bprefix[e];
  return b < be ? b : be;
}

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
  return e * s.B + (s.B - clamp_width(s, e, b));
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
    if (total <= E) {
      // at most as many chunks as experts (decode): one thread per expert
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
    } else {
      // more chunks (large batches): the first chunk of every expert, then
      // the chunks spread over the threads, so that a heavily loaded expert's
      // chunks are not one thread's serial loop (the same records)
      __shared__ int scb[257];
      if (e < E) scb[e] = cbase;
      __syncthreads();
      for (int c = tid; c < total; c += PM_NT) {
        // the chunk's expert: the largest e with scb[e] <= c
        int lo = 0, hi = E - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (scb[mid] <= c) lo = mid; else hi = mid - 1;
        }
        const int ce = lo, cc = c - scb[ce];
        const int me = off[(ce + 1) * B] - off[ce * B];
        const int s0 = off[ce * B] + s.cs * cc;
        const int mm = min(s.cs, me - s.cs * cc);
        int mask = 0, cnt = 0;
        for (int L = 0; L < B; ++L) {
          const int lo2 = off[ce * B + L], hi2 = off[ce * B + L + 1];
          if (hi2 > lo2 && hi2 > s0 && lo2 < s0 + mm) mask |= 1 << (B - L - 1);
          cnt |= min(max(hi2 - s0, 0), mm) << (8 * (B - L - 1));
        }
        pp.chunks[c] = make_int4(ce, s0, mm, mask);
        pp.chunk_cnt[c] = cnt;
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


// LDS of the one-block plan.  The caller fills sexp (expert of a valid pair,
// else -1) and sbits (its width) for every pair.
struct alignas(16) PlanSmallLds {
  uint32_t bm[PM_SMALL_WORDS];
  int pre[PM_SMALL_WORDS];
  int off[1025];
  int wsum[PM_NT / WAVE];
  short sexp[PM_NT * PM_SMALL_PER_T];
  uint8_t sbits[PM_NT * PM_SMALL_PER_T];
  int errs;
};

// Clears the word array and the error flags (before the caller's barrier).
__device__ __forceinline__ void plan_small_clear(const FfnShape& s, PlanSmallLds& L) {
  const int NW = s.E * s.B * s.W;
  for (int j = threadIdx.x; j < NW; j += PM_NT) L.bm[j] = 0u;
  if (threadIdx.x == 0) L.errs = 0;
}

// The plan of NK * W <= PM_SMALL_WORDS entries and P <= PM_NT * PM_SMALL_PER_T
// pairs by one block of PM_NT threads, from sexp / sbits in LDS (filled and
// followed by a barrier).  err: the calling thread's error bits so far.
__device__ void plan_small_core(const FfnShape& s, const PlanPtrs& pp, PlanSmallLds& L, int err) {
  const int tid = threadIdx.x;
  const int W = s.W, P = s.P, NW = s.E * s.B * W;
  // key of each pair; an earlier valid pair of the token with the same
  // expert drops it
  int keys[PM_SMALL_PER_T];
#pragma unroll
  for (int r = 0; r < PM_SMALL_PER_T; ++r) {
    const int i = tid + r * PM_NT;
    keys[r] = -1;
    if (i < P) {
      const int e = L.sexp[i];
      if (e >= 0) {
        bool dup = false;
        for (int j = (i / s.k) * s.k; j < i; ++j) dup |= L.sexp[j] == e;
        if (dup) {
          err |= 2;
        } else {
          keys[r] = e * s.B + (s.B - clamp_width(s, e, L.sbits[i]));
          const int t = i / s.k;
          atomicOr(&L.bm[keys[r] * W + (t >> 5)], 1u << (t & 31));
        }
      }
    }
  }
  if (err) atomicOr(&L.errs, err);
  __syncthreads();

  scan_words(L.bm, L.pre, NW, W, L.off, L.wsum);
  __syncthreads();

  const int nvalid = L.off[s.E * s.B];
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
    put_slot(s, pp, i, kk, L.pre[wi] + __popc(L.bm[wi] & ((1u << (t & 31)) - 1u)));
  }
  plan_chunks(s, pp, L.off, L.wsum);
  if (tid == 0) pp.meta[1] = L.errs;
}

PlanPtrs plan_ptrs(const FfnLayout& Lo, char* ws) {
  PlanPtrs pp;
  pp.pair_key = reinterpret_cast<int*>(ws + Lo.pair_key);
  pp.bitmap = reinterpret_cast<uint32_t*>(ws + Lo.bitmap);
  pp.prefix = reinterpret_cast<int*>(ws + Lo.prefix);
  pp.colerr = reinterpret_cast<int*>(ws + Lo.colerr);
  pp.keycnt = reinterpret_cast<int*>(ws + Lo.keycnt);
  pp.slot_pair = reinterpret_cast<int*>(ws + Lo.slot_pair);
  pp.pair_slot = reinterpret_cast<int*>(ws + Lo.pair_slot);
  pp.slot_info = reinterpret_cast<int*>(ws + Lo.slot_info);
  pp.chunks = reinterpret_cast<int4*>(ws + Lo.chunks);
  pp.chunk_cnt = reinterpret_cast<int*>(ws + Lo.chunk_cnt);
  pp.meta = reinterpret_cast<int*>(ws + Lo.meta);
  pp.expert_off = reinterpret_cast<int*>(ws + Lo.expert_off);
  pp.expert_maxbits = reinterpret_cast<int*>(ws + Lo.expert_maxbits);
  return pp;
}

}  // namespace
}  // namespace moe
