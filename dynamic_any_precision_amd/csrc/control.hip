// Fused decode control: softmax + top-k of every token, the bit allocation and
// the execution plan in one block, for batches of at most 1024 pairs whose
// plan fits the one-block plan.  Same results as the three separate steps
// (route_dev.hpp, alloc.hip, plan_dev.hpp); it saves launches and round trips
// through memory between them.  With more tokens than the block has waves
// the top-k runs as its own kernel (one wave per token across the chip) and
// this kernel takes its output: allocation and plan only.  Here the top-k
// ranks every (token, expert) candidate across the block instead of k
// arg-max rounds per token.
//
// Allocation: the threshold tau of the bisection (the smallest key whose
// strict upper set holds at most n* pairs; MatMoE abstract item (3) and
// review, Core Contribution: binary search for the threshold that meets the
// target average), found here by a radix descent over the P keys in LDS,
// four passes of 8-bit digits instead of 32 one-bit steps.
#include "common.hpp"
#include "kernels.hpp"
#include "plan_dev.hpp"
#include "route_dev.hpp"

namespace moe {

namespace {

constexpr int CTL_MAX_PAIRS = PM_NT;
constexpr int CTL_TOPK_TOKENS = PM_NT / WAVE;  // tokens up to which the top-k runs here

__device__ __forceinline__ uint32_t gate_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <bool TOPK>
__global__ __launch_bounds__(PM_NT) void k_control(FfnShape s, PlanPtrs pp, const double* __restrict__ logits,
                                                   int renorm, int n_star, int b_lo, int b_max,
                                                   int* __restrict__ idx_out, float* __restrict__ gate_out,
                                                   uint8_t* __restrict__ bits_out) {
  __shared__ PlanSmallLds L;
  // gate keys live in the plan's prefix array until the plan's scan
  uint32_t* skey = reinterpret_cast<uint32_t*>(L.pre);
  static_assert(CTL_MAX_PAIRS <= PM_SMALL_WORDS, "gate keys fit the prefix array");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  plan_small_clear(s, L);

  if (!TOPK) {
    // top-k done: take its experts and gates
    for (int i = tid; i < s.P; i += PM_NT) {
      L.sexp[i] = (short)idx_out[i];
      skey[i] = gate_key(gate_out[i]);
    }
  }
  if (TOPK) {
    // Top-k by ranks over the whole block: the rank of candidate (t, e) is
    // the number of the token's experts that beat it (larger logit, then
    // smaller index), so rank r is round r of the one-wave arg-max.  Then
    // one wave per token forms the softmax exactly as the top-k kernel does.
    __shared__ uint64_t ckey[CTL_TOPK_TOKENS * 256];
    __shared__ double wl[CTL_TOPK_TOKENS * 8];
    __shared__ int we[CTL_TOPK_TOKENS * 8];
    const int TE = s.T * s.E;
    for (int c = tid; c < TE; c += PM_NT) ckey[c] = order_key64(logits[c]);
    __syncthreads();
    for (int c = tid; c < TE; c += PM_NT) {
      const int t = c / s.E, e = c - t * s.E;
      const uint64_t kv = ckey[c];
      const uint64_t* kt = ckey + t * s.E;
      int rank = 0;
      for (int j = 0; j < s.E; ++j) {
        const uint64_t kj = kt[j];
        rank += (kj > kv || (kj == kv && j < e)) ? 1 : 0;
      }
      if (rank < s.k) {
        we[t * 8 + rank] = e;
        wl[t * 8 + rank] = key_to_double(kv);
      }
    }
    __syncthreads();
    for (int t = wave; t < s.T; t += PM_NT / WAVE) {
      const uint64_t* kt = ckey + t * s.E;
      const double mx = wl[t * 8];
      double ps = 0.0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < s.E) ps += exp(key_to_double(kt[lane + 64 * i]) - mx);
      ps = wave_sum_d(ps);
      const double p = lane < s.k ? exp(wl[t * 8 + (lane < s.k ? lane : 0)] - mx) / ps : 0.0;
      double psel = 0.0;
      if (renorm) {
        const long long pb = __double_as_longlong(p);
        for (int r = 0; r < s.k; ++r) {
          const int lo = __builtin_amdgcn_readlane((int)(uint32_t)pb, r);
          const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), r);
          psel += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
        }
      }
      if (lane < s.k) {
        const int base = t * s.k, e = we[t * 8 + lane];
        const float g = (float)(renorm ? p / psel : p);
        idx_out[base + lane] = e;
        gate_out[base + lane] = g;
        L.sexp[base + lane] = (short)e;
        skey[base + lane] = gate_key(g);
      }
    }
  }
  __syncthreads();

  // Allocation (a block-uniform choice between two exact methods).
  if (s.P <= PM_NT / 4) {
    // Up to 256 pairs: high width iff #{keys >= own key} <= n*, counted by
    // four adjacent threads per pair over the key blocks; the keys past P (up
    // to a multiple of 8) read as 0, below every gate key.
    for (int j = s.P + tid; j < ((s.P + 7) & ~7); j += PM_NT) skey[j] = 0u;
    __syncthreads();
    {
      constexpr int tpp = 4;  // threads per pair
      const int i = tid / tpp, part = tid % tpp;
      const int nblk = (s.P + 7) / 8;
      int ge = 0;
      if (i < s.P) {
        const uint32_t v = skey[i];
        const uint4* k4 = reinterpret_cast<const uint4*>(skey);
        for (int j = part * nblk / tpp; j < (part + 1) * nblk / tpp; ++j) {
          const uint4 a = k4[2 * j], b = k4[2 * j + 1];
          ge += (a.x >= v) + (a.y >= v) + (a.z >= v) + (a.w >= v) + (b.x >= v) + (b.y >= v) + (b.z >= v) + (b.w >= v);
        }
      }
      ge += __shfl_xor(ge, 1, WAVE);
      ge += __shfl_xor(ge, 2, WAVE);
      if (i < s.P && part == 0) {
        const int b = ge <= n_star ? b_max : b_lo;
        bits_out[i] = (uint8_t)b;
        L.sbits[i] = (uint8_t)b;
      }
    }
    __syncthreads();
  } else {
    // More pairs: tau = the smallest key whose strict upper set holds at most
    // n* pairs (the allocation kernel's bisection), found by a radix descent
    // over 8-bit digits from the most significant: in each pass the digit is
    // the smallest d for which the keys above the prefix plus the keys of the
    // prefix's block with a digit above d number at most n* (a histogram of
    // the block's digits and its suffix sums).  A pair is high iff its key
    // exceeds tau.
    {
      __shared__ int hist[256];
      __shared__ uint32_t s_prefix;
      __shared__ int s_above;
      const uint32_t myk = tid < s.P ? skey[tid] : 0u;
      uint32_t prefix = 0u;
      int above = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
        if (tid < s.P && (myk & hmask) == prefix) atomicAdd(&hist[(myk >> shift) & 255u], 1);
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
          // S(d): pairs of the block with a digit above d
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
      }
      if (tid < s.P) {
        const int b = myk > prefix ? b_max : b_lo;
        bits_out[tid] = (uint8_t)b;
        L.sbits[tid] = (uint8_t)b;
      }
    }
    __syncthreads();
  }

  // top-k never repeats an expert and allocation widths lie in [b_lo, b_max]
  plan_small_core(s, pp, L, 0);
}


// One token (T = 1).  Every routed expert then holds at most one pair, so each
// valid pair is a chunk of its own and its slot is its rank in the (expert,
// width) key order of the general plan, and every chunk reads the same token
// row: the token's activation fragment is written once, as chunk 0's, and the
// streaming kernels are told to read it for every chunk.  One block:
//   1. waves 1-3: the fragment (the gather's arithmetic, four k-blocks per wave
//      and pass), while
//   2. wave 0: with logits, the top-k (the top-k kernel's arithmetic) and the
//      allocation of the k pairs (high width iff #{keys >= own key} <= n*, as
//      in the fused control kernel); without, the given experts and widths;
//      then the dropping rules, slots and chunk records of the general plan;
//   3. all threads: expert offsets and widest widths.
constexpr int ONE_NT = 256;

__global__ __launch_bounds__(ONE_NT) void k_one(FfnShape s, PlanPtrs pp, const uint16_t* __restrict__ x,
                                                uint16_t* __restrict__ xg, float2* __restrict__ xvg,
                                                const double* __restrict__ logits, int renorm, int n_star, int b_lo,
                                                int b_max, int* __restrict__ idx, float* __restrict__ gate,
                                                uint8_t* __restrict__ bits) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint4 fr[3][4][16];  // per fragment wave and k-block of a pass: the token row's 16 operand uint4
  __shared__ int s_e[8], s_w[8];       // per pair: expert (-1: dropped) and width
  const int nkb = s.d / 128, tpg = s.g >> 3;

  // 1. activation fragment of the token, chunk 0's place, by waves 1-3 (four
  // k-blocks per wave and pass) while wave 0 routes
  if (wave > 0) {
    const int kbl = lane >> 4, q = lane & 15;
    uint4 (&fw)[4][16] = fr[wave - 1];
    for (int kb0 = 4 * (wave - 1); kb0 < nkb; kb0 += 12) {
      const int kb = kb0 + kbl;
      const bool on = kb < nkb;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (on) v = *reinterpret_cast<const uint4*>(x + kb * 128 + 8 * q);
      const uint32_t in[4] = {v.x, v.y, v.z, v.w};
      float X = 0.f, V = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = 8 * q + j;
        const int cc = col & 31;
        const float xf = bf16_to_f32((j & 1) ? (in[j >> 1] >> 16) : (in[j >> 1] & 0xFFFFu));
        const float sc = 1.0f / (float)(1 << (2 * a_exp(cc & 15)));
        X += xf;
        V += xf * sc;
        const int fp = frag_pos(cc);
        reinterpret_cast<uint16_t*>(fw[kbl])[((fp >> 3) * 4 + (col >> 5)) * 8 + (fp & 7)] =
            (uint16_t)f32_to_bf16(xf * sc);
      }
      for (int msk = 1; msk < tpg; msk <<= 1) {
        X += __shfl_xor(X, msk, WAVE);
        V += __shfl_xor(V, msk, WAVE);
      }
      if (on && (q & (tpg - 1)) == 0) xvg[(size_t)(kb * (128 / s.g) + q / tpg) * 16] = make_float2(X, V);
      // the wave's own LDS writes, then its reads of them (wave-level order)
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (on) {
        const int i = q >> 2, jg = q & 3;
        reinterpret_cast<uint4*>(xg)[(size_t)kb * 256 + i * 64 + act_pos(0, 0, jg)] = fw[kbl][q];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }

  // 2. routing, widths and the plan of the k pairs (lane j: pair j)
  if (wave == 0) {
    const int k = s.k, B = s.B;
    int e = -1, b = 0;
    if (logits) {
      float g = 0.f;
      topk_token(logits, s.E, k, renorm, [&](int j, int ex, float gv) {
        idx[j] = ex;
        gate[j] = gv;
        e = ex;
        g = gv;
      }, lane);
      const uint32_t key = lane < k ? gate_key(g) : 0u;
      int ge = 0;
      for (int r = 0; r < k; ++r) ge += ((uint32_t)__builtin_amdgcn_readlane((int)key, r) >= key) ? 1 : 0;
      b = ge <= n_star ? b_max : b_lo;
      if (lane < k) bits[lane] = (uint8_t)b;
    } else if (lane < k) {
      e = idx[lane];
      b = bits[lane];
    }
    // dropped: an expert or width out of range, or an expert an earlier pair
    // of the token (with a width in range) already has
    int err = 0;
    bool valid = lane < k;
    if (valid && (e < 0 || e >= s.E || b < 1 || b > B)) {
      err |= 1;
      valid = false;
    }
    for (int j = 0; j < k; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j), bj = __builtin_amdgcn_readlane(b, j);
      if (valid && j < lane && ej == e && bj >= 1 && bj <= B) {
        err |= 2;
        valid = false;
      }
    }
    const int w = valid ? clamp_width(s, e, b) : 0;
    const int key = valid ? e * B + (B - w) : 0x7FFFFFFF;
    int slot = 0, nvalid = 0, errs = 0;
    for (int j = 0; j < k; ++j) {
      const int kj = __builtin_amdgcn_readlane(key, j);
      slot += (kj < key) ? 1 : 0;
      nvalid += (kj != 0x7FFFFFFF) ? 1 : 0;
      errs |= __builtin_amdgcn_readlane(err, j);
    }
    if (lane < k) {
      pp.pair_slot[lane] = valid ? slot : -1;
      s_e[lane] = valid ? e : -1;
      s_w[lane] = w;
      if (valid) {
        pp.slot_pair[slot] = lane;
        pp.slot_info[slot] = w << 24;  // token 0
        pp.chunks[slot] = make_int4(e, slot, 1, 1 << (w - 1));
        int cnt = 0;
        for (int bb = 1; bb <= w; ++bb) cnt |= 1 << (8 * (bb - 1));
        pp.chunk_cnt[slot] = cnt;
      }
    }
    if (lane >= nvalid && lane < s.P) pp.slot_pair[lane] = -1;
    if (lane == 0) {
      pp.meta[0] = nvalid;
      pp.meta[1] = errs;
    }
    // shared experts: the token at full width
    if (lane < s.n_shared) {
      pp.chunks[s.max_rchunks + lane] = make_int4(lane, s.P + lane, 1, (1 << (B - 1)) | (1 << 16));
      int cnt = 0;
      for (int bb = 1; bb <= B; ++bb) cnt |= 1 << (8 * (bb - 1));
      pp.chunk_cnt[s.max_rchunks + lane] = cnt;
      pp.slot_info[s.P + lane] = B << 24;
    }
  }
  __syncthreads();

  // 3. expert offsets (valid pairs of smaller experts) and widest widths
  for (int e = tid; e <= s.E; e += ONE_NT) {
    int off = 0, mb = 0;
    for (int j = 0; j < s.k; ++j) {
      const int ej = s_e[j];
      off += (ej >= 0 && ej < e) ? 1 : 0;
      if (ej == e) mb = s_w[j];
    }
    pp.expert_off[e] = off;
    if (e < s.E) pp.expert_maxbits[e] = mb;
  }
}
}  // namespace

bool control_fits(const FfnShape& s) {
  return s.P <= CTL_MAX_PAIRS && (long)s.E * s.B * s.W <= PM_SMALL_WORDS && s.E <= 256;
}

// the top-k inside the control kernel while every token has a wave of its own
bool control_does_topk(const FfnShape& s) { return s.T <= CTL_TOPK_TOKENS; }

hipError_t launch_control(const FfnShape& s, const FfnLayout& L, char* ws, const double* logits, int renorm,
                          int n_star, int b_lo, int b_max, int* idx, float* gate, uint8_t* bits,
                          hipStream_t stream) {
  if (control_does_topk(s))
    hipLaunchKernelGGL(k_control<true>, dim3(1), dim3(PM_NT), 0, stream, s, plan_ptrs(L, ws), logits, renorm, n_star,
                       b_lo, b_max, idx, gate, bits);
  else
    hipLaunchKernelGGL(k_control<false>, dim3(1), dim3(PM_NT), 0, stream, s, plan_ptrs(L, ws), logits, renorm,
                       n_star, b_lo, b_max, idx, gate, bits);
  return hipGetLastError();
}


bool one_token_fits(const FfnShape& s) { return s.T == 1 && s.cs == 16 && s.k <= 8 && s.n_shared <= 64; }

hipError_t launch_one(const FfnShape& s, const FfnLayout& L, char* ws, const uint16_t* x, const double* logits,
                      int renorm, int n_star, int b_lo, int b_max, int* idx, float* gate, uint8_t* bits,
                      hipStream_t stream) {
  hipLaunchKernelGGL(k_one, dim3(1), dim3(ONE_NT), 0, stream, s, plan_ptrs(L, ws), x,
                     reinterpret_cast<uint16_t*>(ws + L.xg), reinterpret_cast<float2*>(ws + L.xvg), logits, renorm,
                     n_star, b_lo, b_max, idx, gate, bits);
  return hipGetLastError();
}

}  // namespace moe
