// Device code of the router's softmax + top-k, shared by the top-k kernel
// and the fused decode control kernel.
#pragma once

#include "common.hpp"

namespace moe {
namespace {

// Order-preserving map of a double to an unsigned 64-bit key (larger logit,
// larger key; -0 and +0 equal).  Logits are finite.
__device__ __forceinline__ uint64_t order_key64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v + 0.0);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Inverse of order_key64 (the logit, with -0 read as +0).
__device__ __forceinline__ double key_to_double(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// (key, index) a beats (key, index) b: larger logit, then smaller index.
__device__ __forceinline__ bool beats(uint64_t ka, int ia, uint64_t kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// One step of the wave arg-max: each lane takes the better of its own
// candidate and the candidate DPP control CTRL moves to it (lanes with no
// source keep their own).
template <int CTRL, int ROWS>
__device__ __forceinline__ void argmax_step(uint32_t& hi, uint32_t& lo, int& ix) {
  const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWS, 0xF, false);
  const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWS, 0xF, false);
  const int oix = __builtin_amdgcn_update_dpp(ix, ix, CTRL, ROWS, 0xF, false);
  const uint64_t ok = ((uint64_t)ohi << 32) | olo, mk = ((uint64_t)hi << 32) | lo;
  if (beats(ok, oix, mk, ix)) {
    hi = ohi;
    lo = olo;
    ix = oix;
  }
}

// Softmax over the E logits of one token and its top k, by one wave
// (emit(j, expert, gate) for j < k, by lane j): k
// rounds of a wave-wide arg-max; lane l owns experts l, l+64, l+128, l+192.
// The arg-max shifts candidates right by 1, 2, 4, 8 lanes within each row of
// 16 and then carries rows 0 and 2 into rows 1 and 3 (row broadcast 15) and
// row 1 into rows 2 and 3 (row broadcast 31): lane 63 ends with the winner.
template <typename Emit>
__device__ void topk_token(const double* __restrict__ lg, int E, int k, int renorm, Emit emit, int lane) {
  double lv[4];
  uint64_t key[4];
  bool avail[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    avail[i] = e < E;
    lv[i] = avail[i] ? lg[e] : 0.0;
    key[i] = avail[i] ? order_key64(lv[i]) : 0ull;
  }
  double mx = 0.0, ps = 0.0;
  int my_e = 0;        // lane r keeps the winner of round r
  double my_l = 0.0;
  for (int r = 0; r < k; ++r) {
    uint64_t bk = 0ull;
    int be = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (avail[i] && beats(key[i], lane + 64 * i, bk, be)) {
        bk = key[i];
        be = lane + 64 * i;
      }
    uint32_t hi = (uint32_t)(bk >> 32), lo = (uint32_t)bk;
    argmax_step<0x111, 0xF>(hi, lo, be);  // row_shr:1
    argmax_step<0x112, 0xF>(hi, lo, be);  // row_shr:2
    argmax_step<0x114, 0xF>(hi, lo, be);  // row_shr:4
    argmax_step<0x118, 0xF>(hi, lo, be);  // row_shr:8
    argmax_step<0x142, 0xA>(hi, lo, be);  // row_bcast:15
    argmax_step<0x143, 0xC>(hi, lo, be);  // row_bcast:31
    be = __builtin_amdgcn_readlane(be, 63);
    // the winner's logit, from its key (no memory round trip)
    const uint64_t wk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, 63) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
    // the owner retires the winner
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (be == lane + 64 * i) avail[i] = false;
    const double bl = key_to_double(wk);
    if (lane == r) {
      my_e = be;
      my_l = bl;
    }
    if (r == 0) {
      mx = bl;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + 64 * i < E) ps += exp(lv[i] - mx);
      ps = wave_sum_d(ps);
    }
  }
  // probabilities of the k winners (lane r: round r), and for renormalised
  // gates their sum in round order
  const double p = lane < k ? exp(my_l - mx) / ps : 0.0;
  double psel = 0.0;
  if (renorm) {
    const long long pb = __double_as_longlong(p);
    for (int r = 0; r < k; ++r) {
      const int lo = __builtin_amdgcn_readlane((int)(uint32_t)pb, r);
      const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(pb >> 32), r);
      psel += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
    }
  }
  if (lane < k) emit(lane, my_e, (float)(renorm ? p / psel : p));
}

}  // namespace
}  // namespace moe
