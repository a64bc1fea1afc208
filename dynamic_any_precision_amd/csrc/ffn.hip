// Any-precision expert FFN: gate/up projection with SwiGLU, down projection,
// gate-weighted combine.
//
// Math (per pair (t, e) at b planes, quant group G of row n, delta = B - b):
//   w = ((q >> delta) * 2^delta + c_delta - z) * s,  c_delta = (2^delta - 1)/2
// (floor-and-compensation read, MatMoE review, Core Contribution).  With
// X_G = sum_{c in G} x_c:
//   sum_c w x_c = s * [ sum_c ((q >> delta) << delta)(c) x_c + (c_delta - z) X_G ].
// The kept high bits are the first b planes, (q >> delta) << delta =
// sum_{p<b} bit_p 2^(B-1-p), so the first sum splits into plane units of one
// or two planes; a unit (p, p+1) contributes 2^(B-2-p) * sum_c f_c x_c with
// f = 2 bit_p + bit_{p+1} (a single plane p uses f = 2 bit_p).
//
// Each unit runs on the bf16 matrix cores: 16 rows x 32 columns of a unit
// become an exact bf16 A operand (values 2^(B-2-p) (128 + f 4^a), see
// common.hpp), the activations, pre-scaled by 4^-a and masked to the pairs
// that read that unit, are the B operand, and v_mfma_f32_16x16x32_bf16 sums
// them in fp32.  Per quant group the fp32 partial is multiplied by s; the
// remaining terms s * (c_delta X_G - 128 F_t V_G) - s z X_G (V_G the
// 4^-a-weighted group sum, F_t the sum of the unit factors the pair reads)
// are two small fp32 products over groups, done with v_mfma_f32_16x16x4f32.
//
// Work items, one per 256-thread block: (chunk of <= 16 pairs of one expert,
// row block).  W13: gate rows 32i..32i+31 and the matching up rows; W2:
// rows 64i..64i+63.  Each wave streams one 16-row tile of the chunk's planes
// once, in 128-bit loads from the lane-interleaved layout, and serves all
// pairs of the chunk; a pair only receives the units its own width covers.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// workspace plan

static size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

FfnShape make_shape(int T, int k, int E, int B, int g, int d, int f, int n_shared, int fs) {
  FfnShape s;
  s.T = T; s.k = k; s.E = E; s.B = B; s.g = g; s.d = d; s.f = f;
  s.n_shared = n_shared; s.fs = n_shared ? fs : 0;
  s.P = T * k;
  s.Pt = s.P + n_shared * T;
  s.W = (T + 31) / 32;
  s.max_rchunks = (E < s.P ? E : s.P) + s.P / 16 + 1;
  s.n_schunks = n_shared * ((T + 15) / 16);
  s.fmax = s.fs > f ? s.fs : f;
  return s;
}

FfnLayout make_layout(const FfnShape& s) {
  FfnLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += al256(bytes); return r; };
  const size_t NK = (size_t)s.E * s.B;
  L.pair_key = take((size_t)s.P * 4);
  L.bitmap = take(NK * s.W * 4);
  L.prefix = take(NK * s.W * 4);
  L.slot_pair = take((size_t)s.P * 4);
  L.pair_slot = take((size_t)s.P * 4);
  L.slot_info = take((size_t)s.Pt * 4);
  L.chunks = take((size_t)(s.max_rchunks + s.n_schunks) * 16);
  L.meta = take(64);
  L.expert_off = take((size_t)(s.E + 1) * 4);
  L.expert_maxbits = take((size_t)s.E * 4);
  L.xb = take((size_t)s.T * s.d * 2);
  L.xv = take((size_t)s.T * (s.d / s.g) * 8);
  L.hb = take((size_t)s.Pt * s.fmax * 2);
  L.hsum = take((size_t)s.Pt * (s.fmax / 16) * 8);
  L.obuf = take((size_t)s.Pt * s.d * 4);
  L.total = o;
  return L;
}

namespace {

// ---------------------------------------------------------------------------
// plane units of a chunk, from the set of widths it holds (bit b-1 = width b)

struct Units {
  int n;
  int p[4];
  int np[4];
};

__host__ __device__ constexpr Units make_units(int mask) {
  Units u{0, {0, 0, 0, 0}, {0, 0, 0, 0}};
  int start = 0;
  for (int b = 1; b <= 4; ++b) {
    if (mask & (1 << (b - 1))) {
      int p = start;
      while (p < b) {
        const int n = (b - p >= 2) ? 2 : 1;
        u.p[u.n] = p;
        u.np[u.n] = n;
        u.n += 1;
        p += n;
      }
      start = b;
    }
  }
  return u;
}

__host__ __device__ constexpr int mask_bmax(int mask) {
  return (mask & 8) ? 4 : (mask & 4) ? 3 : (mask & 2) ? 2 : 1;
}

__host__ __device__ constexpr int mask_bmin(int mask) {
  return (mask & 1) ? 1 : (mask & 2) ? 2 : (mask & 4) ? 3 : 4;
}

constexpr int MODE_W13 = 0;
constexpr int MODE_W2 = 1;

struct FfnArgs {
  MatrixDev m[2];        // [0] routed, [1] shared
  int slices[2];         // work items (16-row tiles) per chunk
  int B, g, T, P, d, fmax;
  const int4* chunks;
  const int* meta;
  int max_rchunks, n_schunks;
  const int* slot_info;
  const uint16_t* xb;    // W13 B source [T][d]
  const float2* xv;      // [T][d/g]
  uint16_t* hb;          // W2 B source [Pt][fmax]
  float2* hsum;          // [Pt][fmax/16]
  float* obuf;           // [Pt][d]
};

__device__ __forceinline__ uint4 load_words(const uint32_t* p, int nq) {
  if (nq == 4) return *reinterpret_cast<const uint4*>(p);
  uint4 r = make_uint4(0, 0, 0, 0);
  if (nq == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    r.x = v.x; r.y = v.y;
  } else if (nq == 3) {
    r.x = p[0]; r.y = p[1]; r.z = p[2];
  } else {
    r.x = p[0];
  }
  return r;
}

__device__ __forceinline__ uint32_t comp(const uint4& v, int w) {
  return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
}

// ---------------------------------------------------------------------------
// Streaming core.
//
// One wave = one work item (chunk of <= 16 pairs of one expert, 16-row
// tile).  The wave streams the tile's planes one 128-column k-block at a
// time (one 32-bit word per lane and plane, 256 contiguous bytes per wave),
// reads the chunk's activation B-fragments and the tile's scales from L2 one
// k-block ahead, and keeps little state, so that many waves share each SIMD
// and hide one another's latencies (no LDS, no barriers).  For gate/up the wave streams the gate tile and then the up
// tile of the same rows and applies SwiGLU.

constexpr int FFN_THREADS = 256;
#ifndef FFN_WPE
#define FFN_WPE 2  // waves per SIMD the kernel is compiled for
#endif

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void run_item(const FfnArgs& a, const MatrixDev& M, int e, int s0, int m, int unit) {
  constexpr Units U = make_units(MASK);
  constexpr int BM = mask_bmax(MASK);
  constexpr int GPQ = 4 * QPK;  // quant groups per quad
  const int lane = threadIdx.x & 63;
  const int tcol = lane & 15;  // token column (B operand, C layout)
  const int jg = lane >> 4;    // K chunk (A/B operand), row quad (C layout)
  const int B = a.B;
  const int K = M.K;
  const int NKB = K >> 7;
  const int NQ = (NKB + 3) >> 2;
  const int NQG = K / a.g;
  const size_t plane_words = (size_t)M.N * K / 32;

  int slot = -1, tok = 0, bt = 0;
  if (tcol < m) {
    slot = s0 + tcol;
    const int info = a.slot_info[slot];
    tok = info & 0xFFFFFF;
    bt = info >> 24;
  }
  // Unit coverage is monotone in the plane index: once a pair stops covering
  // a unit it covers none of the later ones, so the B operand is masked in
  // place as the units advance.
  uint32_t umask[4];
  uint32_t ubias[4];
  float Ft = 0.f;
#pragma unroll
  for (int u = 0; u < U.n; ++u) {
    const bool cov = bt >= U.p[u] + U.np[u];
    umask[u] = cov ? 0xFFFFFFFFu : 0u;
    ubias[u] = vconst(unit_bias(B - 2 - U.p[u]));
    if (cov) Ft += ldexpf(1.0f, B - 2 - U.p[u]);
  }
  const float ct = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;
  const UnpackConst kc = unpack_const();
  const bool bval = bt > 0;
  const uint4* bsrc = reinterpret_cast<const uint4*>(
      MODE == MODE_W13 ? a.xb + (size_t)tok * K + jg * 32 : a.hb + (size_t)(slot < 0 ? 0 : slot) * a.fmax + jg * 32);
  const int tpg = a.g >> 4;

  constexpr int TPU = (MODE == MODE_W13) ? 2 : 1;
  const float* szexp = M.sz + (size_t)e * (M.N >> 4) * NQG * 32;
  const uint32_t* pexp = M.planes + (size_t)e * B * plane_words + lane;
  auto tile_of = [&](int which) { return (MODE == MODE_W13) ? (which == 0 ? unit : (M.N >> 5) + unit) : unit; };

  // operands of one k-block: one plane word per plane, 4 x 16 B of
  // activation fragment, the scales of the lane's four C-layout rows
  struct Ops {
    uint32_t w[BM];
    uint4 b[4];
    float4 s[QPK];
  };
  // the k-blocks of the item's tiles form one stream of TPU*NKB steps
  auto load = [&](int j, Ops& o) {
    const int which = (TPU == 1) ? 0 : j / NKB;
    const int kb = j - which * NKB;
    const int tile = tile_of(which);
    const uint32_t* pb = pexp + (size_t)tile * (K / 2) + 64 * kb;
#pragma unroll
    for (int p = 0; p < BM; ++p) o.w[p] = pb[p * plane_words];
    if (bval) {
      const uint4* bp = bsrc + kb * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) o.b[i] = bp[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o.b[i] = make_uint4(0, 0, 0, 0);
    }
    const float* szt = szexp + (size_t)tile * NQG * 32;
#pragma unroll
    for (int h = 0; h < QPK; ++h)
      o.s[h] = *reinterpret_cast<const float4*>(szt + (size_t)(kb * QPK + h) * 32 + 4 * jg);
  };

  f32x4_t out = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t corr = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t gres = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float cs[QPK], cz[QPK], cX[QPK], cV[QPK];

  // correction operands of the 4*QPK groups of k-blocks kb0..kb0+3 of a tile
  // (lane k-index jg <-> group)
  auto load_corr = [&](int which, int kb0) {
    const float* szt = szexp + (size_t)tile_of(which) * NQG * 32;
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      const int G = kb0 * QPK + 4 * h + jg;
      const bool gv = G < NQG;
      cs[h] = gv ? szt[(size_t)G * 32 + tcol] : 0.f;
      cz[h] = gv ? szt[(size_t)G * 32 + 16 + tcol] : 0.f;
      cX[h] = 0.f;
      cV[h] = 0.f;
      if (gv && bt > 0) {
        if (MODE == MODE_W13) {
          const float2 v = a.xv[(size_t)tok * NQG + G];
          cX[h] = v.x;
          cV[h] = v.y;
        } else {
          const float4* hs =
              reinterpret_cast<const float4*>(a.hsum + (size_t)slot * (a.fmax >> 4) + (size_t)G * tpg);
          for (int pt = 0; pt < tpg / 2; ++pt) {
            const float4 hv = hs[pt];
            cX[h] += hv.x + hv.z;
            cV[h] += hv.y + hv.w;
          }
        }
      }
    }
  };
  auto apply_corr = [&]() {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      const float Kc = ct * cX[h] - 128.0f * Ft * cV[h];
      corr = mfma_f32(cs[h], Kc, corr);
      corr = mfma_f32(-cs[h] * cz[h], cX[h], corr);
    }
  };

  auto compute = [&](Ops& o) {
    f32x4_t acc[QPK];
#pragma unroll
    for (int h = 0; h < QPK; ++h) acc[h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U.n; ++u) {
      if (u > 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o.b[i].x &= umask[u]; o.b[i].y &= umask[u]; o.b[i].z &= umask[u]; o.b[i].w &= umask[u];
        }
      }
      const uint32_t hi = o.w[U.p[u]];
      const uint32_t lo = (U.np[u] == 2) ? o.w[U.p[u] + 1] : 0u;
      u32x4_t A[4];
      unpack_unit(hi, lo, U.np[u] == 2, ubias[u], kc, A);
#pragma unroll
      for (int h = 0; h < QPK; ++h) {
        const bool keep = (QPK == 1) || ((jg >> 1) == h);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4_t bb = keep ? as_u32x4(o.b[i]) : u32x4_t{0u, 0u, 0u, 0u};
          acc[h] = mfma_bf16(as_bf16x8(A[i]), as_bf16x8(bb), acc[h]);
        }
      }
    }
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      out[0] += o.s[h].x * acc[h][0];
      out[1] += o.s[h].y * acc[h][1];
      out[2] += o.s[h].z * acc[h][2];
      out[3] += o.s[h].w * acc[h][3];
    }
  };

  auto finish_tile = [&](int which) {
    const f32x4_t res = out + corr;
    out = f32x4_t{0.f, 0.f, 0.f, 0.f};
    corr = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (MODE == MODE_W13) {
      if (which == 0) {
        gres = res;
        return;
      }
      float Xp = 0.f, Vp = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gval = gres[i];
        const float hval = gval / (1.0f + expf(-gval)) * res[i];
        const float hf = bf16_to_f32(f32_to_bf16(hval));
        const int n = unit * 16 + 4 * jg + i;  // column of W2
        const float ainv = 1.0f / (float)(1 << (2 * a_exp(n & 15)));
        Xp += hf;
        Vp += hf * ainv;
        if (bt > 0) a.hb[(size_t)slot * a.fmax + (n & ~31) + frag_pos(n & 31)] = (uint16_t)f32_to_bf16(hf * ainv);
      }
      Xp += __shfl_xor(Xp, 16, WAVE);
      Vp += __shfl_xor(Vp, 16, WAVE);
      Xp += __shfl_xor(Xp, 32, WAVE);
      Vp += __shfl_xor(Vp, 32, WAVE);
      if (jg == 0 && bt > 0) a.hsum[(size_t)slot * (a.fmax >> 4) + unit] = make_float2(Xp, Vp);
    } else {
      if (bt > 0)
        *reinterpret_cast<float4*>(a.obuf + (size_t)slot * a.d + unit * 16 + 4 * jg) =
            make_float4(res[0], res[1], res[2], res[3]);
    }
  };

  // One stream step: issue the loads PF k-blocks ahead into the ring slot
  // freed by the previous step, then compute this k-block; corrections at
  // every fourth k-block of a tile and at its end.
  constexpr int PF = 3;
  const int NJ = TPU * NKB;
  auto step = [&](int j, Ops& cur, Ops& ahead) {
    if (j + PF < NJ) load(j + PF, ahead);
    const int which = (TPU == 1) ? 0 : j / NKB;
    const int kb = j - which * NKB;
    if ((kb & 3) == 0) load_corr(which, kb);
    compute(cur);
    if ((kb & 3) == 3 || kb == NKB - 1) apply_corr();
    if (kb == NKB - 1) finish_tile(which);
  };

  Ops o0, o1, o2, o3;
  load(0, o0);
  if (1 < NJ) load(1, o1);
  if (2 < NJ) load(2, o2);
  for (int j = 0; j < NJ; j += 4) {
    step(j, o0, o3);
    if (j + 1 < NJ) step(j + 1, o1, o0);
    if (j + 2 < NJ) step(j + 2, o2, o1);
    if (j + 3 < NJ) step(j + 3, o3, o2);
  }
}

template <int MODE, int QPK>
__global__ __launch_bounds__(FFN_THREADS) __attribute__((amdgpu_waves_per_eu(FFN_WPE, FFN_WPE))) void k_ffn(FfnArgs a) {
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  const int n_rc = a.meta[0];
  const long items_r = (long)n_rc * a.slices[0];
  const long items = items_r + (long)a.n_schunks * a.slices[1];
  for (long w = gw; w < items; w += nw) {
    int4 ch;
    int unit, sh;
    if (w < items_r) {
      ch = a.chunks[w / a.slices[0]];
      unit = (int)(w % a.slices[0]);
      sh = 0;
    } else {
      const long w2 = w - items_r;
      ch = a.chunks[a.max_rchunks + w2 / a.slices[1]];
      unit = (int)(w2 % a.slices[1]);
      sh = 1;
    }
    const MatrixDev& M = a.m[sh];
    const int mask = ch.w & 15;
    switch (mask) {
#define MOE_CASE(MK) \
  case MK:           \
    run_item<MODE, QPK, MK>(a, M, ch.x, ch.y, ch.z, unit); \
    break;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
      MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14) MOE_CASE(15)
#undef MOE_CASE
      default:
        break;
    }
  }
}

// ---------------------------------------------------------------------------
// combine: y[t] = (acc ? y[t] : 0) + sum_j gate[t][j] o_(t,j) + sum_s o_(t,shared s)

__global__ __launch_bounds__(256) void k_combine(int T, int k, int d, int P, int n_shared,
                                                 const int* __restrict__ pair_slot, const float* __restrict__ gate,
                                                 const float* __restrict__ obuf, float* __restrict__ y,
                                                 int accumulate) {
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 * 4 >= d) return;
  float4 v = accumulate ? reinterpret_cast<const float4*>(y + (size_t)t * d)[n4] : make_float4(0.f, 0.f, 0.f, 0.f);
  for (int j = 0; j < k; ++j) {
    const int s = pair_slot[t * k + j];
    if (s < 0) continue;
    const float gt = gate[t * k + j];
    const float4 o = reinterpret_cast<const float4*>(obuf + (size_t)s * d)[n4];
    v.x += gt * o.x; v.y += gt * o.y; v.z += gt * o.z; v.w += gt * o.w;
  }
  for (int sh = 0; sh < n_shared; ++sh) {
    const float4 o = reinterpret_cast<const float4*>(obuf + (size_t)(P + sh * T + t) * d)[n4];
    v.x += o.x; v.y += o.y; v.z += o.z; v.w += o.w;
  }
  reinterpret_cast<float4*>(y + (size_t)t * d)[n4] = v;
}

FfnArgs make_args(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared) {
  FfnArgs a;
  a.m[0] = routed;
  a.m[1] = shared;
  a.B = s.B; a.g = s.g; a.T = s.T; a.P = s.P; a.d = s.d; a.fmax = s.fmax;
  a.chunks = reinterpret_cast<const int4*>(ws + L.chunks);
  a.meta = reinterpret_cast<const int*>(ws + L.meta);
  a.max_rchunks = s.max_rchunks;
  a.n_schunks = s.n_schunks;
  a.slot_info = reinterpret_cast<const int*>(ws + L.slot_info);
  a.xb = reinterpret_cast<const uint16_t*>(ws + L.xb);
  a.xv = reinterpret_cast<const float2*>(ws + L.xv);
  a.hb = reinterpret_cast<uint16_t*>(ws + L.hb);
  a.hsum = reinterpret_cast<float2*>(ws + L.hsum);
  a.obuf = reinterpret_cast<float*>(ws + L.obuf);
  return a;
}

hipError_t launch_ffn(int mode, const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                      int num_cu, hipStream_t stream) {
  FfnArgs a = make_args(s, L, ws, routed, shared);
  // work items per chunk: gate/up -> f/16 tile rows, down -> d/16
  if (mode == MODE_W13) {
    a.slices[0] = s.f / 16;
    a.slices[1] = s.n_shared ? s.fs / 16 : 1;
  } else {
    a.slices[0] = s.d / 16;
    a.slices[1] = s.d / 16;
  }
  const int qpk = (s.g == 64) ? 2 : 1;
  const long max_items = (long)s.max_rchunks * a.slices[0] + (long)s.n_schunks * a.slices[1];
  long grid = (max_items + 3) / 4;
  const long cap = (long)num_cu * FFN_WPE;  // FFN_WPE waves per SIMD x 4 SIMDs / 4 waves per block
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  if (mode == MODE_W13) {
    if (qpk == 2)
      hipLaunchKernelGGL((k_ffn<MODE_W13, 2>), dim3(grid), dim3(FFN_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_ffn<MODE_W13, 1>), dim3(grid), dim3(FFN_THREADS), 0, stream, a);
  } else {
    if (qpk == 2)
      hipLaunchKernelGGL((k_ffn<MODE_W2, 2>), dim3(grid), dim3(FFN_THREADS), 0, stream, a);
    else
      hipLaunchKernelGGL((k_ffn<MODE_W2, 1>), dim3(grid), dim3(FFN_THREADS), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ffn_w13(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                          int num_cu, hipStream_t stream) {
  return launch_ffn(MODE_W13, s, L, ws, routed, shared, num_cu, stream);
}

hipError_t launch_ffn_w2(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                         int num_cu, hipStream_t stream) {
  return launch_ffn(MODE_W2, s, L, ws, routed, shared, num_cu, stream);
}

hipError_t launch_combine(const FfnShape& s, const FfnLayout& L, char* ws, const float* gate, float* y,
                          int accumulate, hipStream_t stream) {
  dim3 grid((s.d / 4 + 255) / 256, s.T);
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, s.T, s.k, s.d, s.P, s.n_shared,
                     reinterpret_cast<const int*>(ws + L.pair_slot), gate,
                     reinterpret_cast<const float*>(ws + L.obuf), y, accumulate);
  return hipGetLastError();
}

}  // namespace moe
