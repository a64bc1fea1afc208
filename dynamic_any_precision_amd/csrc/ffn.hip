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
// become an exact bf16 A operand (values 128 + f 4^a, see common.hpp), the
// activations, pre-scaled by 2^(B-2-p) 4^-a and masked to the pairs that
// read that unit, are the B operand, and v_mfma_f32_16x16x32_bf16 sums them
// in fp32.  Per quant group the fp32 partial is multiplied by s; the
// remaining terms s * (c_delta X_G - 128 F_t V_G) - s z X_G (V_G the
// 4^-a-weighted group sum, F_t the sum of the unit factors the pair reads)
// are two small fp32 products over groups, done with v_mfma_f32_16x16x4f32.
//
// Work items: (chunk of <= 16 pairs of one expert, tile pair).  W13: gate
// rows 16i.. and up rows f+16i.. of the expert; W2: rows 32i..32i+31.  A
// wave streams the chunk's planes for its two tiles once, in 128-bit loads
// from the lane-interleaved layout, and serves all pairs of the chunk; a pair
// only receives the units its own width covers.
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
  L.xb = take((size_t)s.T * s.B * s.d * 2);
  L.xv = take((size_t)s.T * (s.d / s.g) * 8);
  L.hb = take((size_t)s.Pt * s.B * s.fmax * 2);
  L.hsum = take((size_t)s.Pt * (s.fmax / 16) * 8);
  L.obuf = take((size_t)s.Pt * s.d * 4);
  L.total = o;
  return L;
}

namespace {

// ---------------------------------------------------------------------------
// activation prep: B-fragment order, per-plane scaling, group sums

__global__ __launch_bounds__(64) void k_xprep(const uint16_t* __restrict__ x, int d, int B, int g,
                                              uint16_t* __restrict__ xb, float2* __restrict__ xv) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int nchunk = d / 32;
  const int cpg = g / 32;  // chunks per quant group
  for (int c0 = 0; c0 < nchunk; c0 += 64) {
    const int ch = c0 + lane;
    float X = 0.f, V = 0.f;
    if (ch < nchunk) {
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * d + ch * 32);
      uint32_t in[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 v = src[q];
        in[4 * q + 0] = v.x; in[4 * q + 1] = v.y; in[4 * q + 2] = v.z; in[4 * q + 3] = v.w;
      }
      float xf[32];
#pragma unroll
      for (int c = 0; c < 32; ++c) {
        xf[c] = bf16_to_f32((c & 1) ? (in[c >> 1] >> 16) : (in[c >> 1] & 0xFFFFu));
        X += xf[c];
        V += xf[c] * (1.0f / (float)(1 << (2 * a_exp(c & 15))));
      }
      for (int p = 0; p < B; ++p) {
        const float pscale = ldexpf(1.0f, B - 2 - p);
        uint16_t out[32];
#pragma unroll
        for (int c = 0; c < 32; ++c) {
          const float v = xf[c] * pscale * (1.0f / (float)(1 << (2 * a_exp(c & 15))));
          out[frag_pos(c)] = (uint16_t)f32_to_bf16(v);
        }
        uint4* dst = reinterpret_cast<uint4*>(xb + ((size_t)t * B + p) * d + ch * 32);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint4 v;
          v.x = out[8 * q + 0] | ((uint32_t)out[8 * q + 1] << 16);
          v.y = out[8 * q + 2] | ((uint32_t)out[8 * q + 3] << 16);
          v.z = out[8 * q + 4] | ((uint32_t)out[8 * q + 5] << 16);
          v.w = out[8 * q + 6] | ((uint32_t)out[8 * q + 7] << 16);
          dst[q] = v;
        }
      }
    }
    // group sums over cpg consecutive chunks (lanes)
    for (int m = 1; m < cpg; m <<= 1) {
      X += __shfl_xor(X, m, WAVE);
      V += __shfl_xor(V, m, WAVE);
    }
    if (ch < nchunk && (lane % cpg) == 0) xv[(size_t)t * (d / g) + ch / cpg] = make_float2(X, V);
  }
}

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

constexpr int MODE_W13 = 0;
constexpr int MODE_W2 = 1;

struct FfnArgs {
  MatrixDev m[2];        // [0] routed, [1] shared
  int tpi[2];            // tile pairs per chunk
  int B, g, T, P, d, fmax;
  const int4* chunks;
  const int* meta;
  int max_rchunks, n_schunks;
  const int* slot_info;
  const uint16_t* xb;    // W13 B source [T][B][d]
  const float2* xv;      // [T][d/g]
  uint16_t* hb;          // [Pt][B][fmax]
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

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void run_item(const FfnArgs& a, const MatrixDev& M, int e, int s0, int m, int ti,
                                         int is_shared) {
  constexpr Units U = make_units(MASK);
  constexpr int BM = mask_bmax(MASK);
  const int lane = threadIdx.x & 63;
  const int tcol = lane & 15;  // token column of this lane (B operand, C layout)
  const int jg = lane >> 4;    // K chunk of this lane (A/B operand) and row quad (C layout)
  const int B = a.B;
  const int K = M.K;
  const int NKB = K >> 7;
  const int NQ = (NKB + 3) >> 2;
  const int NQG = K / a.g;
  const size_t plane_words = (size_t)M.N * K / 32;
  const int tile_words = K / 2;

  // token of this lane's column
  int slot = -1, tok = 0, bt = 0;
  if (tcol < m) {
    slot = s0 + tcol;
    const int info = a.slot_info[slot];
    tok = info & 0xFFFFFF;
    bt = info >> 24;
  }
  bool cov[4];
  float Ft = 0.f;
#pragma unroll
  for (int u = 0; u < U.n; ++u) {
    cov[u] = bt >= U.p[u] + U.np[u];
    if (cov[u]) Ft += ldexpf(1.0f, B - 2 - U.p[u]);
  }
  const float ct = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;

  // tiles of this work item
  int tr[2];
  if (MODE == MODE_W13) {
    tr[0] = ti;
    tr[1] = (M.N >> 5) + ti;  // up rows start at f = N/2
  } else {
    tr[0] = 2 * ti;
    tr[1] = 2 * ti + 1;
  }
  const uint32_t* pbase[2];
  const float* szb[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    pbase[r] = M.planes + (size_t)e * B * plane_words + (size_t)tr[r] * tile_words;
    szb[r] = M.sz + ((size_t)e * (M.N >> 4) + tr[r]) * NQG * 32;
  }
  // B-operand source of this lane
  const uint16_t* bsrc;
  if (MODE == MODE_W13) {
    bsrc = a.xb + (size_t)tok * B * K;
  } else {
    bsrc = a.hb + (size_t)(slot < 0 ? 0 : slot) * B * a.fmax;
  }
  const size_t bstride = (MODE == MODE_W13) ? (size_t)K : (size_t)a.fmax;

  f32x4_t out[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) out[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wq[2][BM];
  {
    const int nq = min(4, NKB);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int p = 0; p < BM; ++p) wq[r][p] = load_words(pbase[r] + p * plane_words + lane * nq, nq);
  }

  for (int q = 0; q < NQ; ++q) {
    const int nq = min(4, NKB - 4 * q);
    uint4 wn[2][BM];
    if (q + 1 < NQ) {
      const int nq1 = min(4, NKB - 4 * (q + 1));
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int p = 0; p < BM; ++p)
          wn[r][p] = load_words(pbase[r] + p * plane_words + 256 * (q + 1) + lane * nq1, nq1);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < nq) {
        const int kb = 4 * q + w;
        f32x4_t acc[QPK][2];
#pragma unroll
        for (int h = 0; h < QPK; ++h)
#pragma unroll
          for (int r = 0; r < 2; ++r) acc[h][r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < U.n; ++u) {
          uint4 bv[4];
          if (cov[u]) {
            const uint4* src =
                reinterpret_cast<const uint4*>(bsrc + (size_t)U.p[u] * bstride + kb * 128 + jg * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = src[i];
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) bv[i] = make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const uint32_t hi = comp(wq[r][U.p[u]], w);
            const uint32_t lo = (U.np[u] == 2) ? comp(wq[r][U.p[u] + 1], w) : 0u;
            Frag16 A;
            unpack_unit(hi, lo, A);
#pragma unroll
            for (int h = 0; h < QPK; ++h) {
              const bool keep = (QPK == 1) || ((jg >> 1) == h);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint4 bb = keep ? bv[i] : make_uint4(0, 0, 0, 0);
                acc[h][r] = mfma_bf16(frag_operand(A, i), as_bf16x8(bb), acc[h][r]);
              }
            }
          }
        }
#pragma unroll
        for (int h = 0; h < QPK; ++h) {
          const int G = kb * QPK + h;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            const float4 s4 = *reinterpret_cast<const float4*>(szb[r] + (size_t)G * 32 + 4 * jg);
            out[r][0] += s4.x * acc[h][r][0];
            out[r][1] += s4.y * acc[h][r][1];
            out[r][2] += s4.z * acc[h][r][2];
            out[r][3] += s4.w * acc[h][r][3];
          }
        }
      }
    }
    if (q + 1 < NQ) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int p = 0; p < BM; ++p) wq[r][p] = wn[r][p];
    }
  }

  // group-sum corrections: s*(c X - 128 F V) - s z X, as fp32 matrix products over groups
  f32x4_t corr[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) corr[r] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int q4 = 0; q4 < NQG; q4 += 4) {
    const int G = q4 + jg;
    const bool gv = G < NQG;
    float X = 0.f, V = 0.f;
    if (gv && bt > 0) {
      if (MODE == MODE_W13) {
        const float2 v = a.xv[(size_t)tok * NQG + G];
        X = v.x;
        V = v.y;
      } else {
        const int tpg = a.g >> 4;  // 16-row partials per quant group
        const float2* hs = a.hsum + (size_t)slot * (a.fmax >> 4) + (size_t)G * tpg;
        for (int pt = 0; pt < tpg; ++pt) {
          const float2 v = hs[pt];
          X += v.x;
          V += v.y;
        }
      }
    }
    const float Kc = ct * X - 128.0f * Ft * V;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      float sv = 0.f, zv = 0.f;
      if (gv) {
        sv = szb[r][(size_t)G * 32 + tcol];
        zv = szb[r][(size_t)G * 32 + 16 + tcol];
      }
      corr[r] = mfma_f32(sv, Kc, corr[r]);
      corr[r] = mfma_f32(-sv * zv, X, corr[r]);
    }
  }

  if (MODE == MODE_W13) {
    const int f = M.N >> 1;
    const size_t hstride = (size_t)a.fmax;
    float Xp = 0.f, Vp = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gval = out[0][i] + corr[0][i];
      const float uval = out[1][i] + corr[1][i];
      const float hval = gval / (1.0f + expf(-gval)) * uval;
      const uint32_t hb16 = f32_to_bf16(hval);
      const float hf = bf16_to_f32(hb16);
      const int n = ti * 16 + 4 * jg + i;  // column of W2
      const float ainv = 1.0f / (float)(1 << (2 * a_exp(n & 15)));
      Xp += hf;
      Vp += hf * ainv;
      if (bt > 0) {
        const int pos = (n & ~31) + frag_pos(n & 31);
#pragma unroll
        for (int u = 0; u < U.n; ++u) {
          if (cov[u]) {
            const float v = hf * ldexpf(1.0f, B - 2 - U.p[u]) * ainv;
            a.hb[((size_t)slot * B + U.p[u]) * hstride + pos] = (uint16_t)f32_to_bf16(v);
          }
        }
      }
    }
    (void)f;
    Xp += __shfl_xor(Xp, 16, WAVE);
    Vp += __shfl_xor(Vp, 16, WAVE);
    Xp += __shfl_xor(Xp, 32, WAVE);
    Vp += __shfl_xor(Vp, 32, WAVE);
    if (jg == 0 && bt > 0) a.hsum[(size_t)slot * (a.fmax >> 4) + ti] = make_float2(Xp, Vp);
  } else {
    if (bt > 0) {
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        float4 o;
        o.x = out[r][0] + corr[r][0];
        o.y = out[r][1] + corr[r][1];
        o.z = out[r][2] + corr[r][2];
        o.w = out[r][3] + corr[r][3];
        *reinterpret_cast<float4*>(a.obuf + (size_t)slot * a.d + tr[r] * 16 + 4 * jg) = o;
      }
    }
  }
  (void)is_shared;
}

template <int MODE, int QPK>
__global__ __launch_bounds__(256) void k_ffn(FfnArgs a) {
  const int gw = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nw = (gridDim.x * blockDim.x) >> 6;
  const int n_rc = a.meta[0];
  const long items_r = (long)n_rc * a.tpi[0];
  const long items = items_r + (long)a.n_schunks * a.tpi[1];
  for (long w = gw; w < items; w += nw) {
    int4 ch;
    int ti, sh;
    if (w < items_r) {
      ch = a.chunks[w / a.tpi[0]];
      ti = (int)(w % a.tpi[0]);
      sh = 0;
    } else {
      const long w2 = w - items_r;
      ch = a.chunks[a.max_rchunks + w2 / a.tpi[1]];
      ti = (int)(w2 % a.tpi[1]);
      sh = 1;
    }
    const MatrixDev& M = a.m[sh];
    const int mask = ch.w & 15;
    switch (mask) {
#define MOE_CASE(MK) \
  case MK:           \
    run_item<MODE, QPK, MK>(a, M, ch.x, ch.y, ch.z, ti, sh); \
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

int grid_for(long max_items, int num_cu) {
  const long waves = max_items;
  long blocks = (waves + 3) / 4;
  const long cap = (long)num_cu * 8;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

hipError_t launch_xprep(const FfnShape& s, const FfnLayout& L, char* ws, const uint16_t* x, hipStream_t stream) {
  hipLaunchKernelGGL(k_xprep, dim3(s.T), dim3(64), 0, stream, x, s.d, s.B, s.g,
                     reinterpret_cast<uint16_t*>(ws + L.xb), reinterpret_cast<float2*>(ws + L.xv));
  return hipGetLastError();
}

hipError_t launch_ffn_w13(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                          int num_cu, hipStream_t stream) {
  FfnArgs a = make_args(s, L, ws, routed, shared);
  a.tpi[0] = s.f / 16;
  a.tpi[1] = s.n_shared ? s.fs / 16 : 1;
  const long max_items = (long)s.max_rchunks * a.tpi[0] + (long)s.n_schunks * a.tpi[1];
  const int grid = grid_for(max_items, num_cu);
  if (s.g == 64)
    hipLaunchKernelGGL((k_ffn<MODE_W13, 2>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_ffn<MODE_W13, 1>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_ffn_w2(const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                         int num_cu, hipStream_t stream) {
  FfnArgs a = make_args(s, L, ws, routed, shared);
  a.tpi[0] = s.d / 32;
  a.tpi[1] = s.d / 32;
  const long max_items = (long)(s.max_rchunks + s.n_schunks) * a.tpi[0];
  const int grid = grid_for(max_items, num_cu);
  if (s.g == 64)
    hipLaunchKernelGGL((k_ffn<MODE_W2, 2>), dim3(grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((k_ffn<MODE_W2, 1>), dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
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
