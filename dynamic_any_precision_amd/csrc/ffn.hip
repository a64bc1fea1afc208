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

// Any-precision expert FFN: activation gather, gate/up projection with
// SwiGLU, down projection, gate-weighted combine.
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
// become an exact bf16 operand (values 2^(B-2-p) (128 + f 4^a), see
// common.hpp), the activations, pre-scaled by 4^-a, are the other operand,
// and v_mfma_f32_16x16x32_bf16 sums them in fp32 as D[token][row].  Per quant
// group the fp32 partial is multiplied by s; a pair only keeps the units its
// own width reads (units are grouped into coverage classes, one accumulator
// each).  The remaining terms s * (c_delta X_G - 128 F_t V_G) - s z X_G (V_G
// the 4^-a-weighted group sum, F_t the sum of the unit factors the pair
// reads) are two small fp32 products over groups (v_mfma_f32_16x16x4f32).
//
// Data movement.  A chunk is <= 16 consecutive slots of one expert.  Its
// activations are gathered once into MFMA-fragment order, 1 KiB per
// (k-block, MFMA index), so that every activation load of the streaming
// loop is one contiguous 1 KiB wave access; gate/up writes the SwiGLU output
// straight into the same order for the down projection.  The weight planes
// are read as 256 contiguous bytes per plane and k-block of a 16-row tile.
// All streaming loads are raw buffer loads: a scalar resource and a scalar
// step offset, so the per-step addressing is scalar work, and an offset
// beyond the resource reads as zero.
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
  const size_t NC = (size_t)s.max_rchunks + s.n_schunks;
  L.pair_key = take((size_t)s.P * 4);
  L.bitmap = take(NK * s.W * 4);
  L.prefix = take(NK * s.W * 4);
  L.slot_pair = take((size_t)s.P * 4);
  L.pair_slot = take((size_t)s.P * 4);
  L.slot_info = take((size_t)s.Pt * 4);
  L.chunks = take(NC * 16);
  L.meta = take(64);
  L.expert_off = take((size_t)(s.E + 1) * 4);
  L.expert_maxbits = take((size_t)s.E * 4);
  L.xg = take(NC * s.d * 16 * 2);
  L.xvg = take(NC * (s.d / s.g) * 16 * 8);
  L.hg = take(NC * s.fmax * 16 * 2);
  L.hsg = take(NC * (s.fmax / 16) * 16 * 8);
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

// Coverage classes: class c holds the units that pairs of width >= w[c]
// read and narrower pairs do not; class 0 is read by every pair of the chunk.
struct Classes {
  int n;
  int w[4];
  int of_unit[4];
};

__host__ __device__ constexpr Classes make_classes(int mask) {
  Classes c{0, {0, 0, 0, 0}, {0, 0, 0, 0}};
  for (int b = 1; b <= 4; ++b)
    if (mask & (1 << (b - 1))) c.w[c.n++] = b;
  const Units u = make_units(mask);
  for (int i = 0; i < u.n; ++i) {
    const int th = u.p[i] + u.np[i];
    int k = 0;
    while (c.w[k] < th) ++k;
    c.of_unit[i] = k;
  }
  return c;
}

constexpr int MODE_W13 = 0;
constexpr int MODE_W2 = 1;

struct FfnArgs {
  MatrixDev m[2];        // [0] routed, [1] shared
  int items[2];          // work items per chunk (routed, shared)
  int B, g, T, P, d, fmax;
  const int4* chunks;
  const int* meta;
  int max_rchunks, n_schunks;
  const int* slot_info;
  const uint16_t* act;   // activation fragments [chunk][K/128][4][64][8]
  const float2* asum;    // W13: (X, V) per [chunk][K/g][16]; W2: per [chunk][K/16][16]
  int act_stride;        // elements per chunk
  int asum_stride;       // float2 per chunk
  uint16_t* hg;          // gate/up output fragments, [chunk][fmax/128][4][64][8]
  float2* hsg;           // gate/up output partial sums [chunk][fmax/16][16]
  float* obuf;           // down output [Pt][d]
};

// Raw buffer loads (resource flags of gfx9: 32-bit data format, untyped).
constexpr uint32_t BUF_FLAGS = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)BUF_FLAGS);
}
__device__ __forceinline__ uint32_t bld32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ float bldf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(bld32(r, voff, soff));
}
__device__ __forceinline__ u32x4_t bld128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ float2 bld64f(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
  return make_float2(__uint_as_float(v[0]), __uint_as_float(v[1]));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------------------
// Activation gather: one block per (chunk, 128-column k-block).  Token rows
// of the chunk are read (zero rows past its length), scaled by 4^-a, put in
// fragment order through LDS and written as 4 KiB contiguous; the plain and
// 4^-a-weighted sums of every quant group go beside them.

struct GatherArgs {
  const uint16_t* x;
  int d, g;
  const int4* chunks;
  const int* meta;
  int max_rchunks;
  const int* slot_info;
  uint16_t* xg;
  float2* xvg;
};

__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int c = blockIdx.x;
  const int kb = blockIdx.y;
  if (c < a.max_rchunks && c >= a.meta[0]) return;
  const int4 ch = a.chunks[c];
  const int s0 = ch.y, m = ch.z;
  const int tid = threadIdx.x, t = tid >> 4, q = tid & 15;
  __shared__ uint4 frag[256];
  uint16_t* fr = reinterpret_cast<uint16_t*>(frag);
  uint32_t in[4] = {0u, 0u, 0u, 0u};
  if (t < m) {
    const int tok = a.slot_info[s0 + t] & 0xFFFFFF;
    const uint4 v = *reinterpret_cast<const uint4*>(a.x + (size_t)tok * a.d + kb * 128 + 8 * q);
    in[0] = v.x; in[1] = v.y; in[2] = v.z; in[3] = v.w;
  }
  float X = 0.f, V = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = 8 * q + j;  // column within the k-block
    const int cc = col & 31;
    const float xf = bf16_to_f32((j & 1) ? (in[j >> 1] >> 16) : (in[j >> 1] & 0xFFFFu));
    const float sc = 1.0f / (float)(1 << (2 * a_exp(cc & 15)));
    X += xf;
    V += xf * sc;
    const int fp = frag_pos(cc);
    fr[((fp >> 3) * 64 + (col >> 5) * 16 + t) * 8 + (fp & 7)] = (uint16_t)f32_to_bf16(xf * sc);
  }
  const int tpg = a.g >> 3;  // threads per quant group
  for (int msk = 1; msk < tpg; msk <<= 1) {
    X += __shfl_xor(X, msk, WAVE);
    V += __shfl_xor(V, msk, WAVE);
  }
  const int NQG = a.d / a.g;
  if ((q & (tpg - 1)) == 0)
    a.xvg[((size_t)c * NQG + kb * (128 / a.g) + q / tpg) * 16 + t] = make_float2(X, V);
  __syncthreads();
  reinterpret_cast<uint4*>(a.xg + ((size_t)c * (a.d / 128) + kb) * 2048)[tid] = frag[tid];
}

// ---------------------------------------------------------------------------
// Streaming core.
//
// One wave = one work item: a chunk and two 16-row tiles that share the
// chunk's activations (gate/up: gate tile u and up tile u; down: tiles 2u
// and 2u+1).  The wave walks the k-blocks of both tiles together: per
// k-block one plane word per lane, plane and tile, one scale per lane and
// tile and 4 x 16 B of activation fragment per lane, prefetched PF k-blocks
// ahead in a register ring.

constexpr int FFN_THREADS = 256;
#ifndef FFN_WPE
#define FFN_WPE 2  // waves per SIMD the kernel is compiled for
#endif
#ifndef FFN_PF
#define FFN_PF 2   // k-blocks in flight ahead of the one being computed
#endif

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void run_item(const FfnArgs& a, const MatrixDev& M, int c, int e, int s0, int m,
                                         int item) {
  constexpr Units U = make_units(MASK);
  constexpr Classes CL = make_classes(MASK);
  constexpr int BM = mask_bmax(MASK);
  constexpr int PF = (QPK == 2) ? 1 : FFN_PF;
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // token row of the activation operand; weight row of D
  const int jg = lane >> 4;   // k-chunk of the operands; token quad of D
  const int B = a.B;
  const int K = M.K;
  const int NKB = K >> 7;
  const int NQG = K / a.g;
  const uint32_t plane_bytes = (uint32_t)((size_t)M.N * K / 8);
  const int tile0 = (MODE == MODE_W13) ? item : 2 * item;
  const int tile1 = (MODE == MODE_W13) ? (M.N >> 5) + item : 2 * item + 1;

  // token of the activation row (correction operand)
  float FA = 0.f, ctA = 0.f;
  {
    const int bt = r16 < m ? (a.slot_info[s0 + r16] >> 24) : 0;
#pragma unroll
    for (int u = 0; u < U.n; ++u)
      if (bt >= U.p[u] + U.np[u]) FA += ldexpf(1.0f, B - 2 - U.p[u]);
    ctA = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;
  }
  // tokens 4jg+i of D: per-class factors (class 0 is read by every pair)
  float fac[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tk = 4 * jg + i;
    const int bt = tk < m ? (a.slot_info[s0 + tk] >> 24) : 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) fac[k][i] = (k < CL.n && bt >= CL.w[k]) ? 1.0f : 0.0f;
  }
  uint32_t ubias[4];
#pragma unroll
  for (int u = 0; u < U.n; ++u) ubias[u] = vconst(unit_bias(B - 2 - U.p[u]));
  const UnpackConst kc = unpack_const();

  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(M.planes + (size_t)e * B * (plane_bytes / 4), (uint32_t)B * plane_bytes);
  const uint32_t sz_bytes = (uint32_t)((M.N >> 4) * NQG * 128);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(M.sz + (size_t)e * (sz_bytes / 4), sz_bytes);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + (size_t)c * a.act_stride, (uint32_t)K * 32);
  const int nsum = (MODE == MODE_W13) ? NQG : (K >> 4);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.asum + (size_t)c * a.asum_stride, (uint32_t)nsum * 128);

  struct Ops {
    u32x4_t act[4];
    uint32_t w0[BM], w1[BM];
    float s0[QPK], s1[QPK];
  };
  const uint32_t t0off = (uint32_t)tile0 * (K / 2) * 4;
  const uint32_t t1off = (uint32_t)tile1 * (K / 2) * 4;
  const uint32_t s0off = (uint32_t)tile0 * NQG * 128;
  const uint32_t s1off = (uint32_t)tile1 * NQG * 128;
  auto load = [&](int kb, Ops& o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o.act[i] = bld128(ra, lane * 16 + i * 1024, kb * 4096);
#pragma unroll
    for (int p = 0; p < BM; ++p) o.w0[p] = bld32(rp, lane * 4, t0off + kb * 256 + p * plane_bytes);
#pragma unroll
    for (int p = 0; p < BM; ++p) o.w1[p] = bld32(rp, lane * 4, t1off + kb * 256 + p * plane_bytes);
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      o.s0[h] = bldf(rs, r16 * 4, s0off + (kb * QPK + h) * 128);
      o.s1[h] = bldf(rs, r16 * 4, s1off + (kb * QPK + h) * 128);
    }
  };

  f32x4_t out0 = f32x4_t{0.f, 0.f, 0.f, 0.f}, out1 = out0, corr0 = out0, corr1 = out0;
  float cs0[QPK], cz0[QPK], cs1[QPK], cz1[QPK], cX[QPK], cV[QPK];

  // correction operands of the 4*QPK groups starting at k-block kb0:
  // lane (r16, jg) holds group kb0*QPK + 4h + jg of token / weight row r16
  auto load_corr = [&](int kb0) {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      const int G0 = kb0 * QPK + 4 * h;
      const bool gv = G0 + jg < NQG;
      const uint32_t vs = gv ? (uint32_t)(jg * 32 + r16) * 4 : OOB;
      cs0[h] = bldf(rs, vs, s0off + G0 * 128);
      cz0[h] = bldf(rs, vs, s0off + G0 * 128 + 64);
      cs1[h] = bldf(rs, vs, s1off + G0 * 128);
      cz1[h] = bldf(rs, vs, s1off + G0 * 128 + 64);
      if (MODE == MODE_W13) {
        const float2 v = bld64f(rx, gv ? (uint32_t)(jg * 16 + r16) * 8 : OOB, G0 * 128);
        cX[h] = v.x;
        cV[h] = v.y;
      } else {
        const int tpg = a.g >> 4;  // 16-column partial sums per group
        const uint32_t vo = gv ? (uint32_t)(jg * tpg * 16 + r16) * 8 : OOB;
        float X = 0.f, V = 0.f;
        for (int pt = 0; pt < tpg; ++pt) {
          const float2 v = bld64f(rx, vo, (G0 * tpg + pt) * 128);
          X += v.x;
          V += v.y;
        }
        cX[h] = X;
        cV[h] = V;
      }
    }
  };
  auto apply_corr = [&]() {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      const float Kc = ctA * cX[h] - 128.0f * FA * cV[h];
      corr0 = mfma_f32(Kc, cs0[h], corr0);
      corr0 = mfma_f32(cX[h], -cs0[h] * cz0[h], corr0);
      corr1 = mfma_f32(Kc, cs1[h], corr1);
      corr1 = mfma_f32(cX[h], -cs1[h] * cz1[h], corr1);
    }
  };

  // lanes whose k-chunk belongs to group h of a two-group k-block
  const uint32_t hmask0 = (QPK == 2 && (jg >> 1) != 0) ? 0u : 0xFFFFFFFFu;
  const uint32_t hmask1 = (QPK == 2 && (jg >> 1) != 1) ? 0u : 0xFFFFFFFFu;

  auto tile_mfma = [&](const u32x4_t (&act)[QPK][4], const uint32_t (&w)[BM], f32x4_t (&acc)[4][QPK]) {
#pragma unroll
    for (int k = 0; k < CL.n; ++k)
#pragma unroll
      for (int h = 0; h < QPK; ++h) acc[k][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < U.n; ++u) {
      const uint32_t hi = w[U.p[u]];
      const uint32_t lo = (U.np[u] == 2) ? w[U.p[u] + 1] : 0u;
      u32x4_t W[4];
      unpack_unit(hi, lo, U.np[u] == 2, ubias[u], kc, W);
      const int k = CL.of_unit[u];
#pragma unroll
      for (int h = 0; h < QPK; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[k][h] = mfma_bf16(as_bf16x8(act[h][i]), as_bf16x8(W[i]), acc[k][h]);
    }
  };
  auto tile_scale = [&](const f32x4_t (&acc)[4][QPK], const float (&s)[QPK], f32x4_t& out) {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[0][h][i];
#pragma unroll
        for (int k = 1; k < CL.n; ++k) v += fac[k][i] * acc[k][h][i];
        out[i] += s[h] * v;
      }
    }
  };

  auto compute = [&](const Ops& o) {
    u32x4_t act[QPK][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (QPK == 1) {
        act[0][i] = o.act[i];
      } else {
        act[0][i] = o.act[i] & hmask0;
        act[QPK - 1][i] = o.act[i] & hmask1;
      }
    }
    f32x4_t acc0[4][QPK], acc1[4][QPK];
    tile_mfma(act, o.w0, acc0);
    tile_mfma(act, o.w1, acc1);
    tile_scale(acc0, o.s0, out0);
    tile_scale(acc1, o.s1, out1);
  };

  auto finish = [&]() {
    const f32x4_t res0 = out0 + corr0;
    const f32x4_t res1 = out1 + corr1;
    if (MODE == MODE_W13) {
      // h column n of the down projection's input; tokens 4jg+i
      const int n = item * 16 + r16;
      const int cc = n & 31;
      const int fp = frag_pos(cc);
      const float ainv = 1.0f / (float)(1 << (2 * a_exp(cc & 15)));
      uint16_t* hrow = a.hg + (size_t)c * a.fmax * 16 +
                       ((size_t)((n >> 7) * 4 + (fp >> 3)) * 64 + ((n & 127) >> 5) * 16) * 8 + (fp & 7);
      float Xp[4], Vp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gval = res0[i];
        const float hval = gval / (1.0f + expf(-gval)) * res1[i];
        const float hf = bf16_to_f32(f32_to_bf16(hval));
        hrow[(4 * jg + i) * 8] = (uint16_t)f32_to_bf16(hf * ainv);
        Xp[i] = hf;
        Vp[i] = hf * ainv;
      }
#pragma unroll
      for (int msk = 1; msk < 16; msk <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Xp[i] += __shfl_xor(Xp[i], msk, WAVE);
          Vp[i] += __shfl_xor(Vp[i], msk, WAVE);
        }
      if (r16 == 0) {
        float4* hs = reinterpret_cast<float4*>(a.hsg + (size_t)c * (a.fmax >> 4) * 16 + item * 16 + 4 * jg);
        hs[0] = make_float4(Xp[0], Vp[0], Xp[1], Vp[1]);
        hs[1] = make_float4(Xp[2], Vp[2], Xp[3], Vp[3]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = 4 * jg + i;
        if (tk < m) {
          float* orow = a.obuf + (size_t)(s0 + tk) * a.d;
          orow[tile0 * 16 + r16] = res0[i];
          orow[tile1 * 16 + r16] = res1[i];
        }
      }
    }
  };

  // k-block step: loads PF ahead into the slot the previous step freed,
  // corrections every fourth k-block and at the end.
  auto step = [&](int kb, const Ops& cur, Ops& ahead) {
    if (kb + PF < NKB) load(kb + PF, ahead);
    if ((kb & 3) == 0) load_corr(kb);
    compute(cur);
    if ((kb & 3) == 3 || kb == NKB - 1) apply_corr();
  };

  Ops o[PF + 1];
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (q < NKB) load(q, o[q]);
  for (int kb0 = 0; kb0 < NKB; kb0 += PF + 1) {
#pragma unroll
    for (int q = 0; q <= PF; ++q)
      if (kb0 + q < NKB) step(kb0 + q, o[q], o[(q + PF) % (PF + 1)]);
  }
  finish();
}

template <int MODE, int QPK>
__global__ __launch_bounds__(FFN_THREADS) __attribute__((amdgpu_waves_per_eu(FFN_WPE, FFN_WPE))) void k_ffn(FfnArgs a) {
  const int gw = uniform((int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6));
  const int nw = (int)((gridDim.x * blockDim.x) >> 6);
  const int n_rc = a.meta[0];
  const int items_r = n_rc * a.items[0];
  const int items = items_r + a.n_schunks * a.items[1];
  for (int w = gw; w < items; w += nw) {
    int c, item, sh;
    if (w < items_r) {
      c = w / a.items[0];
      item = w - c * a.items[0];
      sh = 0;
    } else {
      const int w2 = w - items_r;
      const int cs = w2 / a.items[1];
      item = w2 - cs * a.items[1];
      c = a.max_rchunks + cs;
      sh = 1;
    }
    const int4 ch = a.chunks[c];
    const MatrixDev& M = a.m[sh];
    switch (ch.w & 15) {
#define MOE_CASE(MK) \
  case MK:           \
    run_item<MODE, QPK, MK>(a, M, c, ch.x, ch.y, ch.z, item); \
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
  a.hg = reinterpret_cast<uint16_t*>(ws + L.hg);
  a.hsg = reinterpret_cast<float2*>(ws + L.hsg);
  a.obuf = reinterpret_cast<float*>(ws + L.obuf);
  return a;
}

hipError_t launch_ffn(int mode, const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                      int num_cu, hipStream_t stream) {
  FfnArgs a = make_args(s, L, ws, routed, shared);
  // work items per chunk: gate/up -> f/16 tile pairs, down -> d/32 tile pairs
  if (mode == MODE_W13) {
    a.items[0] = s.f / 16;
    a.items[1] = s.n_shared ? s.fs / 16 : 1;
    a.act = reinterpret_cast<const uint16_t*>(ws + L.xg);
    a.act_stride = s.d * 16;
    a.asum = reinterpret_cast<const float2*>(ws + L.xvg);
    a.asum_stride = (s.d / s.g) * 16;
  } else {
    a.items[0] = s.d / 32;
    a.items[1] = s.d / 32;
    a.act = reinterpret_cast<const uint16_t*>(ws + L.hg);
    a.act_stride = s.fmax * 16;
    a.asum = reinterpret_cast<const float2*>(ws + L.hsg);
    a.asum_stride = (s.fmax / 16) * 16;
  }
  const int qpk = (s.g == 64) ? 2 : 1;
  const long max_items = (long)s.max_rchunks * a.items[0] + (long)s.n_schunks * a.items[1];
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

hipError_t launch_gather(const FfnShape& s, const FfnLayout& L, char* ws, const uint16_t* x, hipStream_t stream) {
  GatherArgs a;
  a.x = x;
  a.d = s.d;
  a.g = s.g;
  a.chunks = reinterpret_cast<const int4*>(ws + L.chunks);
  a.meta = reinterpret_cast<const int*>(ws + L.meta);
  a.max_rchunks = s.max_rchunks;
  a.slot_info = reinterpret_cast<const int*>(ws + L.slot_info);
  a.xg = reinterpret_cast<uint16_t*>(ws + L.xg);
  a.xvg = reinterpret_cast<float2*>(ws + L.xvg);
  hipLaunchKernelGGL(k_gather, dim3(s.max_rchunks + s.n_schunks, s.d / 128), dim3(256), 0, stream, a);
  return hipGetLastError();
}

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
