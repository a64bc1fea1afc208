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
  // Wide chunks (64 pairs, four 16-token blocks) once experts average 32
  // or more pairs: a workgroup then expands each weight unit once for 64
  // tokens (the grouped matrix-core path of prefill-sized batches).
  s.cs = (s.P >= 32 * E && f % 64 == 0 && s.fs % 64 == 0) ? 64 : 16;
  s.sub = s.cs / 16;
  s.max_rchunks = (E < s.P ? E : s.P) + s.P / s.cs + 1;
  s.n_schunks = n_shared * ((T + s.cs - 1) / s.cs);
  s.fmax = s.fs > f ? s.fs : f;
  s.bprefix = nullptr;
  s.act_shared = 0;
  return s;
}

FfnLayout make_layout(const FfnShape& s) {
  FfnLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += al256(bytes); return r; };
  const size_t NK = (size_t)s.E * s.B;
  const size_t NC = (size_t)s.max_rchunks + s.n_schunks;
  const size_t NB = NC * s.sub;  // 16-token blocks
  L.pair_key = take((size_t)s.P * 4);
  L.bitmap = take(NK * s.W * 4);
  L.prefix = take(NK * s.W * 4);
  L.colerr = take((size_t)s.W * 4);
  L.keycnt = take(NK * 4);
  L.slot_pair = take((size_t)s.P * 4);
  L.pair_slot = take((size_t)s.P * 4);
  L.slot_info = take((size_t)s.Pt * 4);
  L.chunks = take(NC * 16);
  L.chunk_cnt = take(NC * 4);
  L.meta = take(64);
  L.expert_off = take((size_t)(s.E + 1) * 4);
  L.expert_maxbits = take((size_t)s.E * 4);
  L.xg = take(NB * s.d * 16 * 2);
  L.xvg = take(NB * (s.d / s.g) * 16 * 8);
  L.hg = take(NB * s.fmax * 16 * 2);
  L.hsg = take(NB * (s.fmax / 16) * 16 * 8);
  L.obuf = take((size_t)s.Pt * s.d * 4);
  L.hsgg = take(s.cs == 64 ? NB * (s.fmax / s.g) * 16 * 8 : 0);
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
  const int* chunk_cnt;  // per chunk: pairs of width >= b in byte b-1
  const int* meta;
  int max_rchunks, n_schunks;
  const int* slot_info;
  const uint16_t* act;   // activation fragments [chunk][K/128][4][64][8]
  const float2* asum;    // W13: (X, V) per [chunk][K/g][16]; W2: per [chunk][16][fmax/16]
  int act_stride;        // elements per chunk
  int asum_stride;       // float2 per chunk
  int act_shared;        // gate/up: every chunk reads chunk 0's activations (one token: all chunks hold it)
  uint16_t* hg;          // gate/up output fragments, [chunk][fmax/128][4][64][8]
  float2* hsg;           // gate/up output partial sums [chunk][16][fmax/16]
  float2* hsgg;          // wide chunks: gate/up output group sums [block][fmax/g][16]
  int sub;               // 16-token blocks per chunk
  float* obuf;           // down output [Pt][d]
  const int* bprefix;    // routed bank: per-expert plane prefix (null: every expert stores B planes)
};

// Raw buffer loads (resource flags of gfx9: 32-bit data format, untyped).
constexpr uint32_t BUF_FLAGS = 0x00020000u;
constexpr uint32_t OOB = 0x80000000u;       // lane offset that reads zero
constexpr uint32_t OOB_STEP = 0x40000000u;  // added to every offset of a step past the end (no wrap with OOB)

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

// Width of pair t of a chunk from its counts of pairs of width >= b (pairs
// are sorted by width, widest first); 0 past the chunk's end.
__device__ __forceinline__ int width_of(int cnt, int t) {
  return (t < (cnt & 255)) + (t < ((cnt >> 8) & 255)) + (t < ((cnt >> 16) & 255)) + (t < ((cnt >> 24) & 255));
}

// ---------------------------------------------------------------------------
// Activation gather: one block per (chunk, 128-column k-block).  Token rows
// of the chunk are read (zero rows past its length), scaled by 4^-a (8^-a
// for wide chunks), put in fragment order through LDS and written as 4 KiB
// contiguous; the plain and scaled sums of every quant group go beside them.

struct GatherArgs {
  const uint16_t* x;
  int d, g, sub;
  const int4* chunks;
  const int* meta;
  int max_rchunks;
  const int* slot_info;
  uint16_t* xg;
  float2* xvg;
};

// GKB k-blocks per block, their row loads all issued first: four for 64-pair
// chunks, one for 16-pair chunks (more and smaller blocks)
template <int GKB>
__global__ __launch_bounds__(256) void k_gather(GatherArgs a) {
  const int c = blockIdx.x;  // 16-token block: chunk c / sub, block c % sub of it
  const int kb0 = blockIdx.y * GKB;
  const int nkb = a.d / 128;
  const int kb1 = kb0 + GKB < nkb ? kb0 + GKB : nkb;
  const int ck = c / a.sub;
  // the chunk record is loaded with the routed chunk count, not after it
  // (every record index is inside the chunk array)
  const int nrc = a.meta[0];
  const int4 ch = a.chunks[ck];
  if (ck < a.max_rchunks && ck >= nrc) return;
  const int s0 = ch.y + 16 * (c - ck * a.sub), m = ch.z - 16 * (c - ck * a.sub);
  const int tid = threadIdx.x, t = tid >> 4, q = tid & 15;
  __shared__ uint4 frag[GKB][256];
  uint32_t in[GKB][4];
  const int tok = t < m ? (a.slot_info[s0 + t] & 0xFFFFFF) : 0;
#pragma unroll
  for (int g = 0; g < GKB; ++g) {
    const int kb = kb0 + g;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (t < m && kb < kb1) v = *reinterpret_cast<const uint4*>(a.x + (size_t)tok * a.d + kb * 128 + 8 * q);
    in[g][0] = v.x; in[g][1] = v.y; in[g][2] = v.z; in[g][3] = v.w;
  }
  const int tpg = a.g >> 3;  // threads per quant group
  const int NQG = a.d / a.g;
  // 16-pair chunks: rows past the chunk's pairs are never read (the FFN
  // loads them as out-of-range, i.e. zero), so only live rows are written;
  // 64-pair chunks copy whole blocks and get zero rows.
  const bool live = a.sub > 1 || t < m;
#pragma unroll
  for (int g = 0; g < GKB; ++g) {
    const int kb = kb0 + g;
    if (kb >= kb1) break;
    uint16_t* fr = reinterpret_cast<uint16_t*>(frag[g]);
    float X = 0.f, V = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = 8 * q + j;  // column within the k-block
      const int cc = col & 31;
      const float xf = bf16_to_f32((j & 1) ? (in[g][j >> 1] >> 16) : (in[g][j >> 1] & 0xFFFFu));
      // 4^-a for the plane-unit operands of 16-pair chunks, 8^-a for the
      // nibble operands of 64-pair chunks
      const float sc = a.sub > 1 ? 1.0f / (float)(1 << (3 * a_nib(cc & 15))) : 1.0f / (float)(1 << (2 * a_exp(cc & 15)));
      X += xf;
      V += xf * sc;
      const int fp = frag_pos(cc);
      const int pos = a.sub > 1 ? (col >> 5) * 16 + t : t * 4 + (col >> 5);
      fr[((fp >> 3) * 64 + pos) * 8 + (fp & 7)] = (uint16_t)f32_to_bf16(xf * sc);
    }
    for (int msk = 1; msk < tpg; msk <<= 1) {
      X += __shfl_xor(X, msk, WAVE);
      V += __shfl_xor(V, msk, WAVE);
    }
    if ((q & (tpg - 1)) == 0 && live)
      a.xvg[((size_t)c * NQG + kb * (128 / a.g) + q / tpg) * 16 + t] = make_float2(X, V);
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < GKB; ++g) {
    const int kb = kb0 + g;
    if (kb >= kb1) break;
    if (a.sub > 1 || ((tid & 63) >> 2) < m)
      reinterpret_cast<uint4*>(a.xg + ((size_t)c * nkb + kb) * 2048)[tid] = frag[g][tid];
  }
}

// ---------------------------------------------------------------------------
// Streaming core.
//
// One wave = one work item: a chunk and NT 16-row tiles that share the
// chunk's activations (gate/up: the gate and up tiles of NT/2 row blocks;
// down: NT consecutive tiles).  The wave walks the k-blocks of its tiles
// together: per k-block one plane word per lane, plane and tile, a scale and
// a zero per lane and tile, the token's group sums and 4 x 16 B of
// activation fragment per lane, prefetched PF k-blocks ahead in a register
// ring.  The group-sum terms are applied with the scales already in
// registers (gate/up: every 4/QPK k-blocks; down: per k-block).

constexpr int FFN_THREADS = 256;
#ifndef FFN_WPE
#define FFN_WPE 2  // waves per SIMD the gate/up kernel is compiled for
#endif
#ifndef FFN_W2_WPE
#define FFN_W2_WPE 3  // waves per SIMD of the down kernel (fewer live registers: one k-block ahead)
#endif
#ifndef FFN_W2_PF
#define FFN_W2_PF 1
#endif
// waves per SIMD of each kernel (two-group k-blocks keep two: more registers)
__host__ __device__ constexpr int ffn_wpe(int mode, int qpk) { return (mode == 1 && qpk == 1) ? FFN_W2_WPE : FFN_WPE; }
#ifndef FFN_PF
#define FFN_PF 2   // k-blocks in flight ahead of the one being computed (two-tile steps)
#endif
#ifndef FFN_W13_NT
#define FFN_W13_NT 2  // gate/up tiles per step (gate and up tiles of FFN_W13_NT/2 row blocks)
#endif
#ifndef FFN_W2_NT
#define FFN_W2_NT 2   // down tiles per step
#endif

// The next item's chunk record, loaded while an item streams
// (vector registers, every lane the same) and made scalar once the stream's
// own waits have covered them, before the item's output stores.
struct NextRec {
  u32x4_t ch;
  uint32_t cnt;
};
struct NextVal {
  int e, s0, m, mask, cnt;
};

// First plane and plane count of expert e: uniform banks store B planes per
// expert; a ragged routed bank stores prefix[e+1] - prefix[e] from prefix[e].
__device__ __forceinline__ void expert_planes(const int* bprefix, int B, int e, int& first, int& count) {
  if (bprefix) {
    first = uniform(bprefix[e]);
    count = uniform(bprefix[e + 1]) - first;
  } else {
    first = e * B;
    count = B;
  }
}

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void run_item(const FfnArgs& a, const MatrixDev& M, const int* bprefix, int c, int e,
                                         int s0, int m, int cnt, int item, const NextRec& nr, NextVal& nv) {
  constexpr Units U = make_units(MASK);
  constexpr Classes CL = make_classes(MASK);
  constexpr int BM = mask_bmax(MASK);
  constexpr int NT = (MODE == MODE_W13) ? FFN_W13_NT : FFN_W2_NT;  // tiles per step
  constexpr int NP = NT / 2;                                       // gate/up: tile pairs
  constexpr int PF = (QPK == 2 || CL.n >= 4 || NT > 2) ? 1 : (ffn_wpe(MODE, QPK) > 2 ? FFN_W2_PF : FFN_PF);  // fewer slots where registers are short
  static_assert(NT % 2 == 0, "tiles per step");
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;  // token row of the activation operand; weight row of D
  const int jg = lane >> 4;   // k-chunk of the operands; token quad of D
  int pfirst, B;              // the expert's first plane and stored width
  expert_planes(bprefix, a.B, e, pfirst, B);
  const int K = M.K;
  const int NKB = K >> 7;
  const int NQG = K / a.g;
  const uint32_t plane_bytes = (uint32_t)((size_t)M.N * K / 8);

  // tiles of the item: gate/up -> gate tiles item*NP + p, then the matching
  // up tiles; down -> tiles item*NT + t
  int tile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    tile[t] = (MODE == MODE_W13) ? (t < NP ? item * NP + t : (M.N >> 5) + item * NP + (t - NP)) : item * NT + t;

  // token of the activation row (correction operand)
  float FA = 0.f, ctA = 0.f;
  {
    const int bt = width_of(cnt, r16);
#pragma unroll
    for (int u = 0; u < U.n; ++u)
      if (bt >= U.p[u] + U.np[u]) FA += ldexpf(1.0f, B - 2 - U.p[u]);
    ctA = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;
  }
  // tokens 4jg+i of D: per-class factors (class 0 is read by every pair)
  float fac[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bt = width_of(cnt, 4 * jg + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) fac[k][i] = (k < CL.n && bt >= CL.w[k]) ? 1.0f : 0.0f;
  }
  uint32_t ubias[4];
#pragma unroll
  for (int u = 0; u < U.n; ++u) ubias[u] = vconst(unit_bias(B - 2 - U.p[u]));
  const UnpackConst kc = unpack_const();

  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(M.planes + (size_t)pfirst * (plane_bytes / 4), (uint32_t)B * plane_bytes);
  const uint32_t sz_bytes = (uint32_t)((M.N >> 4) * NQG * 128);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(M.sz + (size_t)e * (sz_bytes / 4), sz_bytes);
  const int ca = (MODE == MODE_W13 && a.act_shared) ? 0 : c;  // chunk whose activations this one reads
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + (size_t)ca * a.act_stride, (uint32_t)K * 32);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.asum + (size_t)ca * a.asum_stride, (uint32_t)a.asum_stride * 8);

  // Per-lane offsets.  Group sums: gate/up reads (X, V) of one group of token
  // r16 in the lanes of that group's k-slot; down reads two of the 16-column
  // partial sums of token r16 per lane (group kb*QPK + (jg & (QPK - 1))).
  // activation rows past the chunk's pairs are zero: their lanes read nothing
  const uint32_t vo_act = r16 < m ? act_pos(MODE, r16, jg) * 16 : OOB;
  const uint32_t vo_pl = lane * 4;
  const uint32_t vo_s = r16 * 4;
  // Gate/up collects the group terms of SPB = 4/QPK k-blocks in the four
  // k-slots of one correction product: k-block j puts its QPK groups in
  // slots (j mod SPB)*QPK + h, i.e. in the lanes jg of that slot.
  constexpr int SPB = 4 / QPK;
  uint32_t vo_x;
  if (MODE == MODE_W13) {
    vo_x = r16 < m ? (uint32_t)((jg % QPK) * 16 + r16) * 8 : OOB;
  } else {
    const int pidx = (QPK == 1) ? 2 * jg : 4 * (jg & 1) + 2 * (jg >> 1);
    vo_x = r16 < m ? (uint32_t)(r16 * (a.fmax >> 4) + pidx) * 8 : OOB;
  }

  struct Ops {
    u32x4_t act[4];
    uint32_t w[NT][BM];
    float s[NT][QPK], z[NT][QPK];
    u32x4_t xs;  // gate/up: (X, V) in .x, .y; down: two (X, V) partials
  };
  uint32_t toff[NT], soff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    toff[t] = (uint32_t)tile[t] * (K / 2) * 4;
    soff[t] = (uint32_t)tile[t] * NQG * 128;
  }
  // Loads of stream step j; past the end every offset is out of range (the
  // loads return zeros and touch no memory), so each step issues the same
  // loads and the wait counts stay exact.
  const int NJ = NKB;
  auto load = [&](int j, Ops& o) {
    const uint32_t oob = (j < NJ) ? 0u : OOB_STEP;
    const uint32_t va = vo_act + oob, vp = vo_pl + oob, vs = vo_s + oob, vx = vo_x + oob;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.act[i] = bld128(ra, va + i * 1024, j * 4096);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < BM; ++p) o.w[t][p] = bld32(rp, vp, toff[t] + j * 256 + p * plane_bytes);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < QPK; ++h) {
        o.s[t][h] = bldf(rs, vs, soff[t] + (j * QPK + h) * 128);
        o.z[t][h] = bldf(rs, vs, soff[t] + (j * QPK + h) * 128 + 64);
      }
    if (MODE == MODE_W13) {
      const float2 v = bld64f(rx, (jg / QPK == j % SPB) ? vx : OOB, j * QPK * 128);
      o.xs = u32x4_t{__float_as_uint(v.x), __float_as_uint(v.y), 0u, 0u};
    } else {
      o.xs = bld128(rx, vx, j * 64);
    }
  };

  f32x4_t out[NT], corr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = corr[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // gate/up: correction operands gathered over SPB k-blocks
  float cAk = 0.f, cAx = 0.f, cBs[NT], cBz[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) cBs[t] = cBz[t] = 0.f;

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
  auto tile_scale = [&](const f32x4_t (&acc)[4][QPK], const float (&s)[QPK], f32x4_t& o) {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[0][h][i];
#pragma unroll
        for (int k = 1; k < CL.n; ++k) v += fac[k][i] * acc[k][h][i];
        o[i] += s[h] * v;
      }
    }
  };
  // Group-sum terms of this k-block's groups: D += K x s - X x (s z), the
  // k-slots of A holding parts of the group sums (down: partial sums of group
  // kb*QPK + (jg & (QPK - 1)) in every slot), so slot jg of B carries the
  // scale of that group.
  auto tile_corr = [&](float Kc, float X, const float (&s)[QPK], const float (&z)[QPK], f32x4_t& cr) {
    const float sb = (QPK == 2 && (jg & 1)) ? s[QPK - 1] : s[0];
    const float zb = (QPK == 2 && (jg & 1)) ? z[QPK - 1] : z[0];
    cr = mfma_f32(Kc, sb, cr);
    cr = mfma_f32(X, -sb * zb, cr);
  };

  // Matrix-core work and the scaling that reads its results are staggered by
  // one tile: tile t's products are scaled after tile t+1's are issued (the
  // step's last tile after the next step's first), so no scaling waits on
  // products issued just before it.  With three or more coverage classes
  // each tile is scaled at once, so only one tile's accumulators are live.
  constexpr bool STAGGER = CL.n < (NT > 2 ? 2 : 3);
  f32x4_t accb[2][4][QPK];
  float sprev[QPK];
#pragma unroll
  for (int h = 0; h < QPK; ++h) {
    sprev[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) accb[1][k][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](const Ops& o, int j) {
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
    float X, V;
    if (MODE == MODE_W13) {
      X = __uint_as_float(o.xs[0]);
      V = __uint_as_float(o.xs[1]);
    } else {
      // two of the group's 16-column partial sums per lane; the k-slot sum
      // of the correction products adds the lanes of a group together
      X = __uint_as_float(o.xs[0]) + __uint_as_float(o.xs[2]);
      V = __uint_as_float(o.xs[1]) + __uint_as_float(o.xs[3]);
    }
    const float Kc = ctA * X - 128.0f * FA * V;
    if (MODE == MODE_W13) {
      // lanes of this k-block's slots take its group terms (the others read zero)
      const bool sel = (jg / QPK) == (j % SPB);
      const int h = jg % QPK;
      cAk += Kc;
      cAx += X;
      if (sel) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          cBs[t] = o.s[t][QPK == 2 ? h : 0];
          cBz[t] = -cBs[t] * o.z[t][QPK == 2 ? h : 0];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (STAGGER) {
        tile_mfma(act, o.w[t], accb[t & 1]);
        // the previous tile: this step's t-1, or the last tile of the previous step
        if (t == 0) {
          tile_scale(accb[1], sprev, out[NT - 1]);
        } else {
          tile_scale(accb[(t - 1) & 1], o.s[t - 1], out[t - 1]);
        }
      } else {
        tile_mfma(act, o.w[t], accb[0]);
        tile_scale(accb[0], o.s[t], out[t]);
      }
    }
    if (STAGGER) {
#pragma unroll
      for (int h = 0; h < QPK; ++h) sprev[h] = o.s[NT - 1][h];
    }
    if (MODE == MODE_W13) {
      if (j % SPB == SPB - 1 || j == NJ - 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          corr[t] = mfma_f32(cAk, cBs[t], corr[t]);
          corr[t] = mfma_f32(cAx, cBz[t], corr[t]);
        }
        cAk = cAx = 0.f;
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) tile_corr(Kc, X, o.s[t], o.z[t], corr[t]);
    }
  };

  // Stream: a main loop of PF+1 unrolled steps (every step issues the loads
  // PF steps ahead into the slot the previous step freed), then the last
  // NJ mod (PF+1) steps, which issue nothing.  The scheduling barriers keep
  // each step's loads together and in step order: loads retire in issue
  // order, so a step's wait then covers its own operands and nothing issued
  // after them.
  Ops o[PF + 1];
#pragma unroll
  for (int q = 0; q < PF; ++q) {
    load(q, o[q]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int j0 = 0;
  for (; j0 + PF + 1 <= NJ; j0 += PF + 1) {
#pragma unroll
    for (int q = 0; q <= PF; ++q) {
      load(j0 + q + PF, o[(q + PF) % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      compute(o[q], j0 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (j0 + q < NJ) compute(o[q], j0 + q);
  if (STAGGER) tile_scale(accb[1], sprev, out[NT - 1]);
  nv.e = uniform((int)nr.ch[0]);
  nv.s0 = uniform((int)nr.ch[1]);
  nv.m = uniform((int)nr.ch[2]);
  nv.mask = uniform((int)nr.ch[3]);
  nv.cnt = uniform((int)nr.cnt);

  if (MODE == MODE_W13) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const f32x4_t res0 = out[p] + corr[p];
      const f32x4_t res1 = out[NP + p] + corr[NP + p];
      // h column n of the down projection's input; tokens 4jg+i
      const int u = item * NP + p;
      const int n = u * 16 + r16;
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
        if (4 * jg + i < m) hrow[(4 * jg + i) * 8] = (uint16_t)f32_to_bf16(hf * ainv);
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
        float2* hs = a.hsg + (size_t)c * a.fmax + u;  // [chunk][token][fmax/16]
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * jg + i < m) hs[(size_t)(4 * jg + i) * (a.fmax >> 4)] = make_float2(Xp[i], Vp[i]);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 4 * jg + i;
      if (tk < m) {
        float* orow = a.obuf + (size_t)(s0 + tk) * a.d;
#pragma unroll
        for (int t = 0; t < NT; ++t) orow[tile[t] * 16 + r16] = out[t][i] + corr[t][i];
      }
    }
  }
}

template <int MODE, int QPK>
__global__ __launch_bounds__(FFN_THREADS) __attribute__((amdgpu_waves_per_eu(ffn_wpe(MODE, QPK), ffn_wpe(MODE, QPK)))) void k_ffn(FfnArgs a) {
  // Blocks are dealt to the 8 XCDs round-robin (block b on XCD b mod 8);
  // each XCD walks one contiguous eighth of the item list, so a chunk's
  // activations are fetched into at most two XCDs' L2 and an XCD streams
  // few experts' planes at a time.  (The mapping only affects where work
  // runs, not what it computes.)  Wave l of an XCD takes items l, l + n,
  // l + 2n, ... of the XCD's range (n waves per XCD).  The next item's chunk
  // record is loaded before the current item streams and read after it.
  const int xcd = blockIdx.x & 7;
  const int lw = uniform((int)(((blockIdx.x >> 3) * blockDim.x + threadIdx.x) >> 6));
  const int nlw = (int)(((gridDim.x >> 3) * blockDim.x) >> 6);
  const int items_r = a.meta[0] * a.items[0];
  const int items = items_r + a.n_schunks * a.items[1];
  const int NC = a.max_rchunks + a.n_schunks;
  const __amdgpu_buffer_rsrc_t rch = make_rsrc(a.chunks, (uint32_t)NC * 16);
  const __amdgpu_buffer_rsrc_t rcn = make_rsrc(a.chunk_cnt, (uint32_t)NC * 4);
  // item w -> chunk, item within the chunk, routed (0) or shared (1)
  auto locate = [&](int w, int& c, int& item, int& sh) {
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
  };
  const MatrixDev m0 = a.m[0], m1 = a.m[1];
  const int w_beg = (int)(((long)items * xcd) >> 3);
  const int w_end = (int)(((long)items * (xcd + 1)) >> 3);
  int w = w_beg + lw;
  if (w >= w_end) return;
  NextVal cur;
  {
    int c, item, sh;
    locate(w, c, item, sh);
    const u32x4_t ch = bld128(rch, 0u, (uint32_t)c * 16);
    cur.cnt = uniform((int)bld32(rcn, 0u, (uint32_t)c * 4));
    cur.e = uniform((int)ch[0]);
    cur.s0 = uniform((int)ch[1]);
    cur.m = uniform((int)ch[2]);
    cur.mask = uniform((int)ch[3]);
  }
  int nxt = w + nlw;
  for (;;) {
    int c, item, sh;
    locate(w, c, item, sh);
    const MatrixDev M = sh ? m1 : m0;
    const bool more = nxt < w_end;
    NextRec nr;
    nr.ch = u32x4_t{0u, 0u, 0u, 0u};
    nr.cnt = 0u;
    if (more) {
      int c2, i2, s2;
      locate(nxt, c2, i2, s2);
      nr.ch = bld128(rch, 0u, (uint32_t)c2 * 16);
      nr.cnt = bld32(rcn, 0u, (uint32_t)c2 * 4);
    }
    NextVal nv;
    switch (cur.mask & 15) {
#define MOE_CASE(MK) \
  case MK:           \
    run_item<MODE, QPK, MK>(a, M, sh ? nullptr : a.bprefix, c, cur.e, cur.s0, cur.m, cur.cnt, item, nr, nv); \
    break;
      MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
      MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14) MOE_CASE(15)
#undef MOE_CASE
      default:
        nv.e = uniform((int)nr.ch[0]);
        nv.s0 = uniform((int)nr.ch[1]);
        nv.m = uniform((int)nr.ch[2]);
        nv.mask = uniform((int)nr.ch[3]);
        nv.cnt = uniform((int)nr.cnt);
        break;
    }
    if (!more) break;
    w = nxt;
    cur = nv;
    nxt += nlw;
  }
}


// ---------------------------------------------------------------------------
// Small batches: k-blocks of an item split over the waves of a workgroup.
//
// When the work items of a call can not fill the chip's waves (a handful of
// tokens: at T = 1 the gate/up step has 8 x 48 items for 2048 wave slots),
// each wave of the whole-K kernel above streams its item's 16 k-blocks as one
// dependent chain.  Here each item gets a workgroup and its k-blocks are cut
// two or four ways; the partial sums meet in LDS.

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void stream_part(const FfnArgs& a, const MatrixDev& M, const int* bprefix, int c, int e,
                                            int m, int cnt, int item, int kb0, int kb1, f32x4_t (&res)[2]) {
  constexpr Units U = make_units(MASK);
  constexpr Classes CL = make_classes(MASK);
  constexpr int BM = mask_bmax(MASK);
  constexpr int NT = 2;
  constexpr int NP = NT / 2;
  constexpr int PF = (QPK == 2 || CL.n >= 4) ? 1 : (ffn_wpe(MODE, QPK) > 2 ? FFN_W2_PF : FFN_PF);
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15;
  const int jg = lane >> 4;
  int pfirst, B;              // the expert's first plane and stored width
  expert_planes(bprefix, a.B, e, pfirst, B);
  const int K = M.K;
  const int NQG = K / a.g;
  const uint32_t plane_bytes = (uint32_t)((size_t)M.N * K / 8);

  int tile[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    tile[t] = (MODE == MODE_W13) ? (t < NP ? item * NP + t : (M.N >> 5) + item * NP + (t - NP)) : item * NT + t;

  float FA = 0.f, ctA = 0.f;
  {
    const int bt = width_of(cnt, r16);
#pragma unroll
    for (int u = 0; u < U.n; ++u)
      if (bt >= U.p[u] + U.np[u]) FA += ldexpf(1.0f, B - 2 - U.p[u]);
    ctA = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;
  }
  float fac[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int bt = width_of(cnt, 4 * jg + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) fac[k][i] = (k < CL.n && bt >= CL.w[k]) ? 1.0f : 0.0f;
  }
  uint32_t ubias[4];
#pragma unroll
  for (int u = 0; u < U.n; ++u) ubias[u] = vconst(unit_bias(B - 2 - U.p[u]));
  const UnpackConst kc = unpack_const();

  const __amdgpu_buffer_rsrc_t rp =
      make_rsrc(M.planes + (size_t)pfirst * (plane_bytes / 4), (uint32_t)B * plane_bytes);
  const uint32_t sz_bytes = (uint32_t)((M.N >> 4) * NQG * 128);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(M.sz + (size_t)e * (sz_bytes / 4), sz_bytes);
  const int ca = (MODE == MODE_W13 && a.act_shared) ? 0 : c;  // chunk whose activations this one reads
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.act + (size_t)ca * a.act_stride, (uint32_t)K * 32);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.asum + (size_t)ca * a.asum_stride, (uint32_t)a.asum_stride * 8);

  const uint32_t vo_act = r16 < m ? act_pos(MODE, r16, jg) * 16 : OOB;
  const uint32_t vo_pl = lane * 4;
  const uint32_t vo_s = r16 * 4;
  constexpr int SPB = 4 / QPK;
  uint32_t vo_x;
  if (MODE == MODE_W13) {
    vo_x = r16 < m ? (uint32_t)((jg % QPK) * 16 + r16) * 8 : OOB;
  } else {
    const int pidx = (QPK == 1) ? 2 * jg : 4 * (jg & 1) + 2 * (jg >> 1);
    vo_x = r16 < m ? (uint32_t)(r16 * (a.fmax >> 4) + pidx) * 8 : OOB;
  }

  struct Ops {
    u32x4_t act[4];
    uint32_t w[NT][BM];
    float s[NT][QPK], z[NT][QPK];
    u32x4_t xs;
  };
  uint32_t toff[NT], soff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    toff[t] = (uint32_t)tile[t] * (K / 2) * 4;
    soff[t] = (uint32_t)tile[t] * NQG * 128;
  }
  // local step j streams k-block kb0 + j; past the range every offset is out of range
  const int NJ = kb1 - kb0;
  auto load = [&](int j, Ops& o) {
    const uint32_t oob = (j < NJ) ? 0u : OOB_STEP;
    const int kb = kb0 + j;
    const uint32_t va = vo_act + oob, vp = vo_pl + oob, vs = vo_s + oob, vx = vo_x + oob;
#pragma unroll
    for (int i = 0; i < 4; ++i) o.act[i] = bld128(ra, va + i * 1024, kb * 4096);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int p = 0; p < BM; ++p) o.w[t][p] = bld32(rp, vp, toff[t] + kb * 256 + p * plane_bytes);
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int h = 0; h < QPK; ++h) {
        o.s[t][h] = bldf(rs, vs, soff[t] + (kb * QPK + h) * 128);
        o.z[t][h] = bldf(rs, vs, soff[t] + (kb * QPK + h) * 128 + 64);
      }
    if (MODE == MODE_W13) {
      const float2 v = bld64f(rx, (jg / QPK == kb % SPB) ? vx : OOB, kb * QPK * 128);
      o.xs = u32x4_t{__float_as_uint(v.x), __float_as_uint(v.y), 0u, 0u};
    } else {
      o.xs = bld128(rx, vx, kb * 64);
    }
  };

  f32x4_t out[NT], corr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) out[t] = corr[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float cAk = 0.f, cAx = 0.f, cBs[NT], cBz[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) cBs[t] = cBz[t] = 0.f;
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
  auto tile_scale = [&](const f32x4_t (&acc)[4][QPK], const float (&s)[QPK], f32x4_t& o) {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = acc[0][h][i];
#pragma unroll
        for (int k = 1; k < CL.n; ++k) v += fac[k][i] * acc[k][h][i];
        o[i] += s[h] * v;
      }
    }
  };
  auto tile_corr = [&](float Kc, float X, const float (&s)[QPK], const float (&z)[QPK], f32x4_t& cr) {
    const float sb = (QPK == 2 && (jg & 1)) ? s[QPK - 1] : s[0];
    const float zb = (QPK == 2 && (jg & 1)) ? z[QPK - 1] : z[0];
    cr = mfma_f32(Kc, sb, cr);
    cr = mfma_f32(X, -sb * zb, cr);
  };

  constexpr bool STAGGER = CL.n < 3;
  f32x4_t accb[2][4][QPK];
  float sprev[QPK];
#pragma unroll
  for (int h = 0; h < QPK; ++h) {
    sprev[h] = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) accb[1][k][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](const Ops& o, int j) {
    const int kb = kb0 + j;
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
    float X, V;
    if (MODE == MODE_W13) {
      X = __uint_as_float(o.xs[0]);
      V = __uint_as_float(o.xs[1]);
    } else {
      X = __uint_as_float(o.xs[0]) + __uint_as_float(o.xs[2]);
      V = __uint_as_float(o.xs[1]) + __uint_as_float(o.xs[3]);
    }
    const float Kc = ctA * X - 128.0f * FA * V;
    if (MODE == MODE_W13) {
      const bool sel = (jg / QPK) == (kb % SPB);
      const int h = jg % QPK;
      cAk += Kc;
      cAx += X;
      if (sel) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          cBs[t] = o.s[t][QPK == 2 ? h : 0];
          cBz[t] = -cBs[t] * o.z[t][QPK == 2 ? h : 0];
        }
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (STAGGER) {
        tile_mfma(act, o.w[t], accb[t & 1]);
        if (t == 0) {
          tile_scale(accb[1], sprev, out[NT - 1]);
        } else {
          tile_scale(accb[(t - 1) & 1], o.s[t - 1], out[t - 1]);
        }
      } else {
        tile_mfma(act, o.w[t], accb[0]);
        tile_scale(accb[0], o.s[t], out[t]);
      }
    }
    if (STAGGER) {
#pragma unroll
      for (int h = 0; h < QPK; ++h) sprev[h] = o.s[NT - 1][h];
    }
    if (MODE == MODE_W13) {
      if (kb % SPB == SPB - 1 || j == NJ - 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          corr[t] = mfma_f32(cAk, cBs[t], corr[t]);
          corr[t] = mfma_f32(cAx, cBz[t], corr[t]);
        }
        cAk = cAx = 0.f;
      }
    } else {
#pragma unroll
      for (int t = 0; t < NT; ++t) tile_corr(Kc, X, o.s[t], o.z[t], corr[t]);
    }
  };

  Ops o[PF + 1];
#pragma unroll
  for (int q = 0; q < PF; ++q) {
    load(q, o[q]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int j0 = 0;
  for (; j0 + PF + 1 <= NJ; j0 += PF + 1) {
#pragma unroll
    for (int q = 0; q <= PF; ++q) {
      load(j0 + q + PF, o[(q + PF) % (PF + 1)]);
      __builtin_amdgcn_sched_barrier(0);
      compute(o[q], j0 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int q = 0; q < PF; ++q)
    if (j0 + q < NJ) compute(o[q], j0 + q);
  if (STAGGER) tile_scale(accb[1], sprev, out[NT - 1]);
#pragma unroll
  for (int t = 0; t < NT; ++t) res[t] = out[t] + corr[t];
}


// Finish an item from its full sum (out + corr over every k-block): gate/up
// -> SwiGLU, bf16 h in the down projection's fragment order and its 16-column
// partial sums; down -> the per-slot output rows.
template <int MODE>
__device__ __forceinline__ void sk_finish(const FfnArgs& a, const f32x4_t (&res)[2], int c, int item, int s0, int m) {
  const int lane = threadIdx.x & 63;
  const int r16 = lane & 15, jg = lane >> 4;
  if (MODE == MODE_W13) {
    const int u = item;  // row block of 16 h columns
    const int n = u * 16 + r16;
    const int cc = n & 31;
    const int fp = frag_pos(cc);
    const float ainv = 1.0f / (float)(1 << (2 * a_exp(cc & 15)));
    uint16_t* hrow = a.hg + (size_t)c * a.fmax * 16 +
                     ((size_t)((n >> 7) * 4 + (fp >> 3)) * 64 + ((n & 127) >> 5) * 16) * 8 + (fp & 7);
    float Xp[4], Vp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float gval = res[0][i];
      const float hval = gval / (1.0f + expf(-gval)) * res[1][i];
      const float hf = bf16_to_f32(f32_to_bf16(hval));
      if (4 * jg + i < m) hrow[(4 * jg + i) * 8] = (uint16_t)f32_to_bf16(hf * ainv);
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
      float2* hs = a.hsg + (size_t)c * a.fmax + u;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * jg + i < m) hs[(size_t)(4 * jg + i) * (a.fmax >> 4)] = make_float2(Xp[i], Vp[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tk = 4 * jg + i;
      if (tk < m) {
        float* orow = a.obuf + (size_t)(s0 + tk) * a.d;
        orow[(item * 2) * 16 + r16] = res[0][i];
        orow[(item * 2 + 1) * 16 + r16] = res[1][i];
      }
    }
  }
}

// An item's place: chunk, item within it, bank, and its chunk record.
struct SkItem {
  int c, item, sh, e, s0, m, mask, cnt, nkb;
};

__device__ __forceinline__ SkItem sk_item(const FfnArgs& a, int it) {
  SkItem r;
  const int items_r = a.meta[0] * a.items[0];
  if (it < items_r) {
    r.c = it / a.items[0];
    r.item = it - r.c * a.items[0];
    r.sh = 0;
  } else {
    const int w2 = it - items_r;
    const int cs = w2 / a.items[1];
    r.item = w2 - cs * a.items[1];
    r.c = a.max_rchunks + cs;
    r.sh = 1;
  }
  r.c = uniform(r.c);
  r.item = uniform(r.item);
  r.sh = uniform(r.sh);
  const int4 ch = a.chunks[r.c];
  r.e = uniform(ch.x);
  r.s0 = uniform(ch.y);
  r.m = uniform(ch.z);
  r.mask = uniform(ch.w) & 15;
  r.cnt = uniform(a.chunk_cnt[r.c]);
  r.nkb = (r.sh ? a.m[1].K : a.m[0].K) >> 7;
  return r;
}

template <int MODE, int QPK>
__device__ __forceinline__ void sk_stream(const FfnArgs& a, const SkItem& it, int kb0, int kb1, f32x4_t (&res)[2]) {
  const MatrixDev M = it.sh ? a.m[1] : a.m[0];
  switch (it.mask) {
#define MOE_CASE(MK) \
  case MK:           \
    stream_part<MODE, QPK, MK>(a, M, it.sh ? nullptr : a.bprefix, it.c, it.e, it.m, it.cnt, it.item, kb0, kb1, res); \
    break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
    MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14) MOE_CASE(15)
#undef MOE_CASE
    default:
      res[0] = res[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      break;
  }
}

// One item per workgroup, its k-blocks split over the KS_WAVES waves (wave q
// streams k-blocks [q K/KS_WAVES, (q+1) K/KS_WAVES) of the item); wave 0 adds
// the partial sums from LDS in wave order and finishes the item.  Workgroup b
// takes item b (an XCD-aware order keeps a chunk's items on one XCD); the
// items past the call's routed chunks leave at once.
template <int MODE, int QPK, int KS_WAVES>
__global__ __launch_bounds__(64 * KS_WAVES) __attribute__((amdgpu_waves_per_eu(ffn_wpe(MODE, QPK), ffn_wpe(MODE, QPK)))) void k_ffn_small(FfnArgs a) {
  __shared__ f32x4_t part[KS_WAVES][2][64];
  const int wave = uniform((int)(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  const int nwg = gridDim.x;
  const int it = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int items = a.meta[0] * a.items[0] + a.n_schunks * a.items[1];
  if (it >= items) return;  // the whole workgroup leaves together
  const SkItem x = sk_item(a, it);
  const int kb0 = uniform(wave * x.nkb / KS_WAVES), kb1 = uniform((wave + 1) * x.nkb / KS_WAVES);
  f32x4_t res[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
  if (kb0 < kb1) sk_stream<MODE, QPK>(a, x, kb0, kb1, res);
  part[wave][0][lane] = res[0];
  part[wave][1][lane] = res[1];
  __syncthreads();
  if (wave == 0) {
    f32x4_t acc[2] = {part[0][0][lane], part[0][1][lane]};
#pragma unroll
    for (int q = 1; q < KS_WAVES; ++q) {
      acc[0] += part[q][0][lane];
      acc[1] += part[q][1][lane];
    }
    sk_finish<MODE>(a, acc, x.c, x.item, x.s0, x.m);
  }
}

// ---------------------------------------------------------------------------
// Wide chunks (prefill-sized batches): one workgroup of 4 waves per item, an
// item being a chunk of <= 64 pairs (four 16-token blocks) and 4 row blocks
// (gate/up: the gate and up tile of row blocks 4i..4i+3, one per wave; down:
// tiles 8i..8i+7, two per wave).  Per 128-column k-block the activation
// fragments of the four token blocks (16 KiB) are copied into LDS once by
// DMA and read by all four waves.  Each wave expands its tiles' planes once
// per k-block into nibble operands (all planes at once, see `unpack_nib`;
// the chunk's narrower widths by one AND per word) and runs, per token
// block, one matrix-core pass per width that block holds: pairs are sorted
// by width, so most blocks hold one width and take one pass.  Double-
// buffered: the copies and weight loads of k-block kb+1 run while kb is
// computed.

constexpr int WIDE_THREADS = 256;
// LDS dwords per ring stage of the weights: per wave, two tiles' plane words
// (64 per plane, up to four planes), then the tiles' scales and zeros of the
// k-block's quant group (16 rows each)
constexpr int WIDE_PL_STAGE = 4 * (2 * 256 + 64);

template <int MODE, int QPK, int MASK>
__device__ __forceinline__ void run_wide(const FfnArgs& a, const MatrixDev& M, const int* bprefix, int c, int e,
                                         int s0, int m, int cnt, int item, uint4* lds, float2* xsl, uint32_t* plds) {
  constexpr int BM = mask_bmax(MASK);
  constexpr int NB = 4;  // token blocks
  // tiles whose operands are live at once: both when the chunk holds at most
  // two widths (each block's activations then serve both), else one
  constexpr int TP = (((MASK & 1) + ((MASK >> 1) & 1) + ((MASK >> 2) & 1) + ((MASK >> 3) & 1)) <= 2) ? 2 : 1;
  const int lane = threadIdx.x & 63;
  const int wave = uniform((int)(threadIdx.x >> 6));  // wave-uniform: scalar resources and LDS bases
  const int r16 = lane & 15, jg = lane >> 4;
  int pfirst, B;              // the expert's first plane and stored width
  expert_planes(bprefix, a.B, e, pfirst, B);
  const int K = M.K;
  const int NKB = K >> 7;
  const int NQG = K / a.g;
  const uint32_t plane_bytes = (uint32_t)((size_t)M.N * K / 8);
  const int tile0 = (MODE == MODE_W13) ? item * 4 + wave : item * 8 + 2 * wave;
  const int tile1 = (MODE == MODE_W13) ? (M.N >> 5) + item * 4 + wave : item * 8 + 2 * wave + 1;

  // per token block: correction weights of the A-view token r16 (one pass of
  // factor 2^(B-4) for a live pair), its width, and the widths the block
  // holds (bit b-1).  c_b = pairs of width >= b; pairs are sorted widest
  // first.
  float FA[NB], ctA[NB];
  uint32_t wda = 0u;  // A-view token widths, nibble b
  int pres = 0;       // 4 bits per block
  const float f_unit = ldexpf(1.0f, B - 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int bt = width_of(cnt, 16 * b + r16);
    FA[b] = bt > 0 ? f_unit : 0.f;
    ctA[b] = bt > 0 ? 0.5f * (ldexpf(1.0f, B - bt) - 1.0f) : 0.f;
    wda |= (uint32_t)bt << (4 * b);
    int pr = 0;
#pragma unroll
    for (int w = 1; w <= 4; ++w) {
      const int cw = (cnt >> (8 * (w - 1))) & 255;
      const int cw1 = w < 4 ? (cnt >> (8 * w)) & 255 : 0;
      const int lo = cw1 > 16 * b ? cw1 : 16 * b;
      const int hi = cw < 16 * b + 16 ? cw : 16 * b + 16;
      if (lo < hi) pr |= 1 << (w - 1);
    }
    pres |= (pr & MASK) << (4 * b);
  }
  pres = uniform(pres);
  const uint32_t ubias = vconst(unit_bias(B - 4));
  NibConst nk = nib_const_plain();
  nk.e2 = vconst(nk.e2);
  nk.e4 = vconst(nk.e4);
  nk.f0 = vconst(nk.f0);
  nk.f3 = vconst(nk.f3);

  const uint32_t sz_bytes = (uint32_t)((M.N >> 4) * NQG * 128);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(M.sz + (size_t)e * (sz_bytes / 4), sz_bytes);
  const uint16_t* actc = a.act + (size_t)c * NB * a.act_stride;

  constexpr int SPB = 4 / QPK;
  const uint32_t vo_s = r16 * 4;
  const uint32_t t0off = (uint32_t)tile0 * (K / 2) * 4, t1off = (uint32_t)tile1 * (K / 2) * 4;
  const uint32_t s0off = (uint32_t)tile0 * NQG * 128, s1off = (uint32_t)tile1 * NQG * 128;

  // plane words of the wave's two tiles at k-block kb -> LDS (one dword per
  // lane, plane and tile); scales and zeros into registers
  // (buffer loads into LDS: a constant lane offset and a scalar step offset,
  // so the per-step addressing is scalar work)
  typedef __attribute__((address_space(3))) void* lds_ptr;
  const __amdgpu_buffer_rsrc_t rpl =
      make_rsrc(M.planes + (size_t)pfirst * (plane_bytes / 4), (uint32_t)B * plane_bytes);
  auto copy_planes = [&](int kb, uint32_t* pst) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int p = 0; p < BM; ++p)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rpl, (lds_ptr)(pst + (wave * 2 + t) * 256 + p * 64), 4,
                                                 lane * 4, (t ? t1off : t0off) + kb * 256 + p * plane_bytes, 0, 0);
  };
  struct Wts {
    float s[2][QPK], z[2][QPK];
  };
  auto load_w = [&](int kb, Wts& o) {
#pragma unroll
    for (int h = 0; h < QPK; ++h) {
      o.s[0][h] = bldf(rs, vo_s, s0off + (kb * QPK + h) * 128);
      o.z[0][h] = bldf(rs, vo_s, s0off + (kb * QPK + h) * 128 + 64);
      o.s[1][h] = bldf(rs, vo_s, s1off + (kb * QPK + h) * 128);
      o.z[1][h] = bldf(rs, vo_s, s1off + (kb * QPK + h) * 128 + 64);
    }
  };
  // group sums (X, V) of k-block kb's groups -> LDS: wave w copies those of
  // token block w (16 QPK float2, one dword per lane)
  // (lanes past the 16 QPK float2 copy what follows them, never read)
  const __amdgpu_buffer_rsrc_t rxs =
      make_rsrc(a.asum + (size_t)(c * NB + wave) * a.asum_stride, (uint32_t)a.asum_stride * 8);
  auto copy_xs = [&](int kb, float2* xst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rxs, (lds_ptr)(xst + wave * 32), 4, lane * 4, kb * QPK * 128, 0, 0);
  };
  // activation fragments of k-block kb for the four token blocks -> LDS
  // buffer: wave w copies token block w, 4 x 1 KiB
  const __amdgpu_buffer_rsrc_t ract = make_rsrc(actc + (size_t)wave * a.act_stride, (uint32_t)a.act_stride * 2);
  auto copy_act = [&](int kb, uint4* ast) {
    uint4* dst = ast + (size_t)wave * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ract, (lds_ptr)(dst + i * 64), 16, lane * 16, kb * 4096 + i * 1024, 0, 0);
  };

  f32x4_t out[2][NB];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) out[t][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float cAk[NB], cAx[NB], cBs[2], cBz[2];
#pragma unroll
  for (int b = 0; b < NB; ++b) cAk[b] = cAx[b] = 0.f;
  cBs[0] = cBs[1] = cBz[0] = cBz[1] = 0.f;
  const uint32_t hmask0 = (QPK == 2 && (jg >> 1) != 0) ? 0u : 0xFFFFFFFFu;
  const uint32_t hmask1 = (QPK == 2 && (jg >> 1) != 1) ? 0u : 0xFFFFFFFFu;

  // One quant group per k-block: the tiles' scales and zeros also travel
  // through LDS, one copy per k-block (lanes 0..31 the 16 scales and 16 zeros
  // of the first tile, lanes 32..63 those of the second), so no stage of the
  // ring holds registers that a later wait would have to cover.
  constexpr bool SZ_LDS = (QPK == 1);
  const uint32_t vo_w = (lane < 32 ? s0off : s1off) + (uint32_t)(lane & 31) * 4;
  auto copy_w = [&](int kb, uint32_t* pst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(pst + 4 * 2 * 256 + wave * 64), 4, vo_w, kb * 128, 0, 0);
  };
  // A k-block's small operands (scales and zeros, group sums, plane words),
  // read from LDS right after the step's barrier, before the next stage's
  // copies are issued, so that no read of them waits for those copies.
  struct Small {
    float s[2], z[2];
    float2 xv[NB];
    uint32_t pw[2][4];
  };
  auto load_small = [&](const float2* xst, const uint32_t* pst, Small& sm) {
    if (SZ_LDS) {
      const float* sc = reinterpret_cast<const float*>(pst + 4 * 2 * 256) + wave * 64;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        sm.s[t] = sc[(t * 2 + 0) * 16 + r16];
        sm.z[t] = sc[(t * 2 + 1) * 16 + r16];
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) sm.xv[b] = xst[b * 32 + (jg % QPK) * 16 + r16];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const uint32_t* pw = pst + (wave * 2 + t) * 256 + lane;
#pragma unroll
      for (int p = 0; p < 4; ++p) sm.pw[t][p] = p < BM ? pw[p * 64] : 0u;
    }
  };
  auto compute = [&](const Wts& o_reg, int kb, const uint4* ast, const Small& sm) {
    Wts o = o_reg;
    if (SZ_LDS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        o.s[t][0] = sm.s[t];
        o.z[t][0] = sm.z[t];
      }
    }
    // the blocks' widths, re-read per k-block so that the branch conditions
    // derived from them are not kept live (as lane masks) across the stream
    int presk = pres;
    asm volatile("" : "+s"(presk));
    // group terms of this k-block
    const bool sel = (jg / QPK) == (kb % SPB);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float2 xv = sm.xv[b];
      const float X = sel ? xv.x : 0.f, V = sel ? xv.y : 0.f;
      cAk[b] += ctA[b] * X - 128.0f * FA[b] * V;
      cAx[b] += X;
    }
    if (sel) {
      const int h = jg % QPK;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        cBs[t] = o.s[t][QPK == 2 ? h : 0];
        cBz[t] = -cBs[t] * o.z[t][QPK == 2 ? h : 0];
      }
    }
#pragma unroll
    for (int t0 = 0; t0 < 2; t0 += TP) {
    // operands of every width the chunk holds, for the TP tiles of this
    // pass: the widest from the planes, the narrower ones by clearing field
    // bits
    u32x4_t W[TP][4][4];
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const uint32_t n3 = sm.pw[t0 + t][0];
      const uint32_t n2 = sm.pw[t0 + t][1];
      const uint32_t n1 = sm.pw[t0 + t][2];
      const uint32_t n0 = sm.pw[t0 + t][3];
      unpack_nib(n3, n2, n1, n0, ubias, nk, W[t][BM - 1]);
      if (MASK & ((1 << (BM - 1)) - 1)) {
        // keep each widest word one AND-OR (re-associating it with the
        // narrower widths' ANDs costs an extra operation per word)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) W[t][BM - 1][i][r] = vconst(W[t][BM - 1][i][r]);
      }
#pragma unroll
      for (int w = 1; w < BM; ++w)
        if (MASK & (1 << (w - 1))) {
#pragma unroll
          for (int i = 0; i < 4; ++i) W[t][w - 1][i] = W[t][BM - 1][i] & nib_width_mask(w, i);
        }
    }
    // One uniform branch per token block: a block of one width w runs one
    // pass per tile on the width-w operands; a block holding several widths
    // runs one pass per width with the activation rows of the other widths
    // cleared.  Each branch scales its own products (no accumulator is
    // carried across branches); the tiles' chains are interleaved.  The
    // block's activations are read from LDS once for the TP tiles, the next
    // block's (double-buffered by block parity) while this one runs.
    u32x4_t av[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) av[0][i] = as_u32x4(ast[lane + i * 64]);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int cb = b & 1;
      if (b + 1 < NB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) av[cb ^ 1][i] = as_u32x4(ast[(size_t)(b + 1) * 256 + lane + i * 64]);
      }
      const int pb = (presk >> (4 * b)) & 15;
#pragma unroll
      for (int w = 4; w >= 1; --w) {
        if (!(MASK & (1 << (w - 1)))) continue;
        if (pb != (1 << (w - 1))) continue;  // uniform: the block holds width w only
        f32x4_t acc[TP][QPK];
#pragma unroll
        for (int t = 0; t < TP; ++t)
#pragma unroll
          for (int h = 0; h < QPK; ++h) acc[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int t = 0; t < TP; ++t) {
            acc[t][0] = mfma_bf16(as_bf16x8(QPK == 1 ? av[cb][i] : (av[cb][i] & hmask0)), as_bf16x8(W[t][w - 1][i]), acc[t][0]);
            if (QPK == 2) acc[t][QPK - 1] = mfma_bf16(as_bf16x8(av[cb][i] & hmask1), as_bf16x8(W[t][w - 1][i]), acc[t][QPK - 1]);
          }
#pragma unroll
        for (int t = 0; t < TP; ++t)
#pragma unroll
          for (int h = 0; h < QPK; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) out[t0 + t][b][i] += o.s[t0 + t][h] * acc[t][h][i];
      }
      if (pb & (pb - 1)) {  // uniform: several widths
        f32x4_t acc[TP][QPK];
#pragma unroll
        for (int t = 0; t < TP; ++t)
#pragma unroll
          for (int h = 0; h < QPK; ++h) acc[t][h] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        // the widths are re-read here so that their comparisons are not
        // kept live across the stream
        const uint32_t wa = (vconst(wda) >> (4 * b)) & 15u;
#pragma unroll
        for (int w = 4; w >= 1; --w) {
          if (!(MASK & (1 << (w - 1)))) continue;
          if (!(pb & (1 << (w - 1)))) continue;
          const uint32_t am = wa == (uint32_t)w ? 0xFFFFFFFFu : 0u;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4_t x0 = av[cb][i] & (am & hmask0);
            const u32x4_t x1 = av[cb][i] & (am & hmask1);
#pragma unroll
            for (int t = 0; t < TP; ++t) {
              acc[t][0] = mfma_bf16(as_bf16x8(x0), as_bf16x8(W[t][w - 1][i]), acc[t][0]);
              if (QPK == 2) acc[t][QPK - 1] = mfma_bf16(as_bf16x8(x1), as_bf16x8(W[t][w - 1][i]), acc[t][QPK - 1]);
            }
          }
        }
#pragma unroll
        for (int t = 0; t < TP; ++t)
#pragma unroll
          for (int h = 0; h < QPK; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) out[t0 + t][b][i] += o.s[t0 + t][h] * acc[t][h][i];
      }
    }
    }
    if (kb % SPB == SPB - 1 || kb == NKB - 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          out[t][b] = mfma_f32(cAk[b], cBs[t], out[t][b]);
          out[t][b] = mfma_f32(cAx[b], cBz[t], out[t][b]);
        }
#pragma unroll
      for (int b = 0; b < NB; ++b) cAk[b] = cAx[b] = 0.f;
    }
  };

  // Three-stage ring: k-block kb+2's copies and weight loads are issued
  // once every wave has passed k-block kb's barrier (so its LDS buffers,
  // last read at kb-1, are free) and run while kb and kb+1 are computed.
  // Every stage issues the same NS vector loads and they retire in issue
  // order, so waiting for all but the newest NS leaves exactly stage kb+1 in
  // flight.  A step takes the buffers of the stage it computes and of the
  // stage it fills as distinct restrict pointers: the LDS reads of one are
  // then known not to alias the copies into the other, and wait only for
  // their own stage (with one buffer array the compiler made every read wait
  // for the copies just issued).
  constexpr int NS = 4 + 1 + 2 * BM + (SZ_LDS ? 1 : 4 * QPK);  // activation and group-sum copies, plane copies, scales and zeros
  Wts wr[3] = {};
  auto stage_a = [&](int st) { return lds + (size_t)st * NB * 256; };
  auto stage_x = [&](int st) { return xsl + st * NB * 32; };
  auto stage_p = [&](int st) { return plds + st * WIDE_PL_STAGE; };
  auto step = [&](int kb, const Wts& wcur, Wts& wnxt, const uint4* __restrict__ acur, const float2* __restrict__ xcur,
                  const uint32_t* __restrict__ pcur, uint4* __restrict__ anxt, float2* __restrict__ xnxt,
                  uint32_t* __restrict__ pnxt) {
    if (kb + 1 < NKB)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(NS));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // A plain barrier, without __syncthreads' release fence: that fence waits
    // for every copy still in flight (stage kb+1 too).  Each wave has waited
    // for its own copies of stage kb above, and has consumed its reads of
    // stage kb-1 (the one refilled next) before arriving; the empty asm
    // statements keep the compiler's memory accesses on their side.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    Small sm;
    load_small(xcur, pcur, sm);
    if (kb + 2 < NKB) {
      copy_act(kb + 2, anxt);
      copy_xs(kb + 2, xnxt);
      copy_planes(kb + 2, pnxt);
      if (SZ_LDS) copy_w(kb + 2, pnxt); else load_w(kb + 2, wnxt);
    }
    compute(wcur, kb, acur, sm);
  };
  // the first two stages' copies (restrict pointers too, so that the reads
  // of the first steps know which copies they wait for)
  auto prime = [&](int kb, uint4* __restrict__ an, float2* __restrict__ xn, uint32_t* __restrict__ pn, Wts& wn) {
    copy_act(kb, an);
    copy_xs(kb, xn);
    copy_planes(kb, pn);
    if (SZ_LDS) copy_w(kb, pn); else load_w(kb, wn);
  };
  prime(0, stage_a(0), stage_x(0), stage_p(0), wr[0]);
  if (NKB > 1) prime(1, stage_a(1), stage_x(1), stage_p(1), wr[1]);
  // both first stages in before the loop: no copy of the prologue is left in
  // flight at the loop's head, where the compiler would otherwise make the
  // loop's reads wait for every copy on every pass
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  // one call site of the step, unrolled three ways, so every pass carries the
  // same alias information
  for (int kb0 = 0; kb0 < NKB; kb0 += 3) {
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int nq = (q + 2) % 3;
      if (kb0 + q < NKB)
        step(kb0 + q, wr[q], wr[nq], stage_a(q), stage_x(q), stage_p(q), stage_a(nq), stage_x(nq), stage_p(nq));
    }
  }

  // epilogue per token block
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int bid = c * NB + b;
    if (MODE == MODE_W13) {
      const int u = item * 4 + wave;   // row block = 16 h columns
      const int n = u * 16 + r16;
      const int cc = n & 31;
      const int fp = frag_pos(cc);
      const float ainv = 1.0f / (float)(1 << (3 * a_nib(cc & 15)));
      uint16_t* hrow = a.hg + (size_t)bid * a.fmax * 16 +
                       ((size_t)((n >> 7) * 4 + (fp >> 3)) * 64 + ((n & 127) >> 5) * 16) * 8 + (fp & 7);
      float Xp[4], Vp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float gval = out[0][b][i];
        const float hval = gval / (1.0f + expf(-gval)) * out[1][b][i];
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
        float2* hs = a.hsg + (size_t)bid * a.fmax + u;  // [block][token][fmax/16]
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[(size_t)(4 * jg + i) * (a.fmax >> 4)] = make_float2(Xp[i], Vp[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tk = 16 * b + 4 * jg + i;
        if (tk < m) {
          float* orow = a.obuf + (size_t)(s0 + tk) * a.d;
          orow[tile0 * 16 + r16] = out[0][b][i];
          orow[tile1 * 16 + r16] = out[1][b][i];
        }
      }
    }
  }
}

template <int MODE, int QPK>
__global__ __launch_bounds__(WIDE_THREADS) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_wide(FfnArgs a) {
  __shared__ uint4 lds[3 * 4 * 256];   // three k-blocks x four token blocks x 4 KiB
  __shared__ float2 xsl[3 * 4 * 32];   // their group sums
  __shared__ uint32_t plds[3 * WIDE_PL_STAGE];  // per k-block and wave: 64 words per tile and plane, then 64 scales and zeros
  // Workgroup b runs on XCD b mod 8 and takes item (b / 8) of that XCD's
  // contiguous eighth of the call's items: the items of one chunk (which
  // share its activations) and the chunks of one expert (which share its
  // weights) then run at the same time on one XCD and meet in its L2.
  const int n_rc = a.meta[0];
  const int items_r = n_rc * a.items[0];
  const int items = items_r + a.n_schunks * a.items[1];
  const int xcd = blockIdx.x & 7;
  const int w = (int)(((long)items * xcd) >> 3) + (int)(blockIdx.x >> 3);
  if (w >= (int)(((long)items * (xcd + 1)) >> 3)) return;
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
  const int cnt = uniform(a.chunk_cnt[c]);
  const MatrixDev& M = a.m[sh];
  switch (ch.w & 15) {
#define MOE_CASE(MK) \
  case MK:           \
    run_wide<MODE, QPK, MK>(a, M, sh ? nullptr : a.bprefix, c, ch.x, ch.y, ch.z, cnt, item, lds, xsl, plds); \
    break;
    MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7) MOE_CASE(8)
    MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13) MOE_CASE(14) MOE_CASE(15)
#undef MOE_CASE
    default:
      break;
  }
}

// Wide chunks: group sums of the gate/up output per 16-token block, token
// and quant group of the down projection's input, from the 16-column
// partial sums.  One thread per (block, group, token).
__global__ __launch_bounds__(256) void k_hsum(const FfnArgs a, int nblocks, int ngroups) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks * ngroups * 16) return;
  const int t = i & 15, G = (i >> 4) % ngroups, bid = (i >> 4) / ngroups;
  const int tpg = a.g >> 4;
  const float2* src = a.hsg + (size_t)bid * a.fmax + (size_t)t * (a.fmax >> 4) + G * tpg;
  float X = 0.f, V = 0.f;
  for (int p = 0; p < tpg; ++p) {
    X += src[p].x;
    V += src[p].y;
  }
  a.hsgg[((size_t)bid * (a.fmax / a.g) + G) * 16 + t] = make_float2(X, V);
}

// ---------------------------------------------------------------------------
// combine: y[t] = (acc ? y[t] : 0) + sum_j gate[t][j] o_(t,j) + sum_s o_(t,shared s)

// top_k <= 8 (checked at the boundary): all slots and gates are loaded
// first, then all rows, then added in pair order, so the loads take one
// round trip each instead of one per pair.
constexpr int CMB_KMAX = 8;

__global__ __launch_bounds__(256) void k_combine(int T, int k, int d, int P, int n_shared,
                                                 const int* __restrict__ pair_slot, const float* __restrict__ gate,
                                                 const float* __restrict__ obuf, float* __restrict__ y,
                                                 int accumulate) {
  const int t = blockIdx.y;
  const int n4 = blockIdx.x * blockDim.x + threadIdx.x;
  if (n4 * 4 >= d) return;
  float4 v = accumulate ? reinterpret_cast<const float4*>(y + (size_t)t * d)[n4] : make_float4(0.f, 0.f, 0.f, 0.f);
  int sl[CMB_KMAX];
  float gt[CMB_KMAX];
#pragma unroll
  for (int j = 0; j < CMB_KMAX; ++j) {
    sl[j] = j < k ? pair_slot[t * k + j] : -1;
    gt[j] = j < k ? gate[t * k + j] : 0.f;
  }
  float4 o[CMB_KMAX];
#pragma unroll
  for (int j = 0; j < CMB_KMAX; ++j)
    o[j] = sl[j] >= 0 ? reinterpret_cast<const float4*>(obuf + (size_t)sl[j] * d)[n4] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int j = 0; j < CMB_KMAX; ++j) {
    if (sl[j] < 0) continue;
    v.x += gt[j] * o[j].x; v.y += gt[j] * o[j].y; v.z += gt[j] * o[j].z; v.w += gt[j] * o[j].w;
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
  a.chunk_cnt = reinterpret_cast<const int*>(ws + L.chunk_cnt);
  a.meta = reinterpret_cast<const int*>(ws + L.meta);
  a.max_rchunks = s.max_rchunks;
  a.n_schunks = s.n_schunks;
  a.slot_info = reinterpret_cast<const int*>(ws + L.slot_info);
  a.hg = reinterpret_cast<uint16_t*>(ws + L.hg);
  a.hsg = reinterpret_cast<float2*>(ws + L.hsg);
  a.obuf = reinterpret_cast<float*>(ws + L.obuf);
  a.hsgg = reinterpret_cast<float2*>(ws + L.hsgg);
  a.sub = s.sub;
  a.bprefix = s.bprefix;
  a.act_shared = s.act_shared;
  return a;
}

hipError_t launch_ffn(int mode, const FfnShape& s, const FfnLayout& L, char* ws, MatrixDev routed, MatrixDev shared,
                      int num_cu, hipStream_t stream) {
  FfnArgs a = make_args(s, L, ws, routed, shared);
  // work items per chunk: gate/up -> f/16 tile pairs, down -> d/32 tile pairs
  if (mode == MODE_W13) {
    a.items[0] = s.f / (8 * FFN_W13_NT);
    a.items[1] = s.n_shared ? s.fs / (8 * FFN_W13_NT) : 1;
    a.act = reinterpret_cast<const uint16_t*>(ws + L.xg);
    a.act_stride = s.d * 16;
    a.asum = reinterpret_cast<const float2*>(ws + L.xvg);
    a.asum_stride = (s.d / s.g) * 16;
  } else {
    a.items[0] = s.d / (16 * FFN_W2_NT);
    a.items[1] = s.d / (16 * FFN_W2_NT);
    a.act = reinterpret_cast<const uint16_t*>(ws + L.hg);
    a.act_stride = s.fmax * 16;
    a.asum = reinterpret_cast<const float2*>(ws + L.hsg);
    a.asum_stride = (s.fmax / 16) * 16;
  }
  const int qpk = (s.g == 64) ? 2 : 1;
  if (s.cs == 64) {
    // wide chunks: 4 row blocks (gate/up) or 8 tiles (down) per workgroup
    if (mode == MODE_W13) {
      a.items[0] = s.f / 64;
      a.items[1] = s.n_shared ? s.fs / 64 : 1;
    } else {
      a.items[0] = s.d / 128;
      a.items[1] = s.d / 128;
      a.asum = a.hsgg;
      a.asum_stride = (s.fmax / s.g) * 16;
      const int nb = (s.max_rchunks + s.n_schunks) * s.sub, ng = s.fmax / s.g;
      hipLaunchKernelGGL(k_hsum, dim3((nb * ng * 16 + 255) / 256), dim3(256), 0, stream, a, nb, ng);
    }
    // 8 x ceil(items / 8) workgroups: every XCD's eighth of the items fits
    const long items = (long)s.max_rchunks * a.items[0] + (long)s.n_schunks * a.items[1];
    const long grid = 8 * ((items + 7) / 8);
    if (mode == MODE_W13) {
      if (qpk == 2)
        hipLaunchKernelGGL((k_wide<MODE_W13, 2>), dim3(grid), dim3(WIDE_THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((k_wide<MODE_W13, 1>), dim3(grid), dim3(WIDE_THREADS), 0, stream, a);
    } else {
      if (qpk == 2)
        hipLaunchKernelGGL((k_wide<MODE_W2, 2>), dim3(grid), dim3(WIDE_THREADS), 0, stream, a);
      else
        hipLaunchKernelGGL((k_wide<MODE_W2, 1>), dim3(grid), dim3(WIDE_THREADS), 0, stream, a);
    }
    return hipGetLastError();
  }
  const long max_items = (long)s.max_rchunks * a.items[0] + (long)s.n_schunks * a.items[1];
  if (max_items <= (long)num_cu * ffn_wpe(mode, qpk) * 2) {
    // at most one item per two wave slots: one workgroup per item, its
    // k-blocks split over the workgroup's waves: four while the items fill at
    // most 2.5 workgroups per CU, else two (more items, shorter chains
    // already)
    const int nwg = (int)((max_items + 7) & ~7L);
    const bool ks4 = max_items * 4 <= (long)num_cu * 10;
    const dim3 g(nwg);
    if (mode == MODE_W13) {
      if (qpk == 2) {
        if (ks4) hipLaunchKernelGGL((k_ffn_small<MODE_W13, 2, 4>), g, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_ffn_small<MODE_W13, 2, 2>), g, dim3(128), 0, stream, a);
      } else {
        if (ks4) hipLaunchKernelGGL((k_ffn_small<MODE_W13, 1, 4>), g, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_ffn_small<MODE_W13, 1, 2>), g, dim3(128), 0, stream, a);
      }
    } else {
      if (qpk == 2) {
        if (ks4) hipLaunchKernelGGL((k_ffn_small<MODE_W2, 2, 4>), g, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_ffn_small<MODE_W2, 2, 2>), g, dim3(128), 0, stream, a);
      } else {
        if (ks4) hipLaunchKernelGGL((k_ffn_small<MODE_W2, 1, 4>), g, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((k_ffn_small<MODE_W2, 1, 2>), g, dim3(128), 0, stream, a);
      }
    }
    return hipGetLastError();
  }
  long grid = (max_items + 3) / 4;
  // waves per SIMD x 4 SIMDs / 4 waves per block
  const long cap = (long)num_cu * ffn_wpe(mode, qpk);
  if (grid > cap) grid = cap;
  grid = (grid + 7) & ~7L;  // whole rounds over the 8 XCDs
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
  a.sub = s.sub;
  a.chunks = reinterpret_cast<const int4*>(ws + L.chunks);
  a.meta = reinterpret_cast<const int*>(ws + L.meta);
  a.max_rchunks = s.max_rchunks;
  a.slot_info = reinterpret_cast<const int*>(ws + L.slot_info);
  a.xg = reinterpret_cast<uint16_t*>(ws + L.xg);
  a.xvg = reinterpret_cast<float2*>(ws + L.xvg);
  const int nb = (s.max_rchunks + s.n_schunks) * s.sub, nkb = s.d / 128;
  if (s.sub > 1)
    hipLaunchKernelGGL(k_gather<4>, dim3(nb, (nkb + 3) / 4), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(k_gather<1>, dim3(nb, nkb), dim3(256), 0, stream, a);
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
  const int* ps = reinterpret_cast<const int*>(ws + L.pair_slot);
  const float* ob = reinterpret_cast<const float*>(ws + L.obuf);
  if (s.k > CMB_KMAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_combine, grid, dim3(256), 0, stream, s.T, s.k, s.d, s.P, s.n_shared, ps, gate, ob, y,
                     accumulate);
  return hipGetLastError();
}

}  // namespace moe
