// Shared device helpers for the gfx950 kernels of libmoe_anyprec.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int WAVE = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even.  Inputs here are finite.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ---------------------------------------------------------------------------
// wave reductions (wave64, shuffles across the full wave)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

// Wave-wide integer sum through DPP lane moves (no LDS round trips):
// quad swaps, half-row and row mirrors give every lane its 16-lane row sum,
// row broadcasts 15 and 31 carry the rows into lane 63.
__device__ __forceinline__ int wave_sum_i_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, WAVE));
  return v;
}

// s_waitcnt immediate that waits until at most n vector memory loads are
// outstanding (n <= 63) and leaves the other counters unconstrained.
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// ---------------------------------------------------------------------------
// Bitplane unpack into bf16 MFMA operands.
//
// One 32-column chunk of one row is held by one lane as a word per plane
// (bit i = column i of the chunk).  A unit of one or two consecutive planes
// (p, p+1) is turned into 16 words of packed bf16 pairs; output word k
// (k = 0..15) carries column k in its low half and column k+16 in its high
// half, each as the bf16 value 2^e (128 + f * 4^a(k)), where f = 2*bit_p +
// bit_{p+1} is the unit's 2-bit field of that column (bit_{p+1} = 0 for a
// one-plane unit), a(k) = (k/2) mod 3 and 2^e the unit's place value
// (e = b_max - 2 - p), carried by the exponent field of the bias constant.
// Placing the field at mantissa offset 2*a(k) lets every output word be made
// by one AND-OR from one of three pre-shifted sources: 24 ALU operations per
// unit and chunk.  The activations that meet word k are pre-scaled by
// 4^-a(k); the constant 2^e * 128 is removed afterwards through the group
// sums, so the products sum to exactly sum_c 2^e f(c) x(c).
//
// MFMA i (i = 0..3) takes output words 4i..4i+3; in the bf16 16x16x32 operand
// layout a lane's 8 K-slots are then (word 4i+u, half h) -> slot 2u+h, i.e.
// column (4i+u) + 16h of the chunk.

__host__ __device__ constexpr int a_exp(int k) { return (k >> 1) % 3; }

// Position of chunk column c (0..31) inside the B-fragment of its chunk:
// mfma index i in bits [4:3], slot in bits [2:0].
__host__ __device__ constexpr int frag_pos(int c) {
  return (((c & 15) >> 2) << 3) | (((c & 3) << 1) | (c >> 4));
}

// bf16 pair bias 2^e * 128 in both halves.
__host__ __device__ constexpr uint32_t unit_bias(int e) {
  return (uint32_t)((134 + e) << 7) * 0x10001u;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// (x & m) | c: one v_and_or_b32 with m and c in VGPRs.  Written in plain C so
// that the compiler sees the instruction: its results feed matrix-core
// operands, and the wait states between the two are the compiler's to insert.
__host__ __device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

struct UnpackConst {
  uint32_t m0, m1, m2;  // field masks at offsets 0, 2, 4 in both halves
};

// Materialise a constant in a VGPR once (opaque to rematerialisation).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  asm volatile("" : "+v"(c));
  return c;
}

__device__ __forceinline__ UnpackConst unpack_const() {
  UnpackConst k;
  k.m0 = vconst(0x00030003u);
  k.m1 = vconst(0x000C000Cu);
  k.m2 = vconst(0x00300030u);
  return k;
}

// Four MFMA A operands (words 4i..4i+3 each) of one unit.
__device__ __forceinline__ void unpack_unit(uint32_t hi, uint32_t lo, bool two, uint32_t bias, UnpackConst k,
                                            u32x4_t (&o)[4]) {
  uint32_t E0, O0;
  if (two) {
    E0 = ((hi << 1) & 0xAAAAAAAAu) | (lo & 0x55555555u);
    O0 = (hi & 0xAAAAAAAAu) | ((lo >> 1) & 0x55555555u);
  } else {
    E0 = (hi << 1) & 0xAAAAAAAAu;
    O0 = hi & 0xAAAAAAAAu;
  }
  const uint32_t E6 = E0 >> 6, E12 = E0 >> 12;
  const uint32_t O6 = O0 >> 6, O12 = O0 >> 12;
  o[0] = u32x4_t{and_or(E0, k.m0, bias), and_or(O0, k.m0, bias), and_or(E0, k.m1, bias), and_or(O0, k.m1, bias)};
  o[1] = u32x4_t{and_or(E0, k.m2, bias), and_or(O0, k.m2, bias), and_or(E6, k.m0, bias), and_or(O6, k.m0, bias)};
  o[2] = u32x4_t{and_or(E6, k.m1, bias), and_or(O6, k.m1, bias), and_or(E6, k.m2, bias), and_or(O6, k.m2, bias)};
  o[3] = u32x4_t{and_or(E12, k.m0, bias), and_or(O12, k.m0, bias), and_or(E12, k.m1, bias), and_or(O12, k.m1, bias)};
}

// ---------------------------------------------------------------------------
// Nibble expansion (wide chunks: one matrix-core pass per width).
//
// All planes of a lane's 32-column chunk of one row at once: plane p becomes
// bit 3 - p of a 4-bit field per column, so the field of a pair read at
// width b (planes p < b, the others zero) is f = ((q >> D) << D) * 2^(4 - B),
// D = B - b.  Output word k (k = 0..15) carries column k in its low half and
// column k + 16 in its high half, each as the bf16 value 2^e (128 + f 8^a)
// with a = a_nib(k) and 2^e = 2^(B - 4) (the bias constant's exponent), so
// a width-b operand is the full-width operand with the field bits of the
// planes p >= b cleared (`nib_width_mask`).  Activations meeting word k are
// pre-scaled by 8^-a; the products then sum to sum_c ((q >> D) << D)(c) x(c)
// plus 2^(B - 4) 128 V, V the 8^-a-weighted sum, removed through the group
// sums.  Two plane pairs are merged into 2-bit fields (columns 2j and 2j+1),
// the two pairs into nibbles of columns 4j + r (one word per r), and each
// output word is one shift and one AND-OR of those: 44 ALU operations per
// chunk of 32 columns at any width.
//
// MFMA i takes words 4i..4i+3 as for `unpack_unit`, so all of MFMA i's words
// share a = i & 1.

__host__ __device__ constexpr int a_nib(int k) { return (k >> 2) & 1; }

__host__ __device__ __forceinline__ uint32_t bit_insert(uint32_t m, uint32_t a, uint32_t b) { return (a & m) | (b & ~m); }

// Field mask of width b (planes 0..b-1 kept) for the words of MFMA i, bias
// bits included.
__host__ __device__ constexpr uint32_t nib_width_mask(int b, int i) {
  return 0xFF80FF80u | ((((0xFu << (4 - b)) & 0xFu) << (3 * (i & 1))) * 0x10001u);
}

struct NibConst {
  uint32_t e2, e4, f0, f3;  // 2-bit lane masks, nibble lane masks, field masks at offsets 0 and 3
};

__host__ __device__ __forceinline__ NibConst nib_const_plain() {
  return NibConst{0xAAAAAAAAu, 0xCCCCCCCCu, 0x000F000Fu, 0x00780078u};
}

// n3..n0: the plane words of nibble bits 3..0 (plane 0 is n3).
__host__ __device__ __forceinline__ void unpack_nib(uint32_t n3, uint32_t n2, uint32_t n1, uint32_t n0, uint32_t bias,
                                                    NibConst k, u32x4_t (&o)[4]) {
  const uint32_t Eh = bit_insert(k.e2, n3 << 1, n2);  // columns 2j: (bit 3, bit 2) at bits 2j+1, 2j
  const uint32_t Oh = bit_insert(k.e2, n3, n2 >> 1);  // columns 2j+1
  const uint32_t El = bit_insert(k.e2, n1 << 1, n0);
  const uint32_t Ol = bit_insert(k.e2, n1, n0 >> 1);
  uint32_t Q[4];
  Q[0] = bit_insert(k.e4, Eh << 2, El);  // nibble j = column 4j
  Q[1] = bit_insert(k.e4, Oh << 2, Ol);  // column 4j + 1
  Q[2] = bit_insert(k.e4, Eh, El >> 2);  // column 4j + 2
  Q[3] = bit_insert(k.e4, Oh, Ol >> 2);  // column 4j + 3
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    o[0][r] = and_or(Q[r], k.f0, bias);
    o[1][r] = and_or(Q[r] >> 1, k.f3, bias);
    o[2][r] = and_or(Q[r] >> 8, k.f0, bias);
    o[3][r] = and_or(Q[r] >> 9, k.f3, bias);
  }
}

// Place of lane (token row r16, k-chunk jg) inside the 1 KiB operand block of
// one matrix-core product, for the streaming kernels' activations.  Gate/up
// (gathered token rows of 16-pair chunks): token-major, r16 * 4 + jg, so the
// live rows of a chunk (the first m) are one contiguous 64 m bytes and a
// load touches m/2 cache lines instead of four separate 256-byte stretches.
// Down (the SwiGLU output h): k-chunk-major, jg * 16 + r16 = lane.
__device__ __forceinline__ uint32_t act_pos(int mode, int r16, int jg) {
  return mode == 0 ? (uint32_t)(r16 * 4 + jg) : (uint32_t)(jg * 16 + r16);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ u32x4_t as_u32x4(uint4 v) { return u32x4_t{v.x, v.y, v.z, v.w}; }

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace moe
