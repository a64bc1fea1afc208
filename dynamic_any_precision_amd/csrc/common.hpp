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

// ---------------------------------------------------------------------------
// Bitplane unpack into bf16 MFMA operands.
//
// One 32-column chunk of one row is held by one lane as a word per plane
// (bit i = column i of the chunk).  A unit of one or two consecutive planes
// (p, p+1) is turned into 16 words of packed bf16 pairs; output word k
// (k = 0..15) carries column k in its low half and column k+16 in its high
// half, each as the bf16 value 128 + f * 4^a(k), where f = 2*bit_p + bit_{p+1}
// is the unit's 2-bit field of that column and a(k) = (k/2) mod 3.  Placing
// the field at mantissa offset 2*a(k) lets every output word be produced by a
// single shift-free AND-OR from one of three pre-shifted sources, so a 32-column
// chunk costs 24 ALU operations per unit.  The activations that meet word k
// are pre-scaled by 4^-a(k), and the constant 128 is removed afterwards
// through the group sums, so the products sum to exactly sum_c f(c) x(c).
//
// MFMA i (i = 0..3) takes output words 4i..4i+3; in the bf16 16x16x32 operand
// layout a lane's 8 K-slots are then (word 4i+u, half h) -> slot 2u+h, i.e.
// column (4i+u) + 16h of the chunk.

__host__ __device__ constexpr int a_exp(int k) { return (k >> 1) % 3; }

// Position of chunk column c (0..31) inside the B-fragment of its chunk:
// returns mfma index i in bits [4:3] and the slot in bits [2:0].
__host__ __device__ constexpr int frag_pos(int c) {
  return (((c & 15) >> 2) << 3) | (((c & 3) << 1) | (c >> 4));
}

struct Frag16 {
  uint32_t w[16];
};

__device__ __forceinline__ void unpack_unit(uint32_t hi, uint32_t lo, Frag16& o) {
  // Even columns: field of column 2m at bits 2m..2m+1; odd columns likewise.
  const uint32_t E0 = ((hi << 1) & 0xAAAAAAAAu) | (lo & 0x55555555u);
  const uint32_t O0 = (hi & 0xAAAAAAAAu) | ((lo >> 1) & 0x55555555u);
  const uint32_t E6 = E0 >> 6, E12 = E0 >> 12;
  const uint32_t O6 = O0 >> 6, O12 = O0 >> 12;
  const uint32_t B = 0x43004300u;
  o.w[0] = (E0 & 0x00030003u) | B;
  o.w[1] = (O0 & 0x00030003u) | B;
  o.w[2] = (E0 & 0x000C000Cu) | B;
  o.w[3] = (O0 & 0x000C000Cu) | B;
  o.w[4] = (E0 & 0x00300030u) | B;
  o.w[5] = (O0 & 0x00300030u) | B;
  o.w[6] = (E6 & 0x00030003u) | B;
  o.w[7] = (O6 & 0x00030003u) | B;
  o.w[8] = (E6 & 0x000C000Cu) | B;
  o.w[9] = (O6 & 0x000C000Cu) | B;
  o.w[10] = (E6 & 0x00300030u) | B;
  o.w[11] = (O6 & 0x00300030u) | B;
  o.w[12] = (E12 & 0x00030003u) | B;
  o.w[13] = (O12 & 0x00030003u) | B;
  o.w[14] = (E12 & 0x000C000Cu) | B;
  o.w[15] = (O12 & 0x000C000Cu) | B;
}

__device__ __forceinline__ bf16x8_t frag_operand(const Frag16& f, int i) {
  bf16x8_t v;
  uint32_t* p = reinterpret_cast<uint32_t*>(&v);
  p[0] = f.w[4 * i + 0];
  p[1] = f.w[4 * i + 1];
  p[2] = f.w[4 * i + 2];
  p[3] = f.w[4 * i + 3];
  return v;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

__device__ __forceinline__ f32x4_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace moe
