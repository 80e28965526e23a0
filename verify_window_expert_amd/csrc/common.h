// Device helpers shared by the window kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxRows = 8;
constexpr int kCounterBytes = 4096;

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// float -> bfloat16, round to nearest even (finite values; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_lo(uint32_t m) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t m) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(m >> 16));
}

// Activation element i as float. The dtype is a template parameter: a runtime branch
// around each load would put every load in its own block and serialise them.
template <bool F32>
__device__ __forceinline__ float load_x(const void* x, long i) {
  if constexpr (F32) return ((const float*)x)[i];
  else return bf16_to_f32(((const uint16_t*)x)[i]);
}

// ------------------------------------------------------------ code -> MFMA operand
//
// A lane's MFMA operand holds 8 consecutive inputs k0..k0+7 of one block. The packed
// 4-bit word of those 8 codes has code i in bits 4i..4i+3. Masking two nibbles at a
// time into the mantissas of the bf16 constant 128.0 (0x4300) gives the exact values
// 128 + q. The lane's elements then hold the inputs in the order
//     element e : input k0 + kPerm[e],   kPerm = {0, 4, 1, 5, 2, 6, 3, 7}
// and the activations staged for the other operand use the same order.
__device__ __forceinline__ bf16x8 q4_to_bf16x8(uint32_t v) {
  u32x4 w;
  w[0] = (v & 0x000F000Fu) | 0x43004300u;
  w[1] = ((v >> 4) & 0x000F000Fu) | 0x43004300u;
  w[2] = ((v >> 8) & 0x000F000Fu) | 0x43004300u;
  w[3] = ((v >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, w);
}

// 2-bit: the 8 codes of one block are 16 bits (code i at bits 2i). Spreading the two
// bytes into the two halves of a word gives, per shift 2i, codes i and i+4: the same
// element order as q4_to_bf16x8.
__device__ __forceinline__ bf16x8 q2_to_bf16x8(uint32_t half16) {
  const uint32_t v = (half16 & 0xFFu) | ((half16 & 0xFF00u) << 8);
  u32x4 w;
  w[0] = (v & 0x00030003u) | 0x43004300u;
  w[1] = ((v >> 2) & 0x00030003u) | 0x43004300u;
  w[2] = ((v >> 4) & 0x00030003u) | 0x43004300u;
  w[3] = ((v >> 6) & 0x00030003u) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, w);
}

// 8-bit signed codes, 4 per word (code i in byte i). Flipping the sign bit gives
// u = q + 128 in [1, 255]; masking bytes into the mantissa of the binary16 constant
// 1024.0 (0x6400) gives exactly 1024 + u = 1152 + q. Element order for the 8 codes
// (words lo, hi) of a block: kPerm8 = {0, 2, 1, 3, 4, 6, 5, 7}.
__device__ __forceinline__ f16x8 q8_to_f16x8(uint32_t lo, uint32_t hi) {
  const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
  u32x4 w;
  w[0] = (a & 0x00FF00FFu) | 0x64006400u;
  w[1] = ((a >> 8) & 0x00FF00FFu) | 0x64006400u;
  w[2] = (b & 0x00FF00FFu) | 0x64006400u;
  w[3] = ((b >> 8) & 0x00FF00FFu) | 0x64006400u;
  return __builtin_bit_cast(f16x8, w);
}

// Input offset (within 8) held by operand element e.
__device__ __forceinline__ int perm_q(int e) { return ((e & 1) << 2) | (e >> 1); }   // 0 4 1 5 2 6 3 7
__device__ __forceinline__ int perm_q8(int e) { return (e & 4) | ((e & 1) << 1) | ((e >> 1) & 1); } // 0 2 1 3 4 6 5 7

// ------------------------------------------------------------------------ MFMA
// 16x16x32: A lane l = A[l%16][8*(l/16) + e], B lane l = B[8*(l/16) + e][l%16],
// C lane l element i = C[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x4 fp32: A lane l = A[l%16][l/16], B lane l = B[l/16][l%16], same C layout.
__device__ __forceinline__ f32x4 mfma_f32x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

}  // namespace sw
