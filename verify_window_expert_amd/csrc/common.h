// Device helpers shared by the window kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sw {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxRows = 8;
constexpr int kMaxTopk = 8;
// word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle
constexpr int kRsrcWord3 = 0x00020000;
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

// One output of the combine: the row's k + 1 expert outputs y[j] times their weights w[j]
// (routed experts in ascending id order, the shared expert last with weight 1), added by
// fused multiply-adds from zero in that order, then the residual. Every kernel that
// forms a layer output uses this one definition, so their outputs agree bit for bit.
__device__ __forceinline__ float combine_one(const float (&w)[kMaxTopk + 1], const float (&y)[kMaxTopk + 1], int k1,
                                             bool has_res, float res) {
  float s = 0.f;
#pragma unroll
  for (int j = 0; j <= kMaxTopk; j++)
    if (j < k1) s = fmaf(w[j], y[j], s);
  if (has_res) s += res;
  return s;
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
//
// The masks and the constant are kept in VGPRs (CodeConsts): with three register
// operands each mask-and-merge is one v_and_or_b32 (VOP3 on gfx9 takes no literal, so
// with literal constants the compiler emits a separate and + or).
struct CodeConsts {
  uint32_t m4, m2, magic;
};

__device__ __forceinline__ CodeConsts code_consts() {
  CodeConsts c;
  asm("v_mov_b32 %0, 0x000f000f" : "=v"(c.m4));
  asm("v_mov_b32 %0, 0x00030003" : "=v"(c.m2));
  asm("v_mov_b32 %0, 0x43004300" : "=v"(c.magic));
  return c;
}

__device__ __forceinline__ bf16x8 q4_to_bf16x8(uint32_t v, const CodeConsts& k) {
  u32x4 w;
  w[0] = (v & k.m4) | k.magic;
  w[1] = ((v >> 4) & k.m4) | k.magic;
  w[2] = ((v >> 8) & k.m4) | k.magic;
  w[3] = ((v >> 12) & k.m4) | k.magic;
  return __builtin_bit_cast(bf16x8, w);
}

// 2-bit: the 8 codes of one block are 16 bits (code i at bits 2i), the low or high half
// of a code word. One byte permute spreads the half's two bytes into the two halves of
// a word; then, per shift 2i, codes i and i+4: the same element order as q4_to_bf16x8.
__device__ __forceinline__ bf16x8 q2_to_bf16x8(uint32_t word, bool high, const CodeConsts& k) {
  const uint32_t v = __builtin_amdgcn_perm(0u, word, high ? 0x0C030C02u : 0x0C010C00u);
  u32x4 w;
  w[0] = (v & k.m2) | k.magic;
  w[1] = ((v >> 2) & k.m2) | k.magic;
  w[2] = ((v >> 4) & k.m2) | k.magic;
  w[3] = ((v >> 6) & k.m2) | k.magic;
  return __builtin_bit_cast(bf16x8, w);
}

// The same conversion with the byte-permute selector in a register (0x0C010C00: the low
// half, 0x0C030C02: the high half), so that lanes can take different halves.
__device__ __forceinline__ bf16x8 q2_to_bf16x8_sel(uint32_t word, uint32_t sel, const CodeConsts& k) {
  const uint32_t v = __builtin_amdgcn_perm(0u, word, sel);
  u32x4 w;
  w[0] = (v & k.m2) | k.magic;
  w[1] = ((v >> 2) & k.m2) | k.magic;
  w[2] = ((v >> 4) & k.m2) | k.magic;
  w[3] = ((v >> 6) & k.m2) | k.magic;
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

// ------------------------------------------------------------ cross-row gathers
// Lane l = 16*q + c holds v_q (one value per 16-lane row q, for column c). Returns, in
// every lane of column c, the four values v_0..v_3 (gfx950 permlane swaps: two rows
// exchange halves, then neighbouring rows).
__device__ __forceinline__ void gather_rows(uint32_t v, uint32_t (&out)[4]) {
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);      // {r0 r1 r0 r1}, {r2 r3 r2 r3}
  const auto lo = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);  // {r0 x4}, {r1 x4}
  const auto hi = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);  // {r2 x4}, {r3 x4}
  out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
}

// Lane l = 16*q + c holds v_q. Returns, in every lane of column c, out[0] = v_0 in lanes
// 0..31 and v_1 in lanes 32..63, out[1] = v_2 in lanes 0..31 and v_3 in lanes 32..63
// (neighbouring rows exchange first, then the halves).
__device__ __forceinline__ void pair_rows(uint32_t v, uint32_t (&out)[2]) {
  const auto t = __builtin_amdgcn_permlane16_swap(v, v, false, false);           // {r0 r0 r2 r2}, {r1 r1 r3 r3}
  const auto u = __builtin_amdgcn_permlane32_swap(t[0], t[1], false, false);     // {r0 r0 r1 r1}, {r2 r2 r3 r3}
  out[0] = u[0]; out[1] = u[1];
}

// ------------------------------------------------------------ wave reductions
// All-reduce over the 64 lanes of a wave without LDS: DPP within rows of 16 (swap
// neighbours, swap pairs, mirror within 8, mirror within 16), then the gfx950 permlane
// swaps across rows. Every lane ends with the same value when op is commutative (each
// step combines two lanes that hold the same pair of operands).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}

// v summed over the 4 lanes of its quad, by two DPP quad permutes (lane ^ 1, then
// lane ^ 2): every lane of the quad gets (v0 + v1) + (v2 + v3) or the same terms in the
// other order, which is the same float. All 4 lanes must be active.
__device__ __forceinline__ float quad_sum(float v) {
  v += __uint_as_float(dpp32<0xB1>(__float_as_uint(v)));   // quad_perm [1,0,3,2]
  v += __uint_as_float(dpp32<0x4E>(__float_as_uint(v)));   // quad_perm [2,3,0,1]
  return v;
}

// A value of N 32-bit words, permuted word by word.
template <int N>
struct Words {
  uint32_t w[N];
};

template <int CTRL, int N>
__device__ __forceinline__ Words<N> dpp_words(const Words<N>& v) {
  Words<N> r;
#pragma unroll
  for (int i = 0; i < N; i++) r.w[i] = dpp32<CTRL>(v.w[i]);
  return r;
}

template <int N, class Op>
__device__ __forceinline__ Words<N> wave_allreduce_words(Words<N> v, Op op) {
  v = op(v, dpp_words<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
  v = op(v, dpp_words<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
  v = op(v, dpp_words<0x141>(v));   // row_half_mirror: 7 - lane within 8
  v = op(v, dpp_words<0x140>(v));   // row_mirror: 15 - lane within 16
  Words<N> a, b;
#pragma unroll
  for (int i = 0; i < N; i++) {     // rows {0,1} and {2,3} exchange
    const auto p = __builtin_amdgcn_permlane16_swap(v.w[i], v.w[i], false, false);
    a.w[i] = p[0];
    b.w[i] = p[1];
  }
  v = op(a, b);
#pragma unroll
  for (int i = 0; i < N; i++) {     // halves exchange
    const auto p = __builtin_amdgcn_permlane32_swap(v.w[i], v.w[i], false, false);
    a.w[i] = p[0];
    b.w[i] = p[1];
  }
  return op(a, b);
}

__device__ __forceinline__ Words<2> words_of(double d) {
  const uint64_t u = __builtin_bit_cast(uint64_t, d);
  return Words<2>{{(uint32_t)u, (uint32_t)(u >> 32)}};
}
__device__ __forceinline__ double double_of(const Words<2>& v) {
  return __builtin_bit_cast(double, (uint64_t)v.w[0] | ((uint64_t)v.w[1] << 32));
}

__device__ __forceinline__ double wave_sum(double x) {
  return double_of(wave_allreduce_words<2>(words_of(x), [](const Words<2>& p, const Words<2>& q) {
    return words_of(double_of(p) + double_of(q));
  }));
}

__device__ __forceinline__ double wave_max(double x) {
  return double_of(wave_allreduce_words<2>(words_of(x), [](const Words<2>& p, const Words<2>& q) {
    return words_of(fmax(double_of(p), double_of(q)));
  }));
}

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

// ------------------------------------------------------------ weight rings
// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), unrolled: ring
// slots are then compile-time register arrays.
template <int N, int I = 0, class Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// Units of a wave's work in rounds of DEPTH through the ring (unit u in slot u % DEPTH):
// full rounds whose refills are all in range, one round whose refills stop at the end,
// then the remainder. A round has no early exit: an exit inside the round would make the
// compiler wait for every outstanding load at the loop head.
template <int DEPTH, class Step>
__device__ __forceinline__ void run_ring(int units, Step&& step) {
  int u0 = 0;
  for (; u0 + 2 * DEPTH <= units; u0 += DEPTH)
    static_for<DEPTH>([&](auto d) __attribute__((always_inline)) { step(d, true); });
  if (u0 + DEPTH <= units) {
    static_for<DEPTH>([&](auto d) __attribute__((always_inline)) { step(d, u0 + d + DEPTH < units); });
    u0 += DEPTH;
  }
  static_for<DEPTH>([&](auto d) __attribute__((always_inline)) {
    if (u0 + d < units) step(d, false);
  });
}

}  // namespace sw
