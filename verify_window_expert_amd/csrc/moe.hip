// Experts of a verify window: fused dequant gate/up matvec with SwiGLU, then the down
// matvec with the weighted combine of each row's experts and the shared expert.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// a window fetches the shared expert and each routed expert its rows use a single time,
// whichever rows share them; "Exactness": a row's arithmetic must not depend on how many
// rows share an expert, so every expert runs the same code for any number of rows.
//
// Matrix-core formulation. The window's rows (at most 8) are the 16-wide M side of a
// v_mfma_f32_16x16x32_bf16: columns 0..7 hold the rows' activations rounded to bf16
// ("hi"), columns 8..15 the bf16 rounding of the remainder ("lo", zero for bf16
// inputs), so hi + lo carries 16 significant bits of a float input. The weights are
// the N side: a lane's 8 packed codes become the exact bf16 values 128 + q. Per 32-input
// block b of weight row n the MFMA gives D = sum (128 + q) x, and
//     sum_k w x = scale * D + (min - 128 * scale) * Sx,   Sx = sum of the block's x,
// with the scale applied to the 4 accumulator values a lane holds and the second term
// for 4 blocks at once by one v_mfma_f32_16x16x4_f32 (A = Sx, B = min - 128*scale).
// A row's result depends only on its own column, so it is the same in any window.
//
// Latency: a window moves only tens of MB, so the kernels are built to keep many loads
// in flight: every wave issues all of its weight loads before it waits on any, the
// activations are staged with 16-byte loads issued together, and routing metadata is
// read once, in parallel, into LDS.
#include "route_core.h"

#include <mutex>
#include <type_traits>

namespace sw {

constexpr int kThreads = 256;   // 4 waves
constexpr int kMaxExperts = 256;
constexpr int kMaxSlots = kMaxRows * kMaxTopk + 1;   // routed experts a window can use + shared
#ifndef SW_GU_DEPTH
#define SW_GU_DEPTH 2
#endif
constexpr int kGuDepth = SW_GU_DEPTH;                // gate/up: units in flight per wave (ring slots)
#ifndef SW_DN_DEPTH
#define SW_DN_DEPTH 2
#endif
constexpr int kDnDepth = SW_DN_DEPTH;                // down: units in flight per wave
#ifndef SW_WEIGHT_AUX
#define SW_WEIGHT_AUX 2                              // weight loads: non-temporal (one use per window;
#endif                                               // measured faster than plain loads)

// ------------------------------------------------------------ activation operand (LDS)
// LDS image of the activation operand: rows [nrows][stride] of bf16, inputs permuted
// within each group of 8 as the code conversion orders them, one all-zero row (read by
// the lanes of absent columns, so no read is predicated), then the block sums Sx
// [blocks][16] (zero for absent columns).
struct ActLds {
  uint16_t* xs;
  float* sx;
  int stride;     // elements per row
  int zero_row;   // index of the zero row
};

__device__ __forceinline__ ActLds act_lds(uint8_t* smem, int K, int nrows) {
  ActLds l;
  l.stride = K + 8;
  l.zero_row = nrows;
  l.xs = (uint16_t*)smem;
  l.sx = (float*)(smem + (size_t)(nrows + 1) * l.stride * 2);
  return l;
}

__host__ __device__ inline size_t act_lds_bytes(int K, int nrows) {
  return (size_t)(nrows + 1) * (K + 8) * 2 + (size_t)(K / 32) * 16 * 4;
}

size_t gateup_lds_bytes(int hidden, int x_dtype) { return act_lds_bytes(hidden, x_dtype == 0 ? 16 : 8); }

// Convert 8 consecutive source values of row j (inputs 8u..8u+7) to bf16 hi (and lo),
// store them permuted, and add the block sums (4 consecutive lanes = one block).
__device__ __forceinline__ void stage_group(const ActLds& l, bool ok, int j, int u, const float (&v)[8], bool with_lo) {
  uint16_t hi[8], lo[8];
  float shi = 0.f, slo = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    hi[e] = f32_to_bf16(v[e]);
    const float hv = bf16_to_f32(hi[e]);
    lo[e] = with_lo ? f32_to_bf16(v[e] - hv) : (uint16_t)0;
    shi += hv;
    slo += bf16_to_f32(lo[e]);
  }
  shi = quad_sum(shi);
  slo = quad_sum(slo);
  if (ok) {
    u32x4 ph, pl;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      ph[w] = (uint32_t)hi[perm_q(2 * w)] | ((uint32_t)hi[perm_q(2 * w + 1)] << 16);
      pl[w] = (uint32_t)lo[perm_q(2 * w)] | ((uint32_t)lo[perm_q(2 * w + 1)] << 16);
    }
    *(u32x4*)(l.xs + (size_t)j * l.stride + 8 * u) = ph;
    if (with_lo) *(u32x4*)(l.xs + (size_t)(8 + j) * l.stride + 8 * u) = pl;
    if ((u & 3) == 0) {
      l.sx[(u >> 2) * 16 + j] = shi;
      if (with_lo) l.sx[(u >> 2) * 16 + 8 + j] = slo;
    }
  }
}

// Zero what staging does not write: the zero row and the block sums of absent columns
// (rows >= nrows; the lo half when there is none). Disjoint from stage_group's writes.
// THREADS is the workgroup size (a constant: reading blockDim costs a load).
template <int THREADS>
__device__ __forceinline__ void zero_absent(const ActLds& l, int K, int nrows, bool with_lo) {
  u32x4* zr = (u32x4*)(l.xs + (size_t)l.zero_row * l.stride);
  for (int i = threadIdx.x; i < l.stride / 8; i += THREADS) zr[i] = u32x4{0u, 0u, 0u, 0u};
  for (int i = threadIdx.x; i < (K / 32) * 16; i += THREADS) {
    const int col = i & 15;
    const bool present = col < 8 ? col < nrows : (with_lo && col - 8 < nrows);
    if (!present) l.sx[i] = 0.f;
  }
}

// Group i (of 8 values) of nsrc rows of width K, converted to floats from the loaded
// words (float source: two 16-byte words; bf16 source: one).
template <bool F32SRC>
__device__ __forceinline__ void group_values(const u32x4 (&raw)[F32SRC ? 2 : 1], bool ok, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 8; e++) {
    if (!ok) {
      v[e] = 0.f;
    } else if constexpr (F32SRC) {
      // element into a plain variable first: a bit cast of a vector-element
      // expression reads the vector's first element
      const uint32_t w = raw[e >> 2][e & 3];
      v[e] = __uint_as_float(w);
    } else {
      v[e] = bf16_to_f32((uint16_t)(raw[0][e >> 1] >> (16 * (e & 1))));
    }
  }
}

template <bool F32SRC>
__device__ __forceinline__ void load_group(u32x4 (&raw)[F32SRC ? 2 : 1], const void* src, int K, int j, int u) {
  if constexpr (F32SRC) {
    const u32x4* p = (const u32x4*)((const float*)src + (long)j * K + 8 * u);
    raw[0] = p[0];
    raw[F32SRC ? 1 : 0] = p[1];
  } else {
    raw[0] = *(const u32x4*)((const uint16_t*)src + (long)j * K + 8 * u);
  }
}

// Groups tid, tid + threads, ... (XG of them) of nsrc rows, loaded into registers.
template <int THREADS, int XG, bool F32SRC>
__device__ __forceinline__ void load_groups(u32x4 (&xr)[XG][F32SRC ? 2 : 1], const void* src, int nsrc, int K) {
  const int ngrp = K / 8, total = nsrc * ngrp;
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int i = min(it * THREADS + (int)threadIdx.x, total - 1);
    load_group<F32SRC>(xr[it], src, K, i / ngrp, i % ngrp);
  }
}

// bf16 source: the values are already the hi part (lo = 0), so the permuted words are
// byte permutes of the loaded words (input i of the group in half i % 2 of word i / 2),
// and the block sum adds the same values in the same order as stage_group.
__device__ __forceinline__ void stage_group_bf16(const ActLds& l, bool ok, int j, int u, const u32x4& w) {
  u32x4 ph;
  ph[0] = __builtin_amdgcn_perm(w[2], w[0], 0x05040100u);   // inputs 0, 4
  ph[1] = __builtin_amdgcn_perm(w[2], w[0], 0x07060302u);   // inputs 1, 5
  ph[2] = __builtin_amdgcn_perm(w[3], w[1], 0x05040100u);   // inputs 2, 6
  ph[3] = __builtin_amdgcn_perm(w[3], w[1], 0x07060302u);   // inputs 3, 7
  float shi = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint32_t word = w[e >> 1];
    shi += __uint_as_float((e & 1) ? (word & 0xFFFF0000u) : (word << 16));
  }
  shi = quad_sum(shi);
  if (ok) {
    *(u32x4*)(l.xs + (size_t)j * l.stride + 8 * u) = ph;
    if ((u & 3) == 0) l.sx[(u >> 2) * 16 + j] = shi;
  }
}

template <int THREADS, int XG, bool F32SRC>
__device__ __forceinline__ void stage_groups(const ActLds& l, const u32x4 (&xr)[XG][F32SRC ? 2 : 1], int nsrc, int K) {
  const int ngrp = K / 8, total = nsrc * ngrp;
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int base = it * THREADS;
    if (base >= total) break;
    const int i = base + threadIdx.x;
    const bool ok = i < total;
    if constexpr (!F32SRC) {
      const u32x4 w = ok ? xr[it][0] : u32x4{0u, 0u, 0u, 0u};
      stage_group_bf16(l, ok, ok ? i / ngrp : 0, ok ? i % ngrp : 0, w);
    } else {
      float v[8];
      group_values<F32SRC>(xr[it], ok, v);
      stage_group(l, ok, ok ? i / ngrp : 0, ok ? i % ngrp : 0, v, F32SRC);
    }
  }
}

// Place of input k0 + k (k < 8) in its group of 8 in the image: the code conversion's
// order holds input perm_q(e) at element e, so input k sits at element 2 (k % 4) + k / 4.
// For the 16 inputs of a tile (k < 16): the group's base plus that place.
__device__ __forceinline__ int tile_pos(int k) { return (k & 8) | ((k & 3) << 1) | ((k >> 2) & 1); }

// A lane's view of the image: its row (its column c, or the zero row) at its k-offset,
// and its block-sum column.
struct ActLane {
  const uint16_t* row;   // + blk * 32 -> the lane's 8 elements of block blk
  const float* sx;       // + blk4 * 16 -> Sx of block blk4 + q for column c
};

__device__ __forceinline__ ActLane act_lane(const ActLds& l, bool col_ok) {
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  ActLane al;
  al.row = l.xs + (size_t)(col_ok ? c : l.zero_row) * l.stride + q * 8;
  al.sx = l.sx + q * 16 + c;
  return al;
}

// Paired form (bf16 activations: at most 8 of the 16 MFMA columns hold rows). Two
// blocks b = 2p and b' = 2p + 1 of a k-group share one accumulator tile: columns 0..7
// take rows 0..7 against block b, columns 8..15 the same rows against block b'. In MFMA
// m (0, 1) of the pair, lanes of k-slice q supply block b + ((q / 2) xor m) (their own
// stored inputs 8q..8q+7 of that block), and a lane's activation operand is its row's
// inputs where that block matches its column half, else the zero row. Over the two
// MFMAs every input of both blocks meets its row once; lanes 0..31 then hold rows 0..7
// against b, lanes 32..63 against b', so one scale FMA per lane covers both blocks.
struct ActLanePair {
  const uint16_t* row[2];   // MFMA m: + blk * 32 (blk = the pair's first block)
  const float* sx;
};

__device__ __forceinline__ ActLanePair act_lane_pair(const ActLds& l, int R) {
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  const int half = c >> 3, r = c & 7;                 // column half: block b or b'
  const int m_real = (q >> 1) ^ half;                 // the MFMA whose block matches
  ActLanePair al;
#pragma unroll
  for (int m = 0; m < 2; m++) {
    const bool real = m == m_real && r < R;
    al.row[m] = l.xs + (size_t)(real ? r : l.zero_row) * l.stride + half * 32 + q * 8;
  }
  al.sx = l.sx + q * 16 + c;
  return al;
}

// ---------------------------------------------------------------------------- weights
// One (matrix, 16-row tile) as two buffer resources: its codes and its metadata from
// k-group 0 on (the tiled layout of the header: k-group g at g * 1024 code bytes and
// g * 16 * NB metadata words). A load then takes the lane's fixed offset in a VGPR and
// the k-group's offset in an SGPR: no per-load address arithmetic on the vector ALU,
// and the hardware range check keeps every load inside the tile.
struct TileRsrc {
  __amdgpu_buffer_rsrc_t codes, meta;
};


// An expert id read at run time, clamped into [0, E] (E = the shared expert), so that
// a load is always inside the weights even for an unspecified table entry.
__device__ __forceinline__ int clamp_expert(int e, int E) { return min(max(e, 0), E); }

template <int BITS>
__device__ __forceinline__ TileRsrc tile_rsrc(const QDev& m, int expert, int E, int tile, int NG) {
  constexpr int NB = 512 / BITS / 32;
  const bool shared = expert == E;
  const uint8_t* c = shared ? m.sh_codes : m.codes + (long)expert * m.stride_codes;
  const uint8_t* mt = shared ? m.sh_meta : m.meta + (long)expert * m.stride_meta_bytes;
  const long chunk = (long)tile * NG;
  TileRsrc r;
  r.codes = __builtin_amdgcn_make_buffer_rsrc((void*)(c + chunk * 1024), (short)0, NG * 1024, kRsrcWord3);
  r.meta = __builtin_amdgcn_make_buffer_rsrc((void*)(mt + chunk * 16 * NB * 4), (short)0, NG * 16 * NB * 4, kRsrcWord3);
  return r;
}

// Weight loads of one k-group of one matrix for this lane (issued, not yet used): the
// lane's 16 bytes of codes, and (per 4 blocks) the metadata of block 4h + l/16 of row
// l%16, one word per lane. mac_kgroup gathers the row's other blocks from the lanes of
// the same column (gather_rows) instead of loading them four times.
template <int BITS>
struct KGroup {
  static constexpr int NB = 512 / BITS / 32;   // blocks per k-group
  u32x4 codes;
  uint32_t meta[NB / 4];
};

template <int BITS>
__device__ __forceinline__ void load_kgroup(KGroup<BITS>& kg, const TileRsrc& r, int g) {
  constexpr int NB = KGroup<BITS>::NB;
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  kg.codes = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r.codes, lane * 16, g * 1024, SW_WEIGHT_AUX));
#pragma unroll
  for (int h = 0; h < NB / 4; h++)
    kg.meta[h] = __builtin_amdgcn_raw_buffer_load_b32(r.meta, (c * NB + 4 * h + q) * 4, g * 16 * NB * 4, SW_WEIGHT_AUX);
}

template <int BITS>
__device__ __forceinline__ bf16x8 code_operand(const KGroup<BITS>& kg, int beta, const CodeConsts& cc) {
  return BITS == 4 ? q4_to_bf16x8(kg.codes[beta], cc)
                   : q2_to_bf16x8(kg.codes[beta >> 1], (beta & 1) != 0, cc);
}

// Accumulate one k-group of one matrix (or two matrices against the same activations)
// into acc (C layout: column 4*(l/16)+i, row l%16).
// The (min - 128 scale) Sx terms go to mn0 / mn1 (which may be acc0 / acc1 themselves).
template <int BITS, bool TWO>
__device__ __forceinline__ void mac_kgroup(const KGroup<BITS>& k0, const KGroup<BITS>& k1, const ActLane& al, int g,
                                           const CodeConsts& cc, f32x4& acc0, f32x4& acc1, f32x4& mn0, f32x4& mn1) {
  constexpr int NB = KGroup<BITS>::NB;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = 0; h < NB / 4; h++) {
    uint32_t m0[4], m1[4];
    gather_rows(k0.meta[h], m0);
    if (TWO) gather_rows(k1.meta[h], m1);
    bf16x8 ax[4];
#pragma unroll
    for (int b = 0; b < 4; b++) ax[b] = *(const bf16x8*)(al.row + (g * NB + 4 * h + b) * 32);
    const float sx = al.sx[(g * NB + 4 * h) * 16];
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int beta = 4 * h + b;
      const f32x4 d0 = mfma_bf16(ax[b], code_operand<BITS>(k0, beta, cc), z);
      const float s0 = f16_lo(m0[b]);
#pragma unroll
      for (int i = 0; i < 4; i++) acc0[i] = fmaf(s0, d0[i], acc0[i]);
      if (TWO) {
        const f32x4 d1 = mfma_bf16(ax[b], code_operand<BITS>(k1, beta, cc), z);
        const float s1 = f16_lo(m1[b]);
#pragma unroll
        for (int i = 0; i < 4; i++) acc1[i] = fmaf(s1, d1[i], acc1[i]);
      }
    }
    // (min - 128 scale) * Sx of blocks 4h..4h+3 by one fp32 MFMA: the lane supplies
    // block 4h + l/16, exactly the word it loaded
    mn0 = mfma_f32x4(sx, f16_hi(k0.meta[h]) - 128.f * f16_lo(k0.meta[h]), mn0);
    if (TWO) mn1 = mfma_f32x4(sx, f16_hi(k1.meta[h]) - 128.f * f16_lo(k1.meta[h]), mn1);
  }
}

// The lane's code operand for MFMA m of pair p of 4-block group h: block
// 4h + 2p + ((q / 2) xor m). sel2[m] holds the 2-bit half selector for that block; at
// 4 bits the lane picks one of two stored words.
template <int BITS>
__device__ __forceinline__ bf16x8 code_operand_pair(const KGroup<BITS>& kg, int h, int p, int m, bool upper,
                                                    const uint32_t (&sel2)[2], const CodeConsts& cc) {
  if constexpr (BITS == 4) {
    const uint32_t w0 = kg.codes[2 * p], w1 = kg.codes[2 * p + 1];
    return q4_to_bf16x8((upper != (m != 0)) ? w1 : w0, cc);
  } else {
    return q2_to_bf16x8_sel(kg.codes[2 * h + p], sel2[m], cc);
  }
}

// mac_kgroup in the paired form (bf16 activations; see ActLanePair). acc holds rows
// 0..7 against the even blocks in lanes 0..31 and against the odd blocks in lanes
// 32..63; the min terms (mn) fill lanes 0..31 only, as before.
template <int BITS, bool TWO>
__device__ __forceinline__ void mac_kgroup_pair(const KGroup<BITS>& k0, const KGroup<BITS>& k1, const ActLanePair& al,
                                                int g, const CodeConsts& cc, const uint32_t (&sel2)[2], f32x4& acc0,
                                                f32x4& acc1, f32x4& mn0, f32x4& mn1) {
  constexpr int NB = KGroup<BITS>::NB;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  const bool upper = (threadIdx.x & 63) >= 32;
#pragma unroll
  for (int h = 0; h < NB / 4; h++) {
    uint32_t m0[2], m1[2];
    pair_rows(k0.meta[h], m0);
    if (TWO) pair_rows(k1.meta[h], m1);
    const float sx = al.sx[(g * NB + 4 * h) * 16];
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const int blk = g * NB + 4 * h + 2 * p;
      const bf16x8 a0 = *(const bf16x8*)(al.row[0] + blk * 32);
      const bf16x8 a1 = *(const bf16x8*)(al.row[1] + blk * 32);
      f32x4 d0 = mfma_bf16(a0, code_operand_pair<BITS>(k0, h, p, 0, upper, sel2, cc), z);
      d0 = mfma_bf16(a1, code_operand_pair<BITS>(k0, h, p, 1, upper, sel2, cc), d0);
      const float s0 = f16_lo(m0[p]);
#pragma unroll
      for (int i = 0; i < 4; i++) acc0[i] = fmaf(s0, d0[i], acc0[i]);
      if (TWO) {
        f32x4 d1 = mfma_bf16(a0, code_operand_pair<BITS>(k1, h, p, 0, upper, sel2, cc), z);
        d1 = mfma_bf16(a1, code_operand_pair<BITS>(k1, h, p, 1, upper, sel2, cc), d1);
        const float s1 = f16_lo(m1[p]);
#pragma unroll
        for (int i = 0; i < 4; i++) acc1[i] = fmaf(s1, d1[i], acc1[i]);
      }
    }
    mn0 = mfma_f32x4(sx, f16_hi(k0.meta[h]) - 128.f * f16_lo(k0.meta[h]), mn0);
    if (TWO) mn1 = mfma_f32x4(sx, f16_hi(k1.meta[h]) - 128.f * f16_lo(k1.meta[h]), mn1);
  }
}

// The dot-product form of mac_kgroup (bf16 activations only), for comparison with the
// matrix cores: lane (n = l % 16, j = l / 16) takes, for each of the window's rows r < R,
// the dot of its 8 codes of a block (as the exact bf16 values 128 + q) with the row's
// same 8 inputs (v_dot2_f32_bf16, four per block and row) and adds scale x dot; the lane of
// j = 0 also adds (min - 128 scale) x the block's sum of the row's inputs. Absent rows cost
// nothing. The 4 lanes of a row n are summed at the item's end (sum_q).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8_bf16(const bf16x8& a, const bf16x8& b) {
  const u32x4 ua = __builtin_bit_cast(u32x4, a), ub = __builtin_bit_cast(u32x4, b);
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    // each word into a plain variable first: a bit cast of a vector-element expression
    // reads the vector's first element
    const uint32_t wa = ua[i], wb = ub[i];
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wa), __builtin_bit_cast(bf16x2, wb), d, false);
  }
  return d;
}

template <int BITS>
__device__ __forceinline__ void mac_kgroup_valu(const KGroup<BITS>& k0, const KGroup<BITS>& k1, const ActLds& l, int R,
                                                int g, const CodeConsts& cc, float (&ag)[kMaxRows],
                                                float (&au)[kMaxRows]) {
  constexpr int NB = KGroup<BITS>::NB;
  const int q = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int h = 0; h < NB / 4; h++) {
    uint32_t m0[4], m1[4];
    gather_rows(k0.meta[h], m0);
    gather_rows(k1.meta[h], m1);
#pragma unroll
    for (int b = 0; b < 4; b++) {
      const int beta = 4 * h + b, blk = g * NB + beta;
      const bf16x8 wg = code_operand<BITS>(k0, beta, cc), wu = code_operand<BITS>(k1, beta, cc);
      const float sg = f16_lo(m0[b]), su = f16_lo(m1[b]);
      const float cg = q == 0 ? fmaf(-128.f, sg, f16_hi(m0[b])) : 0.f;
      const float cu = q == 0 ? fmaf(-128.f, su, f16_hi(m1[b])) : 0.f;
#pragma unroll
      for (int r = 0; r < kMaxRows; r++) {
        if (r < R) {
          const bf16x8 xv = *(const bf16x8*)(l.xs + (size_t)r * l.stride + blk * 32 + q * 8);
          const float sx = l.sx[blk * 16 + r];
          ag[r] = fmaf(cg, sx, fmaf(sg, dot8_bf16(wg, xv), ag[r]));
          au[r] = fmaf(cu, sx, fmaf(su, dot8_bf16(wu, xv), au[r]));
        }
      }
    }
  }
}

// v summed over the 4 lanes l % 16 + 16 j (j = 0..3), in every one of them: the halves of
// the wave exchange, then neighbouring rows of 16 ((v_j + v_j^2) + (v_j^1 + v_j^3), the
// same float in all four).
__device__ __forceinline__ float sum_q(float v) {
  const int j = (threadIdx.x & 63) >> 4;
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float(j < 2 ? p32[1] : p32[0]);
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v += __uint_as_float((j & 1) ? p16[0] : p16[1]);
  return v;
}

#ifndef SW_GU_VALU
#define SW_GU_VALU 0
#endif
#ifndef SW_GU_PAIR
#define SW_GU_PAIR 1
#endif

// ------------------------------------------------------------------------ gate / up
// Persistent, one workgroup of 8 or 16 waves per compute unit. A worker is a group of S
// waves of one workgroup (S = 2 when the k-groups split evenly and LDS holds the
// partial sums, else 1: a choice made from the shapes alone, so that a row's arithmetic
// is the same in every window); it owns whole items (slot, 16-row ffn tile), and wave p of the group streams k-groups
// [p NG/S, (p+1) NG/S) of the item's gate and up rows through the ring. With S = 2 the
// two partial sums meet in LDS and the second wave to arrive adds them in part order
// (so the result does not depend on which arrives first) and writes h. Items go to
// groups wave-major (item i: workgroup i % grid) so every compute unit gets a share.
//
// Start-up: the activations, the routing tables and the active count are loaded in one
// round; each wave then requests its first ring of weights and only then stages the
// activation image in LDS, so the staging overlaps the weights' flight.

// Waves of a gate/up workgroup: 16 where a wave's registers fit in 128 (bf16 activations
// of at most 4 groups of 8 per thread, i.e. rows * hidden <= 32768; 4-bit weights, or
// 2-bit in the fused layer's kernel), so that one workgroup per compute unit deals the
// items over 2040 two-wave groups; else 8 (1020 groups). The routing core runs once per
// workgroup either way (its rows on waves 0..7). This choice depends on the window's
// rows, so it never decides the k-split: see gateup_plan.
inline bool gu_wants_16(int bits, int x_dtype, int rows, int hidden, bool routed) {
  return (bits == 4 || (bits == 2 && routed)) && x_dtype != 0 && rows * (hidden / 8) <= 4 * 1024;
}
// k-split partials: [wave][parity][lane < 32][8]
constexpr size_t part_bytes(int waves) { return (size_t)waves * 2 * 32 * 8 * 4; }

// The k-split S (1 or 2) from the shapes alone: 2 when the k-groups split evenly and an
// 8-wave workgroup's partial buffers fit next to the activation image, so that a row's
// sums are the same in every window. Then the waves: 16 where gu_wants_16 says so and
// the buffers of 16 waves fit as well (with S = 1 there are none), else 8. Returns the
// dynamic LDS bytes.
static size_t gateup_plan(int hidden, int x_dtype, int bits, int rows, bool routed, size_t static_lds, int& split,
                   int& waves) {
  constexpr size_t kLds = 160 * 1024;
  const size_t image = gateup_lds_bytes(hidden, x_dtype);
  const int NG = hidden / (512 / bits);
  split = (NG % 2 == 0 && image + part_bytes(8) + static_lds <= kLds) ? 2 : 1;
  const size_t parts16 = split == 2 ? part_bytes(16) : 0;
  waves = gu_wants_16(bits, x_dtype, rows, hidden, routed) && image + parts16 + static_lds <= kLds ? 16 : 8;
  return image + (split == 2 ? part_bytes(waves) : 0);
}
size_t route_core_lds_bytes() { return sizeof(RouteLds); }

// s_waitcnt lgkmcnt(0) that the compiler does not move memory operations across
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// The routing core's LDS, present only in the fused layer's gate/up kernel.
template <bool ROUTED>
struct RouteLdsIf {
  RouteLds v;
};
template <>
struct RouteLdsIf<false> {};

// ROUTED: the fused layer. Every workgroup runs the routing core (route_core.h) on the
// router's partials and takes the window's tables from its own LDS (one more
// workgroup, the last, writes the routing outputs and owns no items); otherwise the
// tables come from strata_route_out.
template <int BITS, bool F32IN, int XG, bool ROUTED, int WAVES>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4)))
void k_gateup(GateUpArgs a) {
  constexpr int DEPTH = kGuDepth;
  constexpr int kGuWaves = WAVES, kGuThreads = 64 * kGuWaves;
  static_assert(kGuThreads >= kRouteCoreThreads, "the routing core takes one wave per row");
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_act_g[kMaxSlots];
  __shared__ int s_off_g[kMaxSlots + 1];
  __shared__ uint8_t s_mask_g[kMaxExperts + 4];
  __shared__ RouteLdsIf<ROUTED> rl;
  __shared__ int s_cnt[kGuWaves][2], s_done[kGuWaves][2];   // per group and item parity
  int* s_active;
  int* s_off;
  uint8_t* s_mask;
  if constexpr (ROUTED) {
    s_active = rl.v.active; s_off = rl.v.off; s_mask = rl.v.rmask;
  } else {
    s_active = s_act_g; s_off = s_off_g; s_mask = s_mask_g;
  }
  const int H = a.hidden, F = a.ffn, R = a.rows, E = a.n_experts;
  const int tiles = F / 16;
  // the wave index via readfirstlane: the compiler then knows it (and every count
  // derived from it) is uniform in the wave, and keeps the pipeline's control scalar
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  constexpr int G = 512 / BITS;
  const int NG = H / G;
  // (the fused layer's last workgroup only writes the routing outputs: the others own
  // the items)
  const int grid = ROUTED ? gridDim.x - 1 : gridDim.x;

  // the activations (XG groups of 8 per thread) and the tables, all loads at once
  const ActLds l = act_lds(smem, H, F32IN ? 16 : 8);
  float* const s_part = (float*)(smem + act_lds_bytes(H, F32IN ? 16 : 8));   // k-split partials
  u32x4 xr[XG][F32IN ? 2 : 1];
  int sa = 0, so = 0, act0 = 0, act1 = 0, n_active = 0;
  uint8_t sm = 0;
  if constexpr (ROUTED) {
    // the router's partials (requested first) and the activations; then the routing
    // core, which leaves the window's tables in LDS (two candidate experts per lane up
    // to 128 experts, else four: a branch on the expert count, the same in every wave).
    // The last workgroup also takes the weights and writes the routing outputs, and has
    // no items.
    const bool router = blockIdx.x == gridDim.x - 1;
    if (E <= 2 * kWave) {
      RouteRegs<2> rg;
      route_load<2>(a.route, rg);
      load_groups<kGuThreads, XG, F32IN>(xr, a.x, R, H);
      __builtin_amdgcn_sched_barrier(0);
      route_select<2>(a.route, rg, rl.v, router);
    } else {
      RouteRegs<4> rg;
      route_load<4>(a.route, rg);
      load_groups<kGuThreads, XG, F32IN>(xr, a.x, R, H);
      __builtin_amdgcn_sched_barrier(0);
      route_select<4>(a.route, rg, rl.v, router);
    }
    if (router) return;
    n_active = __builtin_amdgcn_readfirstlane(rl.v.n_active);
  } else {
    load_groups<kGuThreads, XG, F32IN>(xr, a.x, R, H);
    sa = a.active[min(tid, a.max_slots - 1)];
    so = a.offsets[min(tid, a.max_slots)];
    sm = a.row_mask[min(tid, E)];
    // every wave's own copy of the active list (lane i: slots i and 64 + i), for the
    // experts of its first units before the LDS tables exist
    act0 = a.active[min(lane, a.max_slots - 1)];
    act1 = a.active[min(64 + lane, a.max_slots - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // the active count: a wave-uniform scalar load in the same round
    n_active = __builtin_amdgcn_readfirstlane(*a.n_active);
  }
  const int S = a.split;
  const int gw = kGuWaves / S;                     // groups per workgroup
  // part of the k-range and group in the workgroup: a group's waves are adjacent
  // (wave S gl + p), so that the hardware's round-robin placement puts them on different
  // SIMDs and a workgroup's first items spread over all four
  const int part = wave % S, gl = wave / S;
  const int Wg = grid * gw;                        // groups
  const int me = gl * grid + blockIdx.x;           // this wave's group
  const int NGs = NG / S;                          // k-groups per part
  const int items = n_active * tiles;
  const int my_items = me < items ? (items - me + Wg - 1) / Wg : 0;
  const int units = my_items * NGs;

  // issue side of the ring: the next unit is k-group part * NGs + is_g of item ordinal
  // is_j, whose tiles are rg / ru; past the last item it stays on the last one
  KGroup<BITS> kgg[DEPTH], kgu[DEPTH];
  int is_j = 0, is_g = 0;
  TileRsrc rg, ru;
  auto set_item = [&](int expert, int j) __attribute__((always_inline)) {
    const int tile = (me + j * Wg) % tiles;
    expert = clamp_expert(expert, E);
    rg = tile_rsrc<BITS>(a.gate, expert, E, tile, NG);
    ru = tile_rsrc<BITS>(a.up, expert, E, tile, NG);
  };
  auto issue_next = [&](auto d_, auto&& expert_of) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    load_kgroup<BITS>(kgg[d], rg, part * NGs + is_g);
    load_kgroup<BITS>(kgu[d], ru, part * NGs + is_g);
    if (++is_g == NGs) {
      is_g = 0;
      if (is_j + 1 < my_items) {
        ++is_j;
        set_item(expert_of(is_j), is_j);
      }
    }
  };
  // The first ring of weights is requested as soon as this round's loads are back (the
  // experts come from the wave's copy of the active list); the activation image, the
  // tables and the split counters go into LDS while those weights are in flight. A wave
  // without items takes a path of its own, so that in the working one the compiler sees
  // exactly the weight loads issued after the round and waits for the round only.
  auto stage = [&]() __attribute__((always_inline)) {
    if constexpr (!ROUTED) {
      if (tid < a.max_slots) s_active[tid] = sa;
      if (tid <= a.max_slots) s_off[tid] = so;
      if (tid <= E) s_mask[tid] = sm;
    }
    if (tid < kGuWaves * 2) { (&s_cnt[0][0])[tid] = 0; (&s_done[0][0])[tid] = 0; }
    zero_absent<kGuThreads>(l, H, R, F32IN);
    stage_groups<kGuThreads, XG, F32IN>(l, xr, R, H);   // the launcher picks XG to cover all groups
  };
  if (units == 0) {
    stage();
    __syncthreads();
    return;
  }
  auto reg_of = [&](int j) __attribute__((always_inline)) {
    const int slot = min((me + j * Wg) / tiles, a.max_slots - 1);
    if constexpr (ROUTED)   // the tables are already in LDS
      return __builtin_amdgcn_readfirstlane(s_active[slot]);
    else
      return slot < 64 ? __builtin_amdgcn_readlane(act0, slot) : __builtin_amdgcn_readlane(act1, slot - 64);
  };
  set_item(reg_of(0), 0);
  static_for<DEPTH>([&](auto d) __attribute__((always_inline)) { issue_next(d, reg_of); });
  __builtin_amdgcn_sched_barrier(0);
  stage();
  __syncthreads();
  // from here on, the expert of item ordinal j comes from the LDS table
  auto lds_of = [&](int j) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(s_active[min((me + j * Wg) / tiles, kMaxSlots - 1)]);
  };

  const int c = lane & 15, q = lane >> 4;
  const ActLane al = act_lane(l, (c & 7) < R && (c < 8 || F32IN));
  const CodeConsts cc = code_consts();
  constexpr bool VALU = SW_GU_VALU && !F32IN;   // the dot-product form (comparison builds)
  constexpr bool PAIR = SW_GU_PAIR && !F32IN && !VALU;   // two blocks per accumulator tile
  const ActLanePair alp = act_lane_pair(l, R);
  uint32_t sel2[2];   // 2-bit half selectors of MFMA 0 and 1 (lanes 32..63 start on the odd block)
  sel2[0] = lane >= 32 ? 0x0C030C02u : 0x0C010C00u;
  sel2[1] = lane >= 32 ? 0x0C010C00u : 0x0C030C02u;
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f}, mg = ag, mu = ag;
  // the min terms accumulate apart from the scale FMAs (mg, mu), except where the
  // registers would not hold them (2-bit float input at the largest activation sets)
  constexpr bool SEP_MIN = !(BITS == 2 && F32IN && XG >= 16);
  float ag8[kMaxRows], au8[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; r++) { ag8[r] = 0.f; au8[r] = 0.f; }
  int cu_j = 0, cu_g = 0;
  // h = silu(gate) * up for the item's rows, from the finished sums (lanes < 32 hold
  // rows 0..7), split into its bf16 hi and lo parts (hi | lo << 16, one word) and stored
  // at the input's place in its group of 8, the order the down kernel stages
  const int f_pos = tile_pos(c);
  auto write_h = [&](const f32x4& gs, const f32x4& us) __attribute__((always_inline)) {
    const int item = me + cu_j * Wg;
    const int slot = item / tiles, tile = item % tiles, e = s_active[slot];
    const uint32_t rmask = s_mask[e];
    const int ent0 = s_off[slot];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 4 * q + i;
      if (r < R && ((rmask >> r) & 1u)) {
        const int ent = ent0 + __builtin_popcount(rmask & ((1u << r) - 1u));
        const float gv = gs[i];
        const float hv = gv / (1.f + expf(-gv)) * us[i];
        const uint32_t hi = f32_to_bf16(hv);
        const uint32_t lo = f32_to_bf16(hv - bf16_to_f32((uint16_t)hi));
        a.h_hi[(long)ent * F + tile * 16 + f_pos] = (uint16_t)hi;
        a.h_lo[(long)ent * F + tile * 16 + f_pos] = (uint16_t)lo;
      }
    }
  };
  // after this wave's last k-group of an item
  auto finish_item = [&]() __attribute__((always_inline)) {
    if constexpr (VALU) {
      // the 4 lanes of each weight row summed; lanes of j = 0, 1 then hold rows 4j .. 4j + 3
      // as the matrix-core form's accumulators do
#pragma unroll
      for (int r = 0; r < kMaxRows; r++) {
        ag8[r] = sum_q(ag8[r]);
        au8[r] = sum_q(au8[r]);
      }
      // (a select by mask bits: a plain select of the two elements becomes a load from a
      // selected address and sends the arrays to scratch memory)
      const uint32_t odd = 0u - (uint32_t)(q & 1);
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ag[i] = __uint_as_float((__float_as_uint(ag8[4 + i]) & odd) | (__float_as_uint(ag8[i]) & ~odd));
        au[i] = __uint_as_float((__float_as_uint(au8[4 + i]) & odd) | (__float_as_uint(au8[i]) & ~odd));
      }
#pragma unroll
      for (int r = 0; r < kMaxRows; r++) { ag8[r] = 0.f; au8[r] = 0.f; }
    } else if constexpr (SEP_MIN) {
      // the min terms' accumulators (kept apart so that the scale FMAs of the next blocks
      // do not wait for each k-group's fp32 MFMA)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ag[i] += mg[i];
        au[i] += mu[i];
      }
      mg = f32x4{0.f, 0.f, 0.f, 0.f};
      mu = mg;
    }
    if constexpr (F32IN || PAIR) {
      // float x: hi column r (lanes 0..31) + lo column 8 + r; paired form: row r against
      // the even blocks + the odd blocks
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ag[i] += __shfl_down(ag[i], 32);
        au[i] += __shfl_down(au[i], 32);
      }
    }   // (bf16 x otherwise: the lo columns read the zero row and hold exact zeros)
    if (S == 1) {
      if (lane < 32) write_h(ag, au);
    } else {
      const int par = cu_j & 1;
      // the buffers of this parity were last used by item cu_j - 2: wait until its
      // last arriver has read them
      // (relaxed atomic loads: a volatile one would make the compiler wait for every
      // outstanding weight load as well)
      if (cu_j >= 2)
        while (__builtin_amdgcn_readfirstlane(__hip_atomic_load(&s_done[gl][par], __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_WORKGROUP)) < cu_j - 1) {}
      float* mine = s_part + ((size_t)(wave * 2 + par) * 32 + lane) * 8;
      if (lane < 32) {
        *(f32x4*)mine = ag;
        *(f32x4*)(mine + 4) = au;
      }
      lds_wait();   // the partial is in LDS before the arrival is counted
      int old = 0;
      if (lane == 0) old = __hip_atomic_fetch_add(&s_cnt[gl][par], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      old = __builtin_amdgcn_readfirstlane(old);
      asm volatile("" ::: "memory");   // no LDS read is hoisted above the arrival
      if (old % 2 == 1) {   // second to arrive: part 0 + part 1, in that order
        if (lane < 32) {
          const float* p0 = s_part + ((size_t)(gl * S * 2 + par) * 32 + lane) * 8;         // wave S gl: part 0
          const float* p1 = s_part + ((size_t)((gl * S + 1) * 2 + par) * 32 + lane) * 8;   // wave S gl + 1: part 1
          const f32x4 g0 = *(const f32x4*)p0, u0 = *(const f32x4*)(p0 + 4);
          const f32x4 g1 = *(const f32x4*)p1, u1 = *(const f32x4*)(p1 + 4);
          f32x4 gs, us;
#pragma unroll
          for (int i = 0; i < 4; i++) {
            gs[i] = g0[i] + g1[i];
            us[i] = u0[i] + u1[i];
          }
          write_h(gs, us);
        }
        lds_wait();   // both partials are read before the buffers are released
        if (lane == 0) __hip_atomic_store(&s_done[gl][par], cu_j + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    ag = f32x4{0.f, 0.f, 0.f, 0.f};
    au = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  run_ring<DEPTH>(units, [&](auto d_, bool refill) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    if constexpr (VALU)
      mac_kgroup_valu<BITS>(kgg[d], kgu[d], l, R, part * NGs + cu_g, cc, ag8, au8);
    else if constexpr (PAIR)
      mac_kgroup_pair<BITS, true>(kgg[d], kgu[d], alp, part * NGs + cu_g, cc, sel2, ag, au, SEP_MIN ? mg : ag,
                                  SEP_MIN ? mu : au);
    else
      mac_kgroup<BITS, true>(kgg[d], kgu[d], al, part * NGs + cu_g, cc, ag, au, SEP_MIN ? mg : ag, SEP_MIN ? mu : au);
    if (refill) issue_next(d_, lds_of);
    if (++cu_g == NGs) {
      finish_item();
      cu_g = 0;
      ++cu_j;
    }
  });
}

// ----------------------------------------------------------------------------- down
// Down, then the combine. A k_down workgroup serves one expert slot (the workgroups of a
// slot split its output tiles) and stages that expert's h once; y is written per entry at
// its place in its row's ascending list of experts, and k_combine adds each row's list in
// order (routed experts ascending, the shared expert last, with combine_one), then the
// residual. In the stack, k_combine_route (route.hip) takes the combine's place between
// layers. Every sum is a function of the row's own values, so a row is the same in any
// window.
//
// h comes from gate/up as two bf16 arrays (hi, and the rounding of the remainder lo),
// [entries][ffn], inputs permuted within each group of 8 as the code conversion orders
// them; the block sums Sx the min term needs are formed while staging, in LDS.


// k_down: persistent, 16 waves per compute unit (one 16-wave workgroup, or two of 8 for
// small windows: dn_waves_of), so that each (slot, output tile) item gets a wave of its
// own at the usual shapes; workgroup b serves expert slot b % n_active (the
// workgroups of a slot split its output tiles) and stages that expert's h once; each
// wave streams whole 16-row output tiles through the ring. y is written for each of the
// expert's rows at that row's place in its ascending list of experts; k_combine sums
// each row's list in order. As in gate/up, h (from L2) is staged in LDS while the first
// weights are in flight.

size_t down_lds_bytes(int ffn) { return act_lds_bytes(ffn, 16); }

// Waves of a down workgroup: 16 (one workgroup per compute unit) for windows of more than
// 4 rows, 8 (two per compute unit, each staging its slot's h) for smaller ones, measured
// faster there; a tile's arithmetic is the same in both, so the choice changes no bit.
inline int dn_waves_of(int rows) { return rows <= 4 ? 8 : 16; }

// 8 inputs of row j already split into bf16 hi and lo in the image order: stored as
// they are, and the block sums add the group's values in image order, then over the 4
// lanes of the block (the layout of ActLds: hi rows 0..7, lo rows 8..15).
__device__ __forceinline__ void stage_group_split(const ActLds& l, bool ok, int j, int u, const u32x4& wh,
                                                  const u32x4& wl) {
  float shi = 0.f, slo = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e++) {
    const uint32_t h = wh[e >> 1], lo = wl[e >> 1];
    shi += __uint_as_float((e & 1) ? (h & 0xFFFF0000u) : (h << 16));
    slo += __uint_as_float((e & 1) ? (lo & 0xFFFF0000u) : (lo << 16));
  }
  shi = quad_sum(shi);
  slo = quad_sum(slo);
  if (ok) {
    *(u32x4*)(l.xs + (size_t)j * l.stride + 8 * u) = wh;
    *(u32x4*)(l.xs + (size_t)(8 + j) * l.stride + 8 * u) = wl;
    if ((u & 3) == 0) {
      l.sx[(u >> 2) * 16 + j] = shi;
      l.sx[(u >> 2) * 16 + 8 + j] = slo;
    }
  }
}

template <int BITS, int XG, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void k_down(DownArgs a) {
  constexpr int DEPTH = kDnDepth;
  constexpr int kDnWaves = WAVES, kDnThreads = 64 * WAVES;
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_ydst[kMaxRows];
  const int H = a.hidden, F = a.ffn, E = a.n_experts;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  constexpr int G = 512 / BITS;
  const int NG = F / G;
  const int tiles_h = H / 16;

  // one round: the active count (scalar) and the slot tables (lane i: slots i, 64 + i)
  const int ms = a.max_slots;
  const int act0 = a.active[min(lane, ms - 1)], act1 = a.active[min(64 + lane, ms - 1)];
  const int off0 = a.offsets[min(lane, ms)], off1 = a.offsets[min(64 + lane, ms)];
  const int n_active = __builtin_amdgcn_readfirstlane(*a.n_active);
  const int slot = blockIdx.x % n_active;
  auto pick = [&](int v0, int v1, int i) __attribute__((always_inline)) {
    return i < 64 ? __builtin_amdgcn_readlane(v0, i) : __builtin_amdgcn_readlane(v1, i - 64);
  };
  const int e = clamp_expert(pick(act0, act1, slot), E);
  const int e0 = pick(off0, off1, slot), ne = pick(off0, off1, slot + 1) - e0;
  // workgroups of this slot: b = slot + k * n_active, k < nw
  const int k = blockIdx.x / n_active;
  const int nw = (gridDim.x - slot + n_active - 1) / n_active;
  // this wave's tiles: t = wave * nw + k + j * (nw * 16), one to one onto 0 .. nw * 16 - 1
  // and its repeats; interleaved so that the slot's tiles spread over all its workgroups
  // (every compute unit streams) instead of filling the first ones
  const int stride = nw * kDnWaves, t0 = wave * nw + k;
  const int my_tiles = t0 < tiles_h ? (tiles_h - t0 + stride - 1) / stride : 0;
  const int units = my_tiles * NG;

  // the expert's h as gate/up wrote it (XG groups of 8 inputs per thread, hi and lo:
  // group i is row i / (F/8), inputs 8 (i % (F/8)) ..), and where each of its entries' y
  // goes: row r's list of experts in ascending id order, position entry_pos
  const ActLds l = act_lds(smem, F, 16);
  const int ngrp = F / 8, total = max(ne, 1) * ngrp;
  u32x4 hr[XG][2];
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int i = min(it * kDnThreads + tid, total - 1);
    const long at = (long)(e0 + i / ngrp) * F + 8 * (i % ngrp);
    hr[it][0] = *(const u32x4*)(a.h_hi + at);
    hr[it][1] = *(const u32x4*)(a.h_lo + at);
  }
  const int ej = e0 + min(lane, max(ne, 1) - 1);
  const int dst_row = a.entry_row[ej], dst_pos = a.entry_pos[ej];
  __builtin_amdgcn_sched_barrier(0);

  // then the first ring of weights (h and the entry table, requested first, come back
  // first), and h goes into LDS while the weights are in flight; a wave without tiles
  // takes a path of its own (as in gate/up)
  auto stage = [&]() __attribute__((always_inline)) {
    if (tid < kMaxRows) s_ydst[tid] = dst_row * (a.top_k + 1) + dst_pos;
    zero_absent<kDnThreads>(l, F, ne, true);
    const int total_e = ne * ngrp;   // the launcher picks XG to cover them
#pragma unroll
    for (int it = 0; it < XG; it++) {
      const int base = it * kDnThreads;
      if (base >= total_e) break;
      const int i = base + tid;
      stage_group_split(l, i < total_e, i < total_e ? i / ngrp : 0, i < total_e ? i % ngrp : 0, hr[it][0], hr[it][1]);
    }
  };
  if (units == 0) {
    stage();
    __syncthreads();
    return;
  }
  KGroup<BITS> kg[DEPTH];
  int is_j = 0, is_g = 0;
  TileRsrc pd = tile_rsrc<BITS>(a.down, e, E, t0, NG);
  auto issue_next = [&](auto d_) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    load_kgroup<BITS>(kg[d], pd, is_g);
    if (++is_g == NG) {
      is_g = 0;
      if (is_j + 1 < my_tiles) {
        ++is_j;
        pd = tile_rsrc<BITS>(a.down, e, E, t0 + is_j * stride, NG);
      }
    }
  };
  static_for<DEPTH>([&](auto d) __attribute__((always_inline)) { issue_next(d); });
  __builtin_amdgcn_sched_barrier(0);
  stage();
  __syncthreads();

  const int c = lane & 15, q = lane >> 4;
  const ActLane al = act_lane(l, (c & 7) < ne);
  const CodeConsts cc = code_consts();
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, mn = acc;
  int cu_j = 0, cu_g = 0;
  run_ring<DEPTH>(units, [&](auto d_, bool refill) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    mac_kgroup<BITS, false>(kg[d], kg[d], al, cu_g, cc, acc, acc, mn, mn);
    if (refill) issue_next(d_);
    if (++cu_g == NG) {
      const int tile = t0 + cu_j * stride;
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] += mn[i];   // the min terms, accumulated apart
      mn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] += __shfl_down(acc[i], 32);
      if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int j = 4 * q + i;
          if (j < ne) a.y[(long)s_ydst[j] * H + tile * 16 + c] = acc[i];
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      cu_g = 0;
      ++cu_j;
    }
  });
}

// ------------------------------------------------------------------------ combine
// Thread = 2 consecutive outputs of one row: the row's k + 1 expert outputs are already
// in its list order (routed experts ascending, the shared expert last) in y, and its
// weights in the same order in row_w, so every load is issued at once (clamped; slots
// past k + 1 are not summed), then the fixed-order sum and the residual.

// 64 threads per workgroup: the combine is a few hundred KB, so more, smaller workgroups
// spread its loads over more compute units (measured 0.2 us per window faster than 256)
constexpr int kCombineThreads = 64, kCombineVec = 2;

template <bool F32IN>
__global__ __launch_bounds__(kCombineThreads) void k_combine(DownArgs a) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int H = a.hidden, R = a.rows, K1 = a.top_k + 1;
  const int HV = H / kCombineVec;
  const int t = blockIdx.x * kCombineThreads + threadIdx.x;
  if (t >= R * HV) return;
  const int r = t / HV, n = kCombineVec * (t % HV);
  float w[kMaxTopk + 1];
  f32x2 yv[kMaxTopk + 1];
#pragma unroll
  for (int j = 0; j <= kMaxTopk; j++) {
    const int jj = min(j, K1 - 1);
    w[j] = a.row_w[r * K1 + jj];
    yv[j] = *(const f32x2*)(a.y + (long)(r * K1 + jj) * H + n);
  }
  float res[2] = {0.f, 0.f};
  if (a.x_res) {
    if constexpr (F32IN) {
      const f32x2 v = *(const f32x2*)((const float*)a.x_res + (long)r * H + n);
      res[0] = v[0]; res[1] = v[1];
    } else {
      const uint32_t v = *(const uint32_t*)((const uint16_t*)a.x_res + (long)r * H + n);
      res[0] = bf16_to_f32((uint16_t)v); res[1] = bf16_to_f32((uint16_t)(v >> 16));
    }
  }
  f32x2 o;
#pragma unroll
  for (int i = 0; i < 2; i++) {
    float yi[kMaxTopk + 1];
#pragma unroll
    for (int j = 0; j <= kMaxTopk; j++) yi[j] = yv[j][i];
    o[i] = combine_one(w, yi, K1, a.x_res != nullptr, res[i]);
  }
  if (a.out) *(f32x2*)(a.out + (long)r * H + n) = o;
  if (a.x_next)
    *(uint32_t*)(a.x_next + (long)r * H + n) = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
}

// ------------------------------------------------------------------------ launchers


// Persistent grids: resident workgroups per compute unit (occupancy of the kernel at
// this block and LDS size, capped by per_cu_max) times the compute units, never more
// than the window can use. Cached per kernel and LDS size, once per process (every GPU
// a process drives is taken to be the same model); the caches are locked, so host
// threads may launch at once.
static int compute_units() {
  static std::mutex m;
  static int cus = 0;
  std::lock_guard<std::mutex> lock(m);
  if (!cus) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return cus;
}

// Workgroups of `kernel` one compute unit holds at this block and LDS size (at least 1).
template <auto kernel>
static int per_cu(int threads, size_t lds) {
  static std::mutex m;
  static size_t cached_lds = 0;
  static int n = 0;
  std::lock_guard<std::mutex> lock(m);
  if (!n || cached_lds != lds) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess || n <= 0) n = 1;
    cached_lds = lds;
  }
  return n;
}

template <auto kernel>
static int persistent_grid(int threads, size_t lds, int max_items, int per_cu_max) {
  const int n = per_cu<kernel>(threads, lds);
  const int resident = compute_units() * (n < per_cu_max ? n : per_cu_max);
  return max_items < resident ? max_items : resident;
}

template <int BITS, bool F32IN, int XG, bool ROUTED, int WAVES = 8>
static int launch_gateup_k(const GateUpArgs& a, size_t lds, int items, hipStream_t s, const Prof* p) {
  auto kern = k_gateup<BITS, F32IN, XG, ROUTED, WAVES>;
  constexpr int threads = 64 * WAVES;
  if (int e = set_lds<k_gateup<BITS, F32IN, XG, ROUTED, WAVES>>(lds)) return e;
  // One workgroup per compute unit. The fused layer has one more workgroup, which writes
  // the routing outputs: when the grid would fill every slot the compute units hold, the
  // items get one slot fewer, so that the extra one starts with the others instead of
  // after the first to finish.
  const int capacity = compute_units() * per_cu<k_gateup<BITS, F32IN, XG, ROUTED, WAVES>>(threads, lds);
  int grid = persistent_grid<k_gateup<BITS, F32IN, XG, ROUTED, WAVES>>(threads, lds, items, 1);
  if (ROUTED && grid + 1 > capacity) grid = capacity - 1;
  grid += ROUTED ? 1 : 0;
  launch(kern, dim3(grid), dim3(threads), lds, s, p, a);
  return 0;
}

template <int BITS, bool F32IN, bool ROUTED>
static int launch_gateup_x(const GateUpArgs& a, size_t lds, int waves, int items, hipStream_t s, const Prof* p) {
  // activation groups of 8 per thread, all loaded up front (rows * hidden / 8 <= 16 * 512
  // for every hidden whose image fits in LDS); 16 waves where gateup_plan says so
  constexpr int kGuThreads = 64 * 8;
  const int groups = a.rows * (a.hidden / 8);
  if constexpr ((BITS == 4 || ROUTED) && !F32IN)
    if (waves == 16) return launch_gateup_k<BITS, F32IN, 4, ROUTED, 16>(a, lds, items, s, p);
  if (groups <= 4 * kGuThreads) return launch_gateup_k<BITS, F32IN, 4, ROUTED>(a, lds, items, s, p);
  if (groups <= 8 * kGuThreads) return launch_gateup_k<BITS, F32IN, 8, ROUTED>(a, lds, items, s, p);
  if (groups <= 16 * kGuThreads) return launch_gateup_k<BITS, F32IN, 16, ROUTED>(a, lds, items, s, p);
  return (int)hipErrorInvalidValue;
}

template <bool ROUTED>
static int launch_gateup_any(const GateUpArgs& a0, int max_slots, hipStream_t s, const Prof* p) {
  GateUpArgs a = a0;
  const bool f32 = a.x_dtype == 0;
  const size_t static_lds = 2048 + (ROUTED ? sizeof(RouteLds) : 0);   // (s_cnt, s_done: 256 B at 16 waves)
  int waves = 8;
  const size_t lds = gateup_plan(a.hidden, a.x_dtype, a.bits, a.rows, ROUTED, static_lds, a.split, waves);
  const int items = max_slots * (a.ffn / 16);
  int e;
  if (a.bits == 4)
    e = f32 ? launch_gateup_x<4, true, ROUTED>(a, lds, waves, items, s, p)
            : launch_gateup_x<4, false, ROUTED>(a, lds, waves, items, s, p);
  else
    e = f32 ? launch_gateup_x<2, true, ROUTED>(a, lds, waves, items, s, p)
            : launch_gateup_x<2, false, ROUTED>(a, lds, waves, items, s, p);
  return e ? e : (int)hipGetLastError();
}

int launch_gateup(const GateUpArgs& a, int max_slots, hipStream_t s, const Prof* p) {
  return launch_gateup_any<false>(a, max_slots, s, p);
}

int launch_gateup_routed(const GateUpArgs& a, int max_slots, hipStream_t s, const Prof* p) {
  return launch_gateup_any<true>(a, max_slots, s, p);
}

template <int BITS, int XG, int WAVES>
static int launch_down_k(const DownArgs& a, size_t lds, int max_slots, hipStream_t s, const Prof* p) {
  if (int e = set_lds<k_down<BITS, XG, WAVES>>(lds)) return e;
  // 16 waves per compute unit; at least one workgroup per slot, so that every expert is
  // served
  int grid = persistent_grid<k_down<BITS, XG, WAVES>>(64 * WAVES, lds, 1 << 30, 16 / WAVES);
  if (grid < max_slots) grid = max_slots;
  launch(k_down<BITS, XG, WAVES>, dim3(grid), dim3(64 * WAVES), lds, s, p, a);
  return 0;
}

template <int BITS, int WAVES>
static int launch_down_w(const DownArgs& a, size_t lds, int max_slots, hipStream_t s, const Prof* p) {
  // h groups (8 inputs) of the window's rows per thread, all loaded up front (rows * ffn / 8)
  constexpr int T = 64 * WAVES;
  const int groups = a.rows * (a.ffn / 8);
  if (groups <= 1 * T) return launch_down_k<BITS, 1, WAVES>(a, lds, max_slots, s, p);
  if (groups <= 2 * T) return launch_down_k<BITS, 2, WAVES>(a, lds, max_slots, s, p);
  if (groups <= 4 * T) return launch_down_k<BITS, 4, WAVES>(a, lds, max_slots, s, p);
  return (int)hipErrorInvalidValue;
}

template <int BITS>
static int launch_down_bits(const DownArgs& a, size_t lds, int max_slots, hipStream_t s, const Prof* p) {
  return dn_waves_of(a.rows) == 8 ? launch_down_w<BITS, 8>(a, lds, max_slots, s, p)
                                  : launch_down_w<BITS, 16>(a, lds, max_slots, s, p);
}

int launch_down(const DownArgs& a, hipStream_t s, const Prof* p, bool combine) {
  const size_t lds = down_lds_bytes(a.ffn);
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  if (!combine) p0.stop = p1.stop;
  const int e = a.bits == 4 ? launch_down_bits<4>(a, lds, a.max_slots, s, p ? &p0 : nullptr)
                            : launch_down_bits<2>(a, lds, a.max_slots, s, p ? &p0 : nullptr);
  if (e || !combine) return e;
  const int cg = (a.rows * (a.hidden / kCombineVec) + kCombineThreads - 1) / kCombineThreads;
  if (a.x_dtype == 0)
    launch(k_combine<true>, dim3(cg), dim3(kCombineThreads), 0, s, p ? &p1 : nullptr, a);
  else
    launch(k_combine<false>, dim3(cg), dim3(kCombineThreads), 0, s, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
