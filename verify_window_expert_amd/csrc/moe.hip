// Experts of a verify window: fused dequant gate/up matvec with SwiGLU, then the down
// matvec with the weighted combine of each row's experts and the shared expert.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// the shared expert and every routed expert the rows use are read once per window for
// all of them; "Exactness": a row's arithmetic must not depend on how many rows share
// an expert, so every expert runs the same code for any number of rows.
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
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kThreads = 256;   // 4 waves
constexpr int kMaxKgPerWave = 4;  // k-groups a wave keeps in flight
constexpr int kMaxTopk = 8;
constexpr int kMaxExperts = 256;
constexpr int kMaxSlots = kMaxRows * kMaxTopk + 1;   // routed experts a window can use + shared

// LDS image of the activation operand: rows [nrows][stride] of bf16, inputs permuted
// within each group of 8 as the code conversion orders them, plus block sums Sx
// [blocks][16] (zero for absent columns).
struct ActLds {
  uint16_t* xs;
  float* sx;
  int stride;  // elements per row
};

__device__ __forceinline__ ActLds act_lds(uint8_t* smem, int K, int nrows) {
  ActLds l;
  l.stride = K + 8;
  l.xs = (uint16_t*)smem;
  l.sx = (float*)(smem + (size_t)nrows * l.stride * 2);
  return l;
}

__host__ __device__ inline size_t act_lds_bytes(int K, int nrows) {
  return (size_t)nrows * (K + 8) * 2 + (size_t)(K / 32) * 16 * 4;
}

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
  shi += __shfl_xor(shi, 1);
  shi += __shfl_xor(shi, 2);
  slo += __shfl_xor(slo, 1);
  slo += __shfl_xor(slo, 2);
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

// Zero the block sums (absent columns must read 0). Call before staging, then barrier.
__device__ __forceinline__ void clear_sx(const ActLds& l, int K) {
  for (int i = threadIdx.x; i < (K / 32) * 16; i += kThreads) l.sx[i] = 0.f;
}

// Stage nsrc rows of K activations (float or bf16) as the A operand, MAXI groups of 8
// per thread per pass: all global loads of a pass are issued before any is used.
template <int MAXI, bool F32SRC>
__device__ __forceinline__ void stage_rows(const ActLds& l, const void* src, int nsrc, int K, bool with_lo) {
  const int ngrp = K / 8, total = nsrc * ngrp;
  const int tid = threadIdx.x;
  for (int pass = 0; pass < total; pass += MAXI * kThreads) {
    // unconditional loads with the index clamped into range (issue back to back)
    u32x4 raw[MAXI][F32SRC ? 2 : 1];
#pragma unroll
    for (int it = 0; it < MAXI; it++) {
      const int i = min(pass + it * kThreads + tid, total - 1);
      const int j = i / ngrp, u = i % ngrp;
      if (F32SRC) {
        const u32x4* p = (const u32x4*)((const float*)src + (long)j * K + 8 * u);
        raw[it][0] = p[0];
        raw[it][F32SRC ? 1 : 0] = p[1];
      } else {
        raw[it][0] = *(const u32x4*)((const uint16_t*)src + (long)j * K + 8 * u);
      }
    }
#pragma unroll
    for (int it = 0; it < MAXI; it++) {
      const int base = pass + it * kThreads;
      if (base >= total) break;  // uniform across the workgroup
      const int i = base + tid;
      const bool ok = i < total;
      const int j = ok ? i / ngrp : 0, u = ok ? i % ngrp : 0;
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; e++) {
        if (!ok) v[e] = 0.f;
        else if (F32SRC) {
          // element into a plain variable first: a bit cast of a vector-element
          // expression reads the vector's first element
          const uint32_t w = raw[it][F32SRC ? (e >> 2) : 0][e & 3];
          v[e] = __uint_as_float(w);
        }
        else v[e] = bf16_to_f32((uint16_t)(raw[it][0][e >> 1] >> (16 * (e & 1))));
      }
      stage_group(l, ok, j, u, v, with_lo);
    }
  }
}

__device__ __forceinline__ bf16x8 act_operand(const ActLds& l, bool col_ok, int c, int blk, int q) {
  if (!col_ok) return bf16x8{};
  return *(const bf16x8*)(l.xs + (size_t)c * l.stride + blk * 32 + q * 8);
}

// Weight loads of one k-group of one matrix for this lane (issued, not yet used).
template <int BITS>
struct KGroup {
  static constexpr int NB = 512 / BITS / 32;   // blocks per k-group
  u32x4 codes;
  uint32_t meta[NB];                           // row l%16: (scale | min << 16) per block
  uint32_t mpart[NB / 4];                      // block 4h + l/16 of row l%16
};

template <int BITS>
__device__ __forceinline__ void load_kgroup(KGroup<BITS>& kg, const uint8_t* codes, const uint8_t* meta, int NG,
                                            int tile, int g) {
  constexpr int NB = KGroup<BITS>::NB;
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  const long chunk = (long)tile * NG + g;
  kg.codes = *((const u32x4*)codes + chunk * 64 + lane);
  const uint32_t* mp = (const uint32_t*)meta + (chunk * 16 + c) * NB;
#pragma unroll
  for (int b = 0; b < NB; b += 4) {
    const u32x4 t = *(const u32x4*)(mp + b);
    kg.meta[b] = t[0]; kg.meta[b + 1] = t[1]; kg.meta[b + 2] = t[2]; kg.meta[b + 3] = t[3];
  }
#pragma unroll
  for (int h = 0; h < NB / 4; h++) kg.mpart[h] = mp[4 * h + q];
}

// Accumulate one k-group of one matrix into acc (C layout: column 4*(l/16)+i, row l%16).
template <int BITS>
__device__ __forceinline__ void mac_kgroup(const KGroup<BITS>& kg, const ActLds& l, bool col_ok, int g, f32x4& acc) {
  constexpr int NB = KGroup<BITS>::NB;
  const int lane = threadIdx.x & 63, c = lane & 15, q = lane >> 4;
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int beta = 0; beta < NB; beta++) {
    const bf16x8 ax = act_operand(l, col_ok, c, g * NB + beta, q);
    const bf16x8 bw = BITS == 4 ? q4_to_bf16x8(kg.codes[beta])
                                : q2_to_bf16x8((kg.codes[beta >> 1] >> (16 * (beta & 1))) & 0xFFFFu);
    const f32x4 d = mfma_bf16(ax, bw, z);
    const float s = f16_lo(kg.meta[beta]);
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = fmaf(s, d[i], acc[i]);
  }
#pragma unroll
  for (int h = 0; h < NB / 4; h++) {
    const float sx = l.sx[(g * NB + 4 * h + q) * 16 + c];
    const uint32_t m = kg.mpart[h];
    acc = mfma_f32x4(sx, f16_hi(m) - 128.f * f16_lo(m), acc);
  }
}

// ------------------------------------------------------------------------ gate / up
// Persistent: workgroup b takes the items (slot, 16-row ffn tile) b, b + grid, ... of the
// window's n_active * (ffn / 16) items. It stages the activations once. For every item
// its 4 waves take the k-groups g = wave, wave + 4, ...; their partial sums meet in LDS
// in wave order, and wave 0 writes h = silu(gate) * up for the expert's rows.

template <int BITS>
__global__ __launch_bounds__(kThreads) void k_gateup(GateUpArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ f32x4 red[4][2][64];
  __shared__ int s_active[kMaxSlots];
  __shared__ int s_off[kMaxSlots + 1];
  __shared__ uint8_t s_mask[kMaxExperts + 4];
  const int H = a.hidden, F = a.ffn, R = a.rows, E = a.n_experts;
  const int tiles = F / 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool f32in = a.x_dtype == 0;
  constexpr int G = 512 / BITS;
  const int NG = H / G;

  // round 1: the first item's expert, the active count and every routing table, all at
  // once (clamped loads; the arrays hold max_slots, max_slots + 1 and E + 1 entries)
  int it = blockIdx.x;
  const int n_active = *a.n_active;
  int e = a.active[it / tiles];
  const int sa = a.active[min(tid, a.max_slots - 1)];
  const int so = a.offsets[min(tid, a.max_slots)];
  const uint8_t sm = a.row_mask[min(tid, E)], sm2 = a.row_mask[min(tid + kThreads, E)];
  const int items = n_active * tiles;
  if (it >= items) return;

  // round 2: the first item's weights (this wave's k-groups, clamped loads)
  KGroup<BITS> kgg[kMaxKgPerWave], kgu[kMaxKgPerWave];
  auto mats = [&](int expert, const uint8_t*& gc, const uint8_t*& gm, const uint8_t*& uc, const uint8_t*& um) {
    const bool shared = expert == E;
    gc = shared ? a.gate.sh_codes : a.gate.codes + expert * a.gate.stride_codes;
    gm = shared ? a.gate.sh_meta : a.gate.meta + expert * a.gate.stride_meta_bytes;
    uc = shared ? a.up.sh_codes : a.up.codes + expert * a.up.stride_codes;
    um = shared ? a.up.sh_meta : a.up.meta + expert * a.up.stride_meta_bytes;
  };
  {
    const uint8_t *gc, *gm, *uc, *um;
    mats(e, gc, gm, uc, um);
#pragma unroll
    for (int i = 0; i < kMaxKgPerWave; i++) {
      const int g = min(wave + 4 * i, NG - 1);
      load_kgroup<BITS>(kgg[i], gc, gm, NG, it % tiles, g);
      load_kgroup<BITS>(kgu[i], uc, um, NG, it % tiles, g);
    }
  }
  if (tid < a.max_slots) s_active[tid] = sa;
  if (tid <= a.max_slots) s_off[tid] = so;
  if (tid <= E) s_mask[tid] = sm;
  if (tid + kThreads <= E) s_mask[tid + kThreads] = sm2;

  // activations (L2-resident), staged while the weights stream in
  const ActLds l = act_lds(smem, H, f32in ? 16 : 8);
  clear_sx(l, H);
  __syncthreads();
  if (f32in) stage_rows<4, true>(l, a.x, R, H, true);
  else stage_rows<8, false>(l, a.x, R, H, false);
  __syncthreads();

  const int c = lane & 15, q = lane >> 4;
  const bool col_ok = (c & 7) < R && (c < 8 || f32in);
  for (;;) {
    const int slot = it / tiles, tile = it % tiles;
    const int next = it + gridDim.x;
    const bool more = next < items;
    const int e_next = s_active[min(next, items - 1) / tiles];
    const uint8_t *ngc, *ngm, *nuc, *num;
    mats(e_next, ngc, ngm, nuc, num);
    f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
    // consume each k-group, then refill its registers with the next item's
#pragma unroll
    for (int i = 0; i < kMaxKgPerWave; i++) {
      const int g = wave + 4 * i;
      if (g < NG) {
        mac_kgroup<BITS>(kgg[i], l, col_ok, g, ag);
        mac_kgroup<BITS>(kgu[i], l, col_ok, g, au);
      }
      if (more) {
        const int gn = min(g, NG - 1);
        load_kgroup<BITS>(kgg[i], ngc, ngm, NG, next % tiles, gn);
        load_kgroup<BITS>(kgu[i], nuc, num, NG, next % tiles, gn);
      }
    }
    // k-groups beyond 4 per wave (wider hidden): streamed, same order
    if (NG > 4 * kMaxKgPerWave) {
      const uint8_t *gc, *gm, *uc, *um;
      mats(e, gc, gm, uc, um);
      for (int g = wave + 4 * kMaxKgPerWave; g < NG; g += 4) {
        KGroup<BITS> tg, tu;
        load_kgroup<BITS>(tg, gc, gm, NG, tile, g);
        load_kgroup<BITS>(tu, uc, um, NG, tile, g);
        mac_kgroup<BITS>(tg, l, col_ok, g, ag);
        mac_kgroup<BITS>(tu, l, col_ok, g, au);
      }
    }

    red[wave][0][lane] = ag;
    red[wave][1][lane] = au;
    __syncthreads();
    if (wave == 0) {
      ag = red[0][0][lane]; au = red[0][1][lane];
#pragma unroll
      for (int w = 1; w < 4; w++) {
        const f32x4 tg = red[w][0][lane], tu = red[w][1][lane];
#pragma unroll
        for (int i = 0; i < 4; i++) { ag[i] += tg[i]; au[i] += tu[i]; }
      }
      // hi column r (lanes 0..31) + lo column 8 + r (lanes 32..63)
#pragma unroll
      for (int i = 0; i < 4; i++) {
        ag[i] += __shfl_down(ag[i], 32);
        au[i] += __shfl_down(au[i], 32);
      }
      if (lane < 32) {
        const uint32_t rmask = s_mask[e];
        const int ent0 = s_off[slot];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = 4 * q + i;
          if (r < R && ((rmask >> r) & 1u)) {
            const int ent = ent0 + __builtin_popcount(rmask & ((1u << r) - 1u));
            const float g = ag[i];
            a.h[(long)ent * F + tile * 16 + c] = g / (1.f + expf(-g)) * au[i];
          }
        }
      }
    }
    if (!more) break;
    __syncthreads();   // red is reused by the next item
    it = next;
    e = e_next;
  }
}

// --------------------------------------------------------------------------- down
// Persistent: workgroup b takes the items (slot, 64 output rows) b, b + grid, ...; for
// an item wave w owns the 16-row tile w and all ffn inputs. y[entry][row] is written
// for each of the expert's rows; k_combine sums them.

constexpr int kDownRange = 64;

template <int BITS>
__global__ __launch_bounds__(kThreads) void k_down(DownArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int H = a.hidden, F = a.ffn, E = a.n_experts;
  const int NR = a.n_ranges;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  constexpr int G = 512 / BITS;
  const int NG = F / G;
  constexpr int KMAX = 8;                 // ffn up to 8 k-groups held in flight
  const int tiles_h = H / 16;

  // round 1: the first item's routing
  int it = blockIdx.x;
  const int n_active = *a.n_active;
  int slot = it / NR;
  int e = a.active[slot];
  int e0 = a.offsets[slot], e1 = a.offsets[slot + 1];
  const int items = n_active * NR;
  if (it >= items) return;

  auto mats = [&](int expert, const uint8_t*& dc, const uint8_t*& dm) {
    const bool shared = expert == E;
    dc = shared ? a.down.sh_codes : a.down.codes + expert * a.down.stride_codes;
    dm = shared ? a.down.sh_meta : a.down.meta + expert * a.down.stride_meta_bytes;
  };
  // round 2: the first item's weights (clamped loads: unused copies of the last
  // k-group / tile)
  KGroup<BITS> kg[KMAX];
  {
    const uint8_t *dc, *dm;
    mats(e, dc, dm);
    const int tile = min((it % NR) * 4 + wave, tiles_h - 1);
#pragma unroll
    for (int i = 0; i < KMAX; i++) load_kgroup<BITS>(kg[i], dc, dm, NG, tile, min(i, NG - 1));
  }

  const ActLds l = act_lds(smem, F, 16);
  const int c = lane & 15, q = lane >> 4;
  for (;;) {
    const int nr = it % NR;
    const int tile = nr * 4 + wave;
    const bool has_tile = tile * 16 < H;
    const int ne = e1 - e0;
    clear_sx(l, F);
    __syncthreads();
    stage_rows<4, true>(l, a.h + (long)e0 * F, ne, F, true);
    // the next item's routing, read while this one computes
    const int next = it + gridDim.x;
    const bool more = next < items;
    const int nslot = min(next, items - 1) / NR;
    const int ne_e = a.active[nslot], ne0 = a.offsets[nslot], ne1 = a.offsets[nslot + 1];
    __syncthreads();
    const uint8_t *ndc, *ndm;
    mats(ne_e, ndc, ndm);
    const int ntile = min((next % NR) * 4 + wave, tiles_h - 1);
    const bool col_ok = (c & 7) < ne;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // consume each k-group, then refill its registers with the next item's
#pragma unroll
    for (int i = 0; i < KMAX; i++) {
      if (has_tile && i < NG) mac_kgroup<BITS>(kg[i], l, col_ok, i, acc);
      if (more) load_kgroup<BITS>(kg[i], ndc, ndm, NG, ntile, min(i, NG - 1));
    }
    if (has_tile) {
      if (NG > KMAX) {
        const uint8_t *dc, *dm;
        mats(e, dc, dm);
        for (int g = KMAX; g < NG; g++) {
          KGroup<BITS> t;
          load_kgroup<BITS>(t, dc, dm, NG, tile, g);
          mac_kgroup<BITS>(t, l, col_ok, g, acc);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] += __shfl_down(acc[i], 32);
      if (lane < 32) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int j = 4 * q + i;
          if (j < ne) a.y[(long)(e0 + j) * H + tile * 16 + c] = acc[i];
        }
      }
    }
    if (!more) break;
    __syncthreads();   // the staged h is replaced by the next item's
    it = next; slot = nslot; e = ne_e; e0 = ne0; e1 = ne1;
  }
}

// ------------------------------------------------------------------------ combine
// Workgroup = 64 output rows of every window row: row r's entries in ascending expert
// order (the shared expert last), weighted, then the residual.

template <bool F32IN>
__global__ __launch_bounds__(kThreads) void k_combine(DownArgs a) {
  __shared__ int s_active[kMaxSlots], s_off[kMaxSlots + 1];
  __shared__ uint8_t s_mask[kMaxExperts + 4];
  __shared__ float s_ew[kMaxRows * kMaxTopk + kMaxRows];
  __shared__ int s_list[kMaxRows][kMaxTopk + 2];
  __shared__ float s_w[kMaxRows][kMaxTopk + 2];
  __shared__ int s_cnt[kMaxRows];
  const int H = a.hidden, R = a.rows, E = a.n_experts;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n_active = *a.n_active;
  // every slot's metadata in one round (clamped loads; the arrays hold max_slots,
  // max_slots + 1, E + 1 and R*k + R entries)
  {
    const int sa = a.active[min(tid, a.max_slots - 1)];
    const int so = a.offsets[min(tid, a.max_slots)];
    const uint8_t sm = a.row_mask[min(tid, E)], sm2 = a.row_mask[min(tid + kThreads, E)];
    const int ne = R * a.top_k + R;
    const float ew = a.entry_w[min(tid, ne - 1)];
    if (tid < a.max_slots) s_active[tid] = sa;
    if (tid <= a.max_slots) s_off[tid] = so;
    if (tid <= E) s_mask[tid] = sm;
    if (tid + kThreads <= E) s_mask[tid + kThreads] = sm2;
    if (tid < ne) s_ew[tid] = ew;
    if (tid < kMaxRows * (kMaxTopk + 2)) { (&s_list[0][0])[tid] = 0; (&s_w[0][0])[tid] = 0.f; }
  }
  __syncthreads();
  // row r's entries in ascending expert order: one ballot per row over the slots
  if (wave == 0) {
    int base[kMaxRows] = {0};
    for (int s0 = 0; s0 < n_active; s0 += 64) {
      const int s = s0 + lane;
      const bool ok = s < n_active;
      const uint32_t m = ok ? s_mask[s_active[s]] : 0u;
#pragma unroll
      for (int r = 0; r < kMaxRows; r++) {
        if (r >= R) break;
        const bool has = (m >> r) & 1u;
        const uint64_t bal = __ballot(has);
        if (has) {
          const int pos = base[r] + __popcll(bal & ((1ull << lane) - 1ull));
          const int ent = s_off[s] + __builtin_popcount(m & ((1u << r) - 1u));
          s_list[r][pos] = ent;
          s_w[r][pos] = s_ew[ent];
        }
        base[r] += __popcll(bal);
      }
    }
#pragma unroll
    for (int r = 0; r < kMaxRows; r++)
      if (r < R && lane == r) s_cnt[r] = base[r];
  }
  __syncthreads();
  const int n0 = blockIdx.x * kDownRange;
  for (int idx = tid; idx < R * kDownRange; idx += kThreads) {
    const int r = idx / kDownRange, n = n0 + idx % kDownRange;
    if (n >= H) continue;
    const int cnt = s_cnt[r];
    float yv[kMaxTopk + 2];   // unused slots read entry 0 and are not summed
#pragma unroll
    for (int t = 0; t < kMaxTopk + 2; t++) yv[t] = a.y[(long)s_list[r][t] * H + n];
    const float res = a.x_res ? load_x<F32IN>(a.x_res, (long)r * H + n) : 0.f;
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < kMaxTopk + 2; t++)
      if (t < cnt) s = fmaf(s_w[r][t], yv[t], s);
    if (a.x_res) s += res;
    a.out[(long)r * H + n] = s;
    if (a.x_next) a.x_next[(long)r * H + n] = f32_to_bf16(s);
  }
}

// ------------------------------------------------------------------------ launchers

// Raise a kernel's dynamic LDS limit above the default 64 KB (once per process and
// kernel; the attribute only grows, so a later smaller launch needs nothing).
template <auto kernel>
static int set_lds(size_t bytes) {
  static size_t granted = 64 * 1024;
  if (bytes <= granted) return 0;
  const int e = (int)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == 0) granted = bytes;
  return e;
}

// Persistent grids: as many workgroups as can be resident at once (occupancy of the
// kernel at this LDS size, per compute unit, times the compute units), never more than
// the window can use. Cached per kernel and LDS size.
template <auto kernel>
static int persistent_grid(size_t lds, int max_items) {
  static size_t cached_lds = 0;
  static int resident = 0;
  if (!resident || cached_lds != lds) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kThreads, lds) != hipSuccess || per_cu <= 0)
      per_cu = 1;
    resident = cus * per_cu;
    cached_lds = lds;
  }
  return max_items < resident ? max_items : resident;
}

int launch_gateup(const GateUpArgs& a, int max_slots, hipStream_t s, const Prof* p) {
  const size_t lds = act_lds_bytes(a.hidden, a.x_dtype == 0 ? 16 : 8);
  const int items = max_slots * (a.ffn / 16);
  if (a.bits == 4) {
    if (int e = set_lds<k_gateup<4>>(lds)) return e;
    launch(k_gateup<4>, dim3(persistent_grid<k_gateup<4>>(lds, items)), dim3(kThreads), lds, s, p, a);
  } else {
    if (int e = set_lds<k_gateup<2>>(lds)) return e;
    launch(k_gateup<2>, dim3(persistent_grid<k_gateup<2>>(lds, items)), dim3(kThreads), lds, s, p, a);
  }
  return (int)hipGetLastError();
}

int down_ranges(int hidden) { return (hidden + kDownRange - 1) / kDownRange; }

int launch_down(const DownArgs& a, int max_slots, hipStream_t s, const Prof* p) {
  const size_t lds = act_lds_bytes(a.ffn, 16);
  const int items = max_slots * a.n_ranges;
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  if (a.bits == 4) {
    if (int e = set_lds<k_down<4>>(lds)) return e;
    launch(k_down<4>, dim3(persistent_grid<k_down<4>>(lds, items)), dim3(kThreads), lds, s, p ? &p0 : nullptr, a);
  } else {
    if (int e = set_lds<k_down<2>>(lds)) return e;
    launch(k_down<2>, dim3(persistent_grid<k_down<2>>(lds, items)), dim3(kThreads), lds, s, p ? &p0 : nullptr, a);
  }
  if (a.x_dtype == 0)
    launch(k_combine<true>, dim3(a.n_ranges), dim3(kThreads), 0, s, p ? &p1 : nullptr, a);
  else
    launch(k_combine<false>, dim3(a.n_ranges), dim3(kThreads), 0, s, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
