// Output head of a verify window: 8-bit block-quantized GEMV and per-row argmax.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// a single fetch of the head serves every row of the window; docs/MULTI_GPU.md, "What each card
// holds": it runs on the card that holds the last layers.
//
// Matrix-core formulation, as for the experts but in binary16: a lane's 8 signed codes
// become the exact binary16 values 1152 + q (q + 128 masked into the mantissa of 1024);
// the rows' activations are scaled per row by a power of two that puts the row's largest
// magnitude in [2^14, 2^15) and are then exact in binary16 (bf16 inputs; float inputs
// keep a binary16 remainder column); per block
//     sum_k w x = scale * (D - 1152 * Sx),  D = sum (1152 + q) x.
// A second one-workgroup launch reduces the per-workgroup argmax candidates.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace sw {

// 12 waves per workgroup: at vocabulary 151936 each of the 3072 waves owns 3 or 4 of the
// 9496 tiles (with 8 waves, 4 or 5), and each SIMD keeps three rings in flight
#ifndef SW_HEAD_WAVES
#define SW_HEAD_WAVES 12
#endif
constexpr int kHeadWaves = SW_HEAD_WAVES, kHeadThreads = 64 * kHeadWaves;
#ifndef SW_HEAD_GRID
#define SW_HEAD_GRID 256
#endif
// 4 units in flight per wave (48 KB per compute unit at 12 waves): measured faster than 2,
// 3, 5, 6, 8 and 12
#ifndef SW_HEAD_DEPTH
#define SW_HEAD_DEPTH 4
#endif
constexpr int kHeadGrid = SW_HEAD_GRID;     // workgroups (one per compute unit of the MI355X)
constexpr int kHeadDepth = SW_HEAD_DEPTH;   // units (one 16-row x 64-input chunk) in flight per wave

int head_workgroups(int vocab) {
  const int tiles = (vocab + 15) / 16;
  return std::min(kHeadGrid, (tiles + kHeadWaves - 1) / kHeadWaves);
}

static size_t head_lds_bytes(int H, int rows) {
  return (size_t)rows * (H + 8) * 2 + (size_t)(H / 32) * 16 * 4;
}

// Wave w of workgroup b owns vocabulary tiles (16 rows) t = w * grid + b, + waves ...; it
// streams their (tile, 64-input k-group) chunks through a ring of kHeadDepth units, the
// first ring requested before the activations are staged. Per unit and 32-input block:
// one f16 MFMA D = sum (1152 + q) x times the block's scale; the -1152 * scale * Sx
// terms of the unit's two blocks by one fp32 MFMA on a second accumulator. After a
// tile: logits (optional) and the lanes' running argmax; at the end, the workgroup's
// candidates per row go to the workspace for k_head_argmax.
template <bool F32IN, int XG>
__global__ __launch_bounds__(kHeadThreads) void k_head(HeadArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float s_scale[kMaxRows], s_unscale[kMaxRows];
  __shared__ uint32_t s_maxbits[kMaxRows];
  __shared__ float s_bv[kHeadWaves][kMaxRows];
  __shared__ int s_bi[kHeadWaves][kMaxRows];
  constexpr int D = kHeadDepth;
  const int H = a.hidden, R = a.rows, V = a.vocab;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int c = lane & 15, q = lane >> 4;
  const int nrows = F32IN ? 16 : 8;
  const int stride = H + 8;
  _Float16* xs = (_Float16*)smem;
  float* sx = (float*)(smem + (size_t)nrows * stride * 2);
  const int NG = H / 64;                       // k-groups of 64 inputs = 2 blocks
  const int tiles = V / 16;
  const int TW = gridDim.x * kHeadWaves;
  const int gw = wave * gridDim.x + blockIdx.x;   // wave-major (measured faster than block-major)
  const int my_tiles = gw < tiles ? (tiles - gw + TW - 1) / TW : 0;
  const int units = my_tiles * NG;

  // the activations: XG groups of 8 per thread (group i: row i / (H/8)), all at once
  const int ngrp = H / 8, total = R * ngrp;
  u32x4 xr[XG][F32IN ? 2 : 1];
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int i = min(it * kHeadThreads + tid, total - 1);
    if constexpr (F32IN) {
      const u32x4* p = (const u32x4*)((const float*)a.x + (long)(i / ngrp) * H + 8 * (i % ngrp));
      xr[it][0] = p[0];
      xr[it][F32IN ? 1 : 0] = p[1];
    } else {
      xr[it][0] = *(const u32x4*)((const uint16_t*)a.x + (long)(i / ngrp) * H + 8 * (i % ngrp));
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // the first ring of weights (past the last unit the ring stays on the last tile)
  const u32x4* codes = (const u32x4*)a.codes;
  const uint32_t* meta = (const uint32_t*)a.meta;
  u32x4 rc[D];
  uint32_t rm[D];
  int is_j = 0, is_g = 0;
  auto issue = [&](auto d_) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    const long chunk = (long)(gw + is_j * TW) * NG + is_g;
    // each weight is used by one window only: non-temporal loads (measured faster here)
    rc[d] = __builtin_nontemporal_load(codes + chunk * 64 + lane);
    rm[d] = __builtin_nontemporal_load(meta + chunk * 16 + c);
    if (++is_g == NG) {
      is_g = 0;
      if (is_j + 1 < my_tiles) ++is_j;
    }
  };
  if (units > 0) static_for<D>([&](auto d) __attribute__((always_inline)) { issue(d); });
  __builtin_amdgcn_sched_barrier(0);

  // per-row power-of-two scale (largest magnitude into [2^14, 2^15)), from the loaded
  // groups: each thread's maximum, combined in LDS (magnitudes order as their bits)
  if (tid < kMaxRows) s_maxbits[tid] = 0u;
  for (int i = tid; i < (H / 32) * 16; i += kHeadThreads) sx[i] = 0.f;
  __syncthreads();
  auto group_vals = [&](int it, float (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < 8; e++) {
      if constexpr (F32IN) {
        const uint32_t w = xr[it][e >> 2][e & 3];
        v[e] = __uint_as_float(w);
      } else {
        v[e] = bf16_to_f32((uint16_t)(xr[it][0][e >> 1] >> (16 * (e & 1))));
      }
    }
  };
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int i = it * kHeadThreads + tid;
    if (it * kHeadThreads < total && i < total) {
      float v[8];
      group_vals(it, v);
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e++) m = fmaxf(m, fabsf(v[e]));
      atomicMax(&s_maxbits[i / ngrp], __float_as_uint(m));
    }
  }
  __syncthreads();
  if (tid < R) {
    const float m = __uint_as_float(s_maxbits[tid]);
    int ex = 0;
    if (m > 0.f) frexpf(m, &ex);        // m = f * 2^ex, f in [0.5, 1)
    const int sh = m > 0.f ? 15 - ex : 0;
    s_scale[tid] = ldexpf(1.f, sh);
    s_unscale[tid] = ldexpf(1.f, -sh);
  }
  __syncthreads();

  // stage the binary16 operand (inputs permuted within groups of 8) and the block sums
#pragma unroll
  for (int it = 0; it < XG; it++) {
    const int base = it * kHeadThreads;
    if (base >= total) break;
    const int i = base + tid;
    const bool ok = i < total;
    const int j = ok ? i / ngrp : 0, u = ok ? i % ngrp : 0;
    float v[8];
    group_vals(it, v);
    _Float16 hi[8], lo[8];
    float shi = 0.f, slo = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float sv = ok ? v[e] * s_scale[j] : 0.f;
      hi[e] = (_Float16)sv;
      lo[e] = F32IN ? (_Float16)(sv - (float)hi[e]) : (_Float16)0.f;
      shi += (float)hi[e];
      slo += (float)lo[e];
    }
    shi = quad_sum(shi);
    slo = quad_sum(slo);
    if (ok) {
      f16x8 ph, pl;
#pragma unroll
      for (int e = 0; e < 8; e++) { ph[e] = hi[perm_q8(e)]; pl[e] = lo[perm_q8(e)]; }
      *(f16x8*)(xs + (size_t)j * stride + 8 * u) = ph;
      if (F32IN) *(f16x8*)(xs + (size_t)(8 + j) * stride + 8 * u) = pl;
      if ((u & 3) == 0) {
        sx[(u >> 2) * 16 + j] = shi;
        if (F32IN) sx[(u >> 2) * 16 + 8 + j] = slo;
      }
    }
  }
  __syncthreads();

  const bool col_ok = (c & 7) < R && (c < 8 || F32IN);
  float best_v[4];
  int best_i[4];
#pragma unroll
  for (int i = 0; i < 4; i++) { best_v[i] = -INFINITY; best_i[i] = 0x7FFFFFFF; }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f}, mn = acc;
  int cu_j = 0, cu_g = 0;
  run_ring<D>(units, [&](auto d_, bool refill) __attribute__((always_inline)) {
    constexpr int d = decltype(d_)::value;
    const u32x4 cw = rc[d];
    const uint32_t mw = rm[d];
    if (refill) issue(d_);
#pragma unroll
    for (int beta = 0; beta < 2; beta++) {
      const int blk = 2 * cu_g + beta;
      f16x8 ax = {};
      if (col_ok) ax = *(const f16x8*)(xs + (size_t)c * stride + blk * 32 + q * 8);
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 dd = mfma_f16(ax, q8_to_f16x8(cw[2 * beta], cw[2 * beta + 1]), z);
      const float sc = beta ? f16_hi(mw) : f16_lo(mw);
#pragma unroll
      for (int i = 0; i < 4; i++) acc[i] = fmaf(sc, dd[i], acc[i]);
    }
    // -1152 * scale * Sx of the unit's blocks: lane (k = l/16 < 2) supplies block 2g + k
    const float am = q < 2 ? sx[(2 * cu_g + q) * 16 + c] : 0.f;
    const float bm = q == 0 ? -1152.f * f16_lo(mw) : (q == 1 ? -1152.f * f16_hi(mw) : 0.f);
    mn = mfma_f32x4(am, bm, mn);
    if (++cu_g == NG) {
      f32x4 tot;
#pragma unroll
      for (int i = 0; i < 4; i++) tot[i] = acc[i] + mn[i];
      if constexpr (F32IN) {
#pragma unroll
        for (int i = 0; i < 4; i++) tot[i] += __shfl_down(tot[i], 32);
      }
      if (lane < 32) {
        const int v = (gw + cu_j * TW) * 16 + c;
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = 4 * q + i;
          if (r < R) {
            const float val = tot[i] * s_unscale[r];
            if (a.logits) a.logits[(long)r * V + v] = val;
            if (val > best_v[i] || (val == best_v[i] && v < best_i[i])) { best_v[i] = val; best_i[i] = v; }
          }
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
      mn = acc;
      cu_g = 0;
      ++cu_j;
    }
  });
  // reduce candidates over the 16 lanes of each row group (columns = vocab)
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float ov = __shfl_xor(best_v[i], off);
      const int oi = __shfl_xor(best_i[i], off);
      if (ov > best_v[i] || (ov == best_v[i] && oi < best_i[i])) { best_v[i] = ov; best_i[i] = oi; }
    }
  }
  if (lane < 32 && c == 0) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int r = 4 * q + i;
      if (r < R) { s_bv[wave][r] = best_v[i]; s_bi[wave][r] = best_i[i]; }
    }
  }
  __syncthreads();
  if (tid < R) {
    float bv = s_bv[0][tid];
    int bi = s_bi[0][tid];
    for (int w = 1; w < kHeadWaves; w++)
      if (s_bv[w][tid] > bv || (s_bv[w][tid] == bv && s_bi[w][tid] < bi)) { bv = s_bv[w][tid]; bi = s_bi[w][tid]; }
    a.part_val[(long)blockIdx.x * R + tid] = bv;
    a.part_idx[(long)blockIdx.x * R + tid] = bi;
  }
}

// Per-row argmax over the workgroups' candidates (one workgroup, after k_head): wave r
// takes row r, every lane loading all its candidates at once (past the last workgroup,
// the last one's again: a repeated candidate does not change an argmax), then a reduction
// over the lanes; ties go to the lower index throughout.
constexpr int kArgmaxPerLane = (kHeadGrid + kWave - 1) / kWave;
__global__ __launch_bounds__(kMaxRows * kWave) void k_head_argmax(HeadArgs a, int nwg) {
  const int R = a.rows, r = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (r >= R) return;
  float v[kArgmaxPerLane];
  int id[kArgmaxPerLane];
#pragma unroll
  for (int j = 0; j < kArgmaxPerLane; j++) {
    const long w = min(lane + kWave * j, nwg - 1);
    v[j] = a.part_val[w * R + r];
    id[j] = a.part_idx[w * R + r];
  }
  float bv = v[0];
  int bi = id[0];
#pragma unroll
  for (int j = 1; j < kArgmaxPerLane; j++)
    if (v[j] > bv || (v[j] == bv && id[j] < bi)) { bv = v[j]; bi = id[j]; }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
  }
  if (lane == 0) a.argmax[r] = bi;
}

// Greedy verification of the window's proposals (Strata docs/BATCHING.md, --batch-mtp
// paragraph; docs/MULTI_GPU.md, --pipeline-windows paragraph): one wave, lane s = slot s.
// With mtp, slot s owns rows 2s (its token) and 2s + 1 (its proposal). The proposal is
// kept when it equals the head's argmax of the token row; the slot then emits it and
// the argmax of the proposal row, else the token row's argmax alone.
__global__ __launch_bounds__(kWave) void k_accept(AcceptArgs a) {
  const int s = threadIdx.x;
  bool kept = false;
  if (s < a.n_slots) {
    const int32_t first = a.argmax[a.mtp ? 2 * s : s];
    int32_t second = -1;
    if (a.mtp) {
      const int32_t prop = a.proposal[s], bonus = a.argmax[2 * s + 1];
      kept = prop == first;
      if (kept) second = bonus;
    }
    a.tokens[2 * s] = first;
    a.tokens[2 * s + 1] = second;
    a.n_tokens[s] = kept ? 2 : 1;
  }
  const uint64_t b = __ballot(kept);
  if (s == 0) *a.n_accepted = (int32_t)__popcll(b);
}

int launch_accept(const AcceptArgs& a, hipStream_t s, const Prof* p) {
  launch(k_accept, dim3(1), dim3(kWave), 0, s, p, a);
  return (int)hipGetLastError();
}

template <bool F32IN, int XG>
static int launch_head_k(const HeadArgs& a, size_t lds, int nwg, hipStream_t s, const Prof* p) {
  if (int e = set_lds<k_head<F32IN, XG>>(lds)) return e;
  launch(k_head<F32IN, XG>, dim3(nwg), dim3(kHeadThreads), lds, s, p, a);
  return 0;
}

template <bool F32IN>
static int launch_head_x(const HeadArgs& a, size_t lds, int nwg, hipStream_t s, const Prof* p) {
  // activation groups of 8 per thread, all loaded up front
  const int groups = a.rows * (a.hidden / 8);
  if (groups <= 4 * kHeadThreads) return launch_head_k<F32IN, 4>(a, lds, nwg, s, p);
  if (groups <= 8 * kHeadThreads) return launch_head_k<F32IN, 8>(a, lds, nwg, s, p);
  if (groups <= 16 * kHeadThreads) return launch_head_k<F32IN, 16>(a, lds, nwg, s, p);
  return (int)hipErrorInvalidValue;
}

int launch_head(const HeadArgs& a, hipStream_t s, const Prof* p) {
  const size_t lds = head_lds_bytes(a.hidden, a.x_dtype == 0 ? 16 : 8);
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  const int nwg = head_workgroups(a.vocab);
  const int e = a.x_dtype == 0 ? launch_head_x<true>(a, lds, nwg, s, p ? &p0 : nullptr)
                               : launch_head_x<false>(a, lds, nwg, s, p ? &p0 : nullptr);
  if (e) return e;
  launch(k_head_argmax, dim3(1), dim3(kMaxRows * kWave), 0, s, p ? &p1 : nullptr, a, nwg);
  return (int)hipGetLastError();
}

}  // namespace sw
