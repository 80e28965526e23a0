// Output head of a verify window: 8-bit block-quantized GEMV and per-row argmax.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// the head is read once per window for all its rows; docs/MULTI_GPU.md, "What each card
// holds": it runs on the card that holds the last layers.
//
// Matrix-core formulation, as for the experts but in binary16: a lane's 8 signed codes
// become the exact binary16 values 1152 + q (q + 128 masked into the mantissa of 1024);
// the rows' activations are scaled per row by a power of two that puts the row's largest
// magnitude in [2^14, 2^15) and are then exact in binary16 (bf16 inputs; float inputs
// keep a binary16 remainder column); per block
//     sum_k w x = scale * (D - 1152 * Sx),  D = sum (1152 + q) x.
// A second one-workgroup launch reduces the per-workgroup argmax candidates.
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kHeadThreads = 256;
constexpr int kHeadTilesPerWave = 4;
constexpr int kHeadRange = 16 * 4 * kHeadTilesPerWave;    // vocab rows per workgroup

int head_workgroups(int vocab) { return (vocab + kHeadRange - 1) / kHeadRange; }

static size_t head_lds_bytes(int H, int rows) {
  return (size_t)rows * (H + 8) * 2 + (size_t)(H / 32) * 16 * 4;
}

template <bool F32IN>
__global__ __launch_bounds__(kHeadThreads) void k_head(HeadArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ float s_scale[kMaxRows], s_unscale[kMaxRows];
  __shared__ float s_bv[4][kMaxRows];
  __shared__ int s_bi[4][kMaxRows];
  const int H = a.hidden, R = a.rows, V = a.vocab;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool f32in = a.x_dtype == 0;
  const int nrows = f32in ? 16 : 8;
  const int stride = H + 8;
  _Float16* xs = (_Float16*)smem;
  float* sx = (float*)(smem + (size_t)nrows * stride * 2);

  // per-row power-of-two scale: largest magnitude into [2^14, 2^15)
  for (int r = wave; r < R; r += 4) {
    float m = 0.f;
    for (int h = lane; h < H; h += kWave) m = fmaxf(m, fabsf(load_x<F32IN>(a.x, (long)r * H + h)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) {
      int ex = 0;
      if (m > 0.f) frexpf(m, &ex);        // m = f * 2^ex, f in [0.5, 1)
      const int sh = m > 0.f ? 15 - ex : 0;
      s_scale[r] = ldexpf(1.f, sh);
      s_unscale[r] = ldexpf(1.f, -sh);
    }
  }
  for (int i = tid; i < (H / 32) * 16; i += kHeadThreads) sx[i] = 0.f;
  __syncthreads();

  // stage binary16 operand (inputs permuted within groups of 8) and block sums
  const int ngrp = H / 8, total = R * ngrp;
  for (int base = 0; base < total; base += kHeadThreads) {
    const int i = base + tid;
    const bool ok = i < total;
    const int j = ok ? i / ngrp : 0, u = ok ? i % ngrp : 0;
    _Float16 hi[8], lo[8];
    float shi = 0.f, slo = 0.f;
#pragma unroll
    for (int e = 0; e < 8; e++) {
      const float v = ok ? load_x<F32IN>(a.x, (long)j * H + 8 * u + e) * s_scale[j] : 0.f;
      hi[e] = (_Float16)v;
      lo[e] = f32in ? (_Float16)(v - (float)hi[e]) : (_Float16)0.f;
      shi += (float)hi[e];
      slo += (float)lo[e];
    }
    shi += __shfl_xor(shi, 1);
    shi += __shfl_xor(shi, 2);
    slo += __shfl_xor(slo, 1);
    slo += __shfl_xor(slo, 2);
    if (ok) {
      f16x8 ph, pl;
#pragma unroll
      for (int e = 0; e < 8; e++) { ph[e] = hi[perm_q8(e)]; pl[e] = lo[perm_q8(e)]; }
      *(f16x8*)(xs + (size_t)j * stride + 8 * u) = ph;
      if (f32in) *(f16x8*)(xs + (size_t)(8 + j) * stride + 8 * u) = pl;
      if ((u & 3) == 0) {
        sx[(u >> 2) * 16 + j] = shi;
        sx[(u >> 2) * 16 + 8 + j] = slo;
      }
    }
  }
  __syncthreads();

  const int c = lane & 15, q = lane >> 4;
  const bool col_ok = (c & 7) < R && (c < 8 || f32in);
  const int NG = H / 64;    // k-groups of 64 inputs = 2 blocks
  float best_v[4];
  int best_i[4];
#pragma unroll
  for (int i = 0; i < 4; i++) { best_v[i] = -INFINITY; best_i[i] = 0x7FFFFFFF; }

  for (int u = 0; u < kHeadTilesPerWave; u++) {
    const int tile = (blockIdx.x * 4 + wave) * kHeadTilesPerWave + u;
    if (tile * 16 >= V) break;
    const u32x4* cp = (const u32x4*)a.codes + (long)tile * NG * 64 + lane;
    const uint32_t* mp = (const uint32_t*)a.meta + ((long)tile * NG * 16 + c);  // 2 x u16 per row
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int g = 0; g < NG; g++) {
      const u32x4 cw = cp[(long)g * 64];
      const uint32_t mw = mp[(long)g * 16];
#pragma unroll
      for (int beta = 0; beta < 2; beta++) {
        const int blk = 2 * g + beta;
        f16x8 ax = {};
        if (col_ok) ax = *(const f16x8*)(xs + (size_t)c * stride + blk * 32 + q * 8);
        const f16x8 bq = q8_to_f16x8(cw[2 * beta], cw[2 * beta + 1]);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 d = mfma_f16(ax, bq, z);
        const float s = beta ? f16_hi(mw) : f16_lo(mw);
        const float* sxb = sx + blk * 16 + 4 * q;
#pragma unroll
        for (int i = 0; i < 4; i++) acc[i] = fmaf(s, fmaf(-1152.f, sxb[i], d[i]), acc[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] += __shfl_down(acc[i], 32);
    if (lane < 32) {
      const int v = tile * 16 + c;
#pragma unroll
      for (int i = 0; i < 4; i++) {
        const int r = 4 * q + i;
        if (r < R) {
          const float val = acc[i] * s_unscale[r];
          if (a.logits) a.logits[(long)r * V + v] = val;
          if (val > best_v[i] || (val == best_v[i] && v < best_i[i])) { best_v[i] = val; best_i[i] = v; }
        }
      }
    }
  }
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
    for (int w = 1; w < 4; w++)
      if (s_bv[w][tid] > bv || (s_bv[w][tid] == bv && s_bi[w][tid] < bi)) { bv = s_bv[w][tid]; bi = s_bi[w][tid]; }
    a.part_val[(long)blockIdx.x * R + tid] = bv;
    a.part_idx[(long)blockIdx.x * R + tid] = bi;
  }

}

// Per-row argmax over the workgroups' candidates (one workgroup, after k_head).
__global__ __launch_bounds__(kHeadThreads) void k_head_argmax(HeadArgs a, int nwg) {
  const int R = a.rows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int r = wave; r < R; r += 4) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
    for (int w = lane; w < nwg; w += kWave) {
      const float v = a.part_val[(long)w * R + r];
      const int id = a.part_idx[(long)w * R + r];
      if (v > bv || (v == bv && id < bi)) { bv = v; bi = id; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (lane == 0) a.argmax[r] = bi;
  }
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

int launch_head(const HeadArgs& a, hipStream_t s, const Prof* p) {
  const size_t lds = head_lds_bytes(a.hidden, a.x_dtype == 0 ? 16 : 8);
  static size_t granted = 64 * 1024;   // raise the dynamic LDS limit once, when needed
  if (lds > granted) {
    if (int e = (int)hipFuncSetAttribute((const void*)k_head<true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
      return e;
    if (int e = (int)hipFuncSetAttribute((const void*)k_head<false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds))
      return e;
    granted = lds;
  }
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  const int nwg = head_workgroups(a.vocab);
  if (a.x_dtype == 0)
    launch(k_head<true>, dim3(nwg), dim3(kHeadThreads), lds, s, p ? &p0 : nullptr, a);
  else
    launch(k_head<false>, dim3(nwg), dim3(kHeadThreads), lds, s, p ? &p0 : nullptr, a);
  launch(k_head_argmax, dim3(1), dim3(kHeadThreads), 0, s, p ? &p1 : nullptr, a, nwg);
  return (int)hipGetLastError();
}

}  // namespace sw
