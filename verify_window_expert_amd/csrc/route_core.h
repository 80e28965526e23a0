// Routing core of a verify window, shared by the router's final kernel and the fused
// layer's gate/up kernel: per row, the partial logits added in chunk order, top-k and
// softmax; then the grouping of the window (the active experts ascending, the shared
// expert last, their rows, and each entry's place in its row's list).
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// each routed expert is fetched a single time per window, however many rows use it; the
// row lists built here are what lets the expert kernels do that.
#pragma once
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kRouteChunk = 512;          // inputs per router workgroup
constexpr int kMaxExpertsRoute = 256;     // the ABI's limit on experts
constexpr int kRouteCoreThreads = 512;    // 8 waves: one per window row
constexpr int kRouteMaxSlots = kMaxRows * 8 + 1;   // routed experts a window can use + shared

// Selection key: larger logit first, then the lower expert index, as one unsigned 64-bit
// integer. The double's bits map monotonically to an unsigned order (negative values
// flipped whole, positive ones with the sign bit set); the low 8 bits then carry
// 255 - expert. Two logits closer than 2^-44 of their magnitude (far below the ~1e-13
// by which two summation orders of the same double sum differ) therefore order by
// index; equal logits always do.
__device__ __forceinline__ uint64_t select_key(double l, int e) {
  uint64_t u = __builtin_bit_cast(uint64_t, l);
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
  return (u & ~0xFFull) | (uint64_t)(255 - e);
}
__device__ __forceinline__ int key_expert(uint64_t k) { return 255 - (int)(k & 0xFF); }

// The largest key of the wave, in every lane.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  const Words<2> w = wave_allreduce_words<2>(Words<2>{{(uint32_t)k, (uint32_t)(k >> 32)}},
                                              [](const Words<2>& p, const Words<2>& q) {
    const uint64_t a = (uint64_t)p.w[0] | ((uint64_t)p.w[1] << 32), b = (uint64_t)q.w[0] | ((uint64_t)q.w[1] << 32);
    return a > b ? p : q;
  });
  return (uint64_t)w.w[0] | ((uint64_t)w.w[1] << 32);
}

// popcount of the bits of m held by the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// The largest 32-bit value of the wave, in every lane.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_allreduce_words<1>(Words<1>{{v}}, [](const Words<1>& p, const Words<1>& q) {
    return Words<1>{{p.w[0] > q.w[0] ? p.w[0] : q.w[0]}};
  }).w[0];
}

// exp(d) for d <= 0 as a float: 2^t with t = d log2(e) split in double into an integer n
// and a fraction f in [-1/2, 1/2]; 2^f by the hardware's exp2 (f rounded to float moves
// it by at most 2^-25, i.e. 2e-8 relative), then scaled by 2^n.
__device__ __forceinline__ float exp_nonpos(double d) {
  const double t = fmax(d * 1.4426950408889634, -1000.0);
  const double n = rint(t);
  return ldexpf(__builtin_amdgcn_exp2f((float)(t - n)), (int)n);
}

// LDS of the routing core, and the window's tables it leaves there.
struct RouteLds {
  uint32_t mask[kMaxExpertsRoute + 1];       // per expert: bit r = row r uses it
  float wt[kMaxRows][kMaxExpertsRoute];      // per (row, expert): the routing weight
  int tot[2][4];
  int rowcnt[4][kMaxRows];
  int active[kRouteMaxSlots];                // the window's tables (as strata_route_out)
  int off[kRouteMaxSlots + 1];
  uint8_t rmask[kMaxExpertsRoute + 4];
  int n_active;
};

// Candidate u of a lane: expert u * 64 + lane, so that each of a wave's loads of the
// partials reads 64 consecutive experts (512 contiguous bytes).
__device__ __forceinline__ int cand_expert(int u, int lane) { return u * kWave + lane; }

// The partials of row `wave` (waves < rows) and the bias, in registers: lane l holds
// experts cand_expert(0..MU-1, l), chunks 0..7 (a router of more than 8 chunks is read
// later, in route_select).
template <int MU>
struct RouteRegs {
  double part[MU][8];
  float bias[MU];
};

template <int MU>
__device__ __forceinline__ void route_load(const RouteArgs& a, RouteRegs<MU>& g) {
  const int R = a.rows, E = a.n_experts;
  const int n_hc = (a.hidden + kRouteChunk - 1) / kRouteChunk;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = min(wave, R - 1);
#pragma unroll
  for (int u = 0; u < MU; u++) {
#pragma unroll
    for (int c = 0; c < 8; c++) g.part[u][c] = 0.0;
    g.bias[u] = 0.f;
  }
  // only the rows and chunks that exist: one workgroup issues every load
  if (wave < R) {
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = min(cand_expert(u, lane), E - 1);
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (c < n_hc) g.part[u][c] = a.partials[((long)c * R + r) * E + ee];
      if (a.bias) g.bias[u] = a.bias[ee];
    }
  }
}

// Top-k, softmax and grouping from the loaded partials, by the workgroup's first
// kRouteCoreThreads threads (all of them must call it). Leaves the tables in s; with
// `out`, also the weights, and writes the tables, the top-k and the weights to a's
// outputs. Ends with a barrier.
//
// Wave r handles row r: lane l holds experts cand_expert(u, l), u < MU, each as one
// unsigned 64-bit key (select_key: larger logit first, ties to the lower index; keys are
// distinct). The k largest keys are those at or above a threshold found by binary search
// on the keys' upper 32 bits (each step counts the candidates at or above a trial value
// with ballots), and, only when several keys share the boundary's upper half, by a
// second search on the lower 32 bits of those. With `out`, each selected key's place in
// the row's list is the number of selected keys above it; the softmax shift is the
// largest key's logit and the denominator a double sum of float exponentials. The row's
// selections go to LDS as a row mask per expert (and a weight per (row, expert)); waves
// 0..3 then list the used experts in ascending order with their rows (ballots give every
// position directly).
template <int MU>
__device__ __forceinline__ void route_select(const RouteArgs& a, const RouteRegs<MU>& g, RouteLds& s, bool out) {
  const int H = a.hidden, E = a.n_experts, R = a.rows, K = a.top_k;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int r = min(wave, R - 1);
  for (int i = tid; i <= E; i += kRouteCoreThreads) s.mask[i] = 0u;
  __syncthreads();

  if (wave < R) {
    double l[MU];
    uint64_t hk[MU];
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = cand_expert(u, lane);
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (c < n_hc) sum += g.part[u][c];
      for (int c = 8; c < n_hc; c++) sum += a.partials[((long)c * R + r) * E + min(ee, E - 1)];   // hidden > 4096
      const bool ok = ee < E;
      l[u] = ok ? sum + (a.bias ? (double)g.bias[u] : 0.0) : -INFINITY;
      hk[u] = ok ? select_key(l[u], ee) : 0ull;   // 0: below every real key (whose upper half is > 0)
    }
    // the threshold on the upper halves: the largest T with at least K upper halves >= T;
    // a trial value with exactly K at or above it already separates the selection (the
    // same set), and ends the search
    uint32_t hi[MU];
#pragma unroll
    for (int u = 0; u < MU; u++) hi[u] = (uint32_t)(hk[u] >> 32);
    uint32_t T = 0;
    for (int b = 31; b >= 0; b--) {
      const uint32_t cand = T | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int u = 0; u < MU; u++) cnt += __popcll(__ballot(hi[u] >= cand));
      if (cnt >= K) {
        T = cand;
        if (cnt == K) break;
      }
    }
    int above = 0, at = 0;
#pragma unroll
    for (int u = 0; u < MU; u++) {
      above += __popcll(__ballot(hi[u] > T));
      at += __popcll(__ballot(hi[u] == T));
    }
    // several keys share the boundary's upper half: the largest K - above of them by
    // their lower halves (distinct, since the keys are)
    uint32_t T2 = 0;
    if (above + at > K) {
      const int need = K - above;
      for (int b = 31; b >= 0; b--) {
        const uint32_t cand = T2 | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < MU; u++) cnt += __popcll(__ballot(hi[u] == T && (uint32_t)hk[u] >= cand));
        if (cnt >= need) T2 = cand;
      }
    }
    bool sel[MU];
#pragma unroll
    for (int u = 0; u < MU; u++) sel[u] = hi[u] > T || (hi[u] == T && (uint32_t)hk[u] >= T2);

    if (out) {
      // each selected key's place: the selected keys above it (K readlane steps over the
      // selection's ballots)
      int rank[MU] = {};
      uint64_t bal[MU];
#pragma unroll
      for (int u = 0; u < MU; u++) bal[u] = __ballot(sel[u]);
#pragma unroll
      for (int v = 0; v < MU; v++) {
        uint64_t m = bal[v];
        while (m) {
          const int sl = __builtin_ctzll(m);
          m &= m - 1;
          const uint64_t kv = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(hk[v] >> 32), sl) << 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)hk[v], sl);
#pragma unroll
          for (int u = 0; u < MU; u++) rank[u] += kv > hk[u];
        }
      }
      // the softmax shift: the logit of the largest key
      int top_lane = 0, top_u = 0;
#pragma unroll
      for (int u = 0; u < MU; u++) {
        const uint64_t b = __ballot(sel[u] && rank[u] == 0);
        if (b) { top_lane = __builtin_ctzll(b); top_u = u; }
      }
      double lu = l[0];
#pragma unroll
      for (int u = 1; u < MU; u++) lu = u == top_u ? l[u] : lu;
      const uint64_t lb = __builtin_bit_cast(uint64_t, lu);
      const double lmax = __builtin_bit_cast(double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lb >> 32), top_lane) << 32) |
                                                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lb, top_lane));
      float ex[MU];
      double zl = 0.0;
#pragma unroll
      for (int u = 0; u < MU; u++) {
        ex[u] = cand_expert(u, lane) < E ? exp_nonpos(l[u] - lmax) : 0.f;
        zl += (double)ex[u];
      }
      const double z = wave_sum(zl);
      double w[MU];
      double wsel = 0.0;
#pragma unroll
      for (int u = 0; u < MU; u++) {
        w[u] = (double)ex[u] / z;
        if (sel[u]) wsel += w[u];
      }
      // weights (divided by their sum over the row's k when asked)
      if (a.renorm) {
        const double tot = wave_sum(wsel);
#pragma unroll
        for (int u = 0; u < MU; u++) w[u] = w[u] / tot;
      }
#pragma unroll
      for (int u = 0; u < MU; u++) {
        if (sel[u]) {
          const int e = cand_expert(u, lane);
          a.topk_idx[r * K + rank[u]] = e;
          a.topk_w[r * K + rank[u]] = (float)w[u];
          s.wt[r][e] = (float)w[u];
          atomicOr(&s.mask[e], 1u << r);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < MU; u++)
        if (sel[u]) atomicOr(&s.mask[cand_expert(u, lane)], 1u << r);
    }
  }
  __syncthreads();

  // grouping: expert e = tid (waves 0..3); mask bit r = row r uses e
  const int e = tid;
  const uint32_t m = e < E ? s.mask[e] : 0u;
  if (e <= E) {
    const uint8_t rm = (uint8_t)(e == E ? (1u << R) - 1u : m);
    s.rmask[e] = rm;
    if (out) a.row_mask[e] = rm;
  }
  const bool used = m != 0u;
  const int cnt = __builtin_popcount(m);
  // positions within the wave: used experts below, entries of the experts below
  const uint64_t bu = __ballot(used);
  const int rank = lanes_below(bu);
  int before = 0, wave_cnt = 0;   // cnt <= 8: four bit planes
#pragma unroll
  for (int b = 0; b < 4; b++) {
    const uint64_t plane = __ballot((cnt >> b) & 1);
    before += lanes_below(plane) << b;
    wave_cnt += __popcll(plane) << b;
  }
  // per row r: the experts of row r below this one (its position in the row's list;
  // only the workgroup that writes the routing outputs needs it)
  uint64_t brow[kMaxRows] = {};
  if (out) {
#pragma unroll
    for (int rr = 0; rr < kMaxRows; rr++) brow[rr] = __ballot((m >> rr) & 1u);
  }
  if (lane == 0 && wave < 4) {
    s.tot[0][wave] = __popcll(bu);
    s.tot[1][wave] = wave_cnt;
    if (out) {
#pragma unroll
      for (int rr = 0; rr < kMaxRows; rr++) s.rowcnt[wave][rr] = __popcll(brow[rr]);
    }
  }
  __syncthreads();
  if (wave < 4) {
    int pf = 0, pc = 0, tot_f = 0, tot_c = 0;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      if (w < wave) { pf += s.tot[0][w]; pc += s.tot[1][w]; }
      tot_f += s.tot[0][w];
      tot_c += s.tot[1][w];
    }
    const int K1 = K + 1;
    // this expert's place in each row's list: experts of that row in lower waves + below
    // this lane in its wave
    int place[kMaxRows] = {};
    if (out) {
#pragma unroll
      for (int rr = 0; rr < kMaxRows; rr++) {
        int p = lanes_below(brow[rr]);
#pragma unroll
        for (int w = 0; w < 3; w++)
          if (w < wave) p += s.rowcnt[w][rr];
        place[rr] = p;
      }
    }
    if (used) {
      const int pos = pf + rank, off = pc + before;
      s.active[pos] = e;
      s.off[pos] = off;
      if (out) {
        a.active[pos] = e;
        a.offsets[pos] = off;
        // the expert's rows ascending, each with its weight and its place in the row's list
        int n = 0;
#pragma unroll
        for (int rr = 0; rr < kMaxRows; rr++) {
          if ((m >> rr) & 1u) {
            const float wt = s.wt[rr][e];
            a.entry_row[off + n] = rr;
            a.entry_w[off + n] = wt;
            a.entry_pos[off + n] = place[rr];
            a.row_w[rr * K1 + place[rr]] = wt;
            n++;
          }
        }
      }
    }
    if (tid == 0) {
      s.active[tot_f] = E;            // shared expert last
      s.off[tot_f] = tot_c;
      s.off[tot_f + 1] = tot_c + R;
      s.n_active = tot_f + 1;
      if (out) {
        a.active[tot_f] = E;
        a.offsets[tot_f] = tot_c;
        a.offsets[tot_f + 1] = tot_c + R;
        *a.n_active = tot_f + 1;
      }
    }
    if (out && tid < R) {
      a.entry_row[tot_c + tid] = tid;
      a.entry_w[tot_c + tid] = 1.0f;
      a.entry_pos[tot_c + tid] = K;
      a.row_w[tid * K1 + K] = 1.0f;
    }
  }
  __syncthreads();
}

}  // namespace sw
