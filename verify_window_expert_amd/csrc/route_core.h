// Routing core of a verify window, shared by the router's final kernel and the fused
// layer's gate/up kernel: per row, the partial logits added in chunk order, top-k and
// softmax; then the grouping of the window (the active experts ascending, the shared
// expert last, their rows, and each entry's place in its row's list).
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// the routed experts the window's rows use are read once for all of them; the row lists
// built here are what lets the expert kernels do that.
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

// The partials of row `wave` (waves < rows) and the bias, in registers: lane l holds
// experts MU*l .. MU*l + MU - 1, chunks 0..7 (a router of more than 8 chunks is read
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
      const int ee = min(MU * lane + u, E - 1);
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (c < n_hc) g.part[u][c] = a.partials[((long)c * R + r) * E + ee];
      if (a.bias) g.bias[u] = a.bias[ee];
    }
  }
}

// Top-k, softmax and grouping from the loaded partials, by the workgroup's first
// kRouteCoreThreads threads (all of them must call it). Leaves the tables in s; with
// `out`, also writes them (and the top-k) to a's outputs. Ends with a barrier.
//
// Wave r handles row r: lane l holds experts MU*l .. MU*l + MU - 1. Top-k takes K rounds;
// in each, the lanes' best remaining keys are compared on their upper 32 bits (one DPP
// max), and only when several lanes share the largest upper half are those lanes' whole
// keys compared. The winner's lane pops it. The softmax shift is the first winner's
// logit; the denominator (double sum of float exponentials) does not depend on the later
// rounds. The row's selections go to LDS as a row mask per expert and a weight per (row,
// expert); waves 0..3 then list the used experts in ascending order with their rows
// (ballots give every position directly).
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
      const int ee = MU * lane + u;
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < 8; c++)
        if (c < n_hc) sum += g.part[u][c];
      for (int c = 8; c < n_hc; c++) sum += a.partials[((long)c * R + r) * E + min(ee, E - 1)];   // hidden > 4096
      const bool ok = ee < E;
      l[u] = ok ? sum + (a.bias ? (double)g.bias[u] : 0.0) : -INFINITY;
      hk[u] = ok ? select_key(l[u], ee) : 0ull;   // 0: below every real key
    }
    // the lane's keys sorted descending
    auto cx = [&](int i, int j) {
      const uint64_t a0 = hk[i], a1 = hk[j];
      hk[i] = a0 > a1 ? a0 : a1;
      hk[j] = a0 > a1 ? a1 : a0;
    };
    static_assert(MU == 2 || MU == 4, "two or four candidates per lane");
    if constexpr (MU == 2) {
      cx(0, 1);
    } else {
      cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
    }
    uint64_t my_key = 0;
    double lmax = 0.0, z = 0.0;
    float ex[MU];
    for (int j = 0; j < K; j++) {
      const uint32_t hi = (uint32_t)(hk[0] >> 32);
      const uint32_t bh = wave_max_u32(hi);
      uint64_t m = __ballot(hi == bh);
      if (__popcll(m) != 1) {   // equal upper halves: the whole keys of those lanes decide
        const uint64_t best = wave_max_key(hi == bh ? hk[0] : 0ull);
        m = __ballot(hk[0] == best);
      }
      const int wl = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
      const uint64_t best = ((uint64_t)__builtin_amdgcn_readlane((int)(uint32_t)(hk[0] >> 32), wl) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)hk[0], wl);
      if (lane == wl) {
#pragma unroll
        for (int u = 0; u + 1 < MU; u++) hk[u] = hk[u + 1];
        hk[MU - 1] = 0;
      }
      if (lane == j) my_key = best;
      if (j == 0) {
        // the shift: the winner's logit, read from the lane that holds it
        const int e0 = key_expert(best), u0 = e0 % MU;
        double lu = l[0];
#pragma unroll
        for (int u = 1; u < MU; u++) lu = u == u0 ? l[u] : lu;
        const uint64_t b = __builtin_bit_cast(uint64_t, lu);
        lmax = __builtin_bit_cast(double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), e0 / MU) << 32) |
                                              (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, e0 / MU));
        double zl = 0.0;
#pragma unroll
        for (int u = 0; u < MU; u++) {
          ex[u] = MU * lane + u < E ? exp_nonpos(l[u] - lmax) : 0.f;
          zl += (double)ex[u];
        }
        z = wave_sum(zl);
      }
    }
    // the K weights in parallel (lane j: the j-th winner's exponential from its lane)
    const int my_e = key_expert(my_key);
    float e_sel = 0.f;
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const float v = __shfl(ex[u], (my_e / MU) & 63);
      if (my_e % MU == u) e_sel = v;
    }
    double my_w = (double)e_sel / z;
    // weights (divided by their sum over the row's k when asked), in selection order
    if (a.renorm) my_w = my_w / wave_sum(lane < K ? my_w : 0.0);
    if (lane < K) {
      if (out) {
        a.topk_idx[r * K + lane] = my_e;
        a.topk_w[r * K + lane] = (float)my_w;
      }
      s.wt[r][my_e] = (float)my_w;
      atomicOr(&s.mask[my_e], 1u << r);
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
  // per row r: the experts of row r below this one (its position in the row's list)
  uint64_t brow[kMaxRows];
#pragma unroll
  for (int rr = 0; rr < kMaxRows; rr++) brow[rr] = __ballot((m >> rr) & 1u);
  if (lane == 0 && wave < 4) {
    s.tot[0][wave] = __popcll(bu);
    s.tot[1][wave] = wave_cnt;
#pragma unroll
    for (int rr = 0; rr < kMaxRows; rr++) s.rowcnt[wave][rr] = __popcll(brow[rr]);
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
    int place[kMaxRows];
#pragma unroll
    for (int rr = 0; rr < kMaxRows; rr++) {
      int p = lanes_below(brow[rr]);
#pragma unroll
      for (int w = 0; w < 3; w++)
        if (w < wave) p += s.rowcnt[w][rr];
      place[rr] = p;
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
