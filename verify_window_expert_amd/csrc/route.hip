// Router of a verify window: GEMV in double from exact products, softmax, top-k with
// the lower expert index winning ties, and the per-expert row lists of the window.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// the router and every routed expert the window's rows use are read once for all of
// them; the row lists built here are what lets the expert kernels do that.
//
// Two launches. k_route_logits: workgroup (expert group eg, input chunk hc), each of its
// 4 waves owns one expert and 512 inputs and writes one double partial per row.
// k_route_final (one workgroup) adds the partials in chunk order, then runs softmax,
// top-k and grouping for the whole window. (A completion ticket in one launch would
// serialise one device-scope atomic per workgroup, which costs more than the launch.)
// Reductions inside a wave use DPP and the permlane swaps (common.h), not LDS.
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kRouteChunk = 512;          // inputs per workgroup
constexpr int kRouteWaves = 4;            // experts per workgroup
constexpr int kMaxExpertsRoute = 256;     // the ABI's limit on experts

template <bool F32IN>
__global__ __launch_bounds__(256) void k_route_logits(RouteArgs a) {
  __shared__ __align__(16) double xs[kMaxRows][kRouteChunk];

  const int H = a.hidden, E = a.n_experts, R = a.rows;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int hc = blockIdx.x % n_hc, eg = blockIdx.x / n_hc;
  const int h0 = hc * kRouteChunk;
  const int hn = min(kRouteChunk, H - h0);   // a multiple of 32 (hidden % 32 == 0)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = eg * kRouteWaves + wave;

  // Every load below is unconditional with its index clamped into range, so a thread's
  // loads issue back to back; values outside the range are zeroed afterwards.
  // gate weights of this wave's expert: inputs 2*lane + 128u, 2*lane + 128u + 1
  constexpr int NU = kRouteChunk / 128;
  float2 gv[NU];
  const float* grow = a.gate_w + (long)min(e, E - 1) * H + h0;
#pragma unroll
  for (int u = 0; u < NU; u++) gv[u] = *(const float2*)(grow + min(128 * u + 2 * lane, hn - 2));
  // the chunk of the window's rows, as doubles (exact): thread t converts row t / 32,
  // inputs 16 (t % 32) .. +15; rows past R and inputs past hn become 0
  {
    const int xr = tid >> 5, xc = 16 * (tid & 31);
    const bool ok = xr < R && xc < hn;
    const long base = (long)min(xr, R - 1) * H + h0 + min(xc, hn - 16);
    float v[16];
    if constexpr (F32IN) {
      const u32x4* p = (const u32x4*)((const float*)a.x + base);
      u32x4 w[4];
#pragma unroll
      for (int i = 0; i < 4; i++) w[i] = p[i];
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const uint32_t b = w[i >> 2][i & 3];
        v[i] = __uint_as_float(b);
      }
    } else {
      const u32x4* p = (const u32x4*)((const uint16_t*)a.x + base);
      u32x4 w[2];
#pragma unroll
      for (int i = 0; i < 2; i++) w[i] = p[i];
#pragma unroll
      for (int i = 0; i < 16; i++) v[i] = bf16_to_f32((uint16_t)(w[i >> 3][(i >> 1) & 3] >> (16 * (i & 1))));
    }
#pragma unroll
    for (int i = 0; i < 16; i += 2)
      *(double2*)&xs[xr][xc + i] = double2{ok ? (double)v[i] : 0.0, ok ? (double)v[i + 1] : 0.0};
  }
#pragma unroll
  for (int u = 0; u < NU; u++)
    if (128 * u + 2 * lane >= hn) gv[u] = float2{0.f, 0.f};
  __syncthreads();

  // all eight rows (rows past R read zeros), then eight independent wave sums
  double acc[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; r++) acc[r] = 0.0;
#pragma unroll
  for (int u = 0; u < NU; u++) {
    const int h = 128 * u + 2 * lane;
#pragma unroll
    for (int r = 0; r < kMaxRows; r++) {
      const double2 xv = *(const double2*)&xs[r][h];
      acc[r] = fma((double)gv[u].x, xv.x, acc[r]);
      acc[r] = fma((double)gv[u].y, xv.y, acc[r]);
    }
  }
  double sum[kMaxRows];
#pragma unroll
  for (int r = 0; r < kMaxRows; r++) sum[r] = wave_sum(acc[r]);
  if (lane < kMaxRows && lane < R && e < E) {
    double s = sum[0];
#pragma unroll
    for (int r = 1; r < kMaxRows; r++) s = lane == r ? sum[r] : s;
    a.partials[((long)hc * R + lane) * E + e] = s;
  }
}

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

constexpr int kFinalThreads = 512;   // one wave per window row

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

// One workgroup: wave r adds row r's partials in chunk order, then top-k and softmax for
// the row (every reduction inside the wave, without LDS); the row's selections go to LDS
// as a row mask per expert and a weight per (row, expert); waves 0..3 then list the used
// experts in ascending order with their rows (ballots give every position directly).
//
// Lane l holds experts MU*l .. MU*l + MU - 1. Top-k takes K rounds; in each, the lanes'
// best remaining keys are compared on their upper 32 bits (one DPP max), and only when
// several lanes share the largest upper half are those lanes' whole keys compared. The
// winner's lane pops it. The softmax shift is the first winner's logit; the denominator
// (double sum of float exponentials) does not depend on the later rounds.
template <int MU>
__global__ __launch_bounds__(kFinalThreads) void k_route_final(RouteArgs a) {
  __shared__ uint32_t s_mask[kMaxExpertsRoute + 1];
  __shared__ float s_wt[kMaxRows][kMaxExpertsRoute];
  __shared__ int s_tot[2][4];
  __shared__ int s_rowcnt[4][kMaxRows];
  const int H = a.hidden, E = a.n_experts, R = a.rows, K = a.top_k;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;

  // every chunk's partial loaded at once (only the rows and chunks that exist: one
  // workgroup issues every load), added in chunk order below, then the bias
  constexpr int MC = 8;
  const int r = min(wave, R - 1);
  double part[MU][MC] = {};
  float bias[MU] = {};
  if (wave < R) {
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = min(MU * lane + u, E - 1);
#pragma unroll
      for (int c = 0; c < MC; c++)
        if (c < n_hc) part[u][c] = a.partials[((long)c * R + r) * E + ee];
      if (a.bias) bias[u] = a.bias[ee];
    }
  }
  // (while those are in flight) clear the row masks
  for (int i = tid; i <= E; i += kFinalThreads) s_mask[i] = 0u;
  __syncthreads();

  if (wave < R) {
    double l[MU];
    uint64_t hk[MU];
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = MU * lane + u;
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < MC; c++)
        if (c < n_hc) sum += part[u][c];
      for (int c = MC; c < n_hc; c++) sum += a.partials[((long)c * R + r) * E + min(ee, E - 1)];   // hidden > 4096
      const bool ok = ee < E;
      l[u] = ok ? sum + (a.bias ? (double)bias[u] : 0.0) : -INFINITY;
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
      a.topk_idx[r * K + lane] = my_e;
      a.topk_w[r * K + lane] = (float)my_w;
      s_wt[r][my_e] = (float)my_w;
      atomicOr(&s_mask[my_e], 1u << r);
    }
  }
  __syncthreads();

  // grouping: expert e = tid (waves 0..3); mask bit r = row r uses e
  const int e = tid;
  const uint32_t m = e < E ? s_mask[e] : 0u;
  if (e <= E) a.row_mask[e] = (uint8_t)(e == E ? (1u << R) - 1u : m);
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
    s_tot[0][wave] = __popcll(bu);
    s_tot[1][wave] = wave_cnt;
#pragma unroll
    for (int rr = 0; rr < kMaxRows; rr++) s_rowcnt[wave][rr] = __popcll(brow[rr]);
  }
  __syncthreads();
  if (wave >= 4) return;
  int pf = 0, pc = 0, tot_f = 0, tot_c = 0;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    if (w < wave) { pf += s_tot[0][w]; pc += s_tot[1][w]; }
    tot_f += s_tot[0][w];
    tot_c += s_tot[1][w];
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
      if (w < wave) p += s_rowcnt[w][rr];
    place[rr] = p;
  }
  if (used) {
    const int pos = pf + rank, off = pc + before;
    a.active[pos] = e;
    a.offsets[pos] = off;
    // the expert's rows ascending, each with its weight and its place in the row's list
    int n = 0;
#pragma unroll
    for (int rr = 0; rr < kMaxRows; rr++) {
      if ((m >> rr) & 1u) {
        const float wt = s_wt[rr][e];
        a.entry_row[off + n] = rr;
        a.entry_w[off + n] = wt;
        a.entry_pos[off + n] = place[rr];
        a.row_w[rr * K1 + place[rr]] = wt;
        n++;
      }
    }
  }
  if (tid == 0) {
    a.active[tot_f] = E;            // shared expert last
    a.offsets[tot_f] = tot_c;
    a.offsets[tot_f + 1] = tot_c + R;
    *a.n_active = tot_f + 1;
  }
  if (tid < R) {
    a.entry_row[tot_c + tid] = tid;
    a.entry_w[tot_c + tid] = 1.0f;
    a.entry_pos[tot_c + tid] = K;
    a.row_w[tid * K1 + K] = 1.0f;
  }
}

// ---------------------------------------------------------- routing counts and tier
// Strata docs/BATCHING.md, the paragraph on batch windows counting the experts they route
// to: every --adapt-every windows the most-routed experts outside the fast tier are
// swapped in for the least-routed resident ones, each swap clearing --adapt-min-gain (the
// incoming count against the outgoing one). One workgroup, thread e = expert e:
//   counts[e] = fmaf(counts[e], decay, rows of the window routed to e)   (float)
// and, on a selection round, each expert's rank in its list (outside the tier: count
// descending; resident: ascending; ties to the lower index), then pair i = (i-th
// outside, i-th resident) swaps while every pair up to it clears the bar.
constexpr int kTierThreads = kMaxExpertsRoute;

__global__ __launch_bounds__(kTierThreads) void k_tier(TierArgs a) {
  // each expert's place as one unsigned 64-bit key: its list (outside the tier 0,
  // resident 1; 2 = no expert), then the count's bits (counts are >= 0, so their bits
  // order like the values; inverted for the outside list, largest first), then the
  // expert index (ties: the lower index first). Its rank in its list is the number of
  // smaller keys less the entries of the lists before it.
  __shared__ __align__(16) uint64_t s_key[kTierThreads];
  __shared__ int s_in[kTierThreads], s_out[kTierThreads];
  __shared__ float s_c[kTierThreads];
  __shared__ int s_n[2], s_fail;
  const int E = a.n_experts, e = threadIdx.x;
  float c = 0.f;
  uint32_t res = 2;
  if (e < E) {
    const uint32_t m = a.row_mask[e];
    const float c0 = a.counts[e];
    if (a.resident) res = a.resident[e] ? 1u : 0u;   // loaded with the counts
    c = fmaf(c0, a.decay, (float)__builtin_popcount(m));
    a.counts[e] = c;
  }
  if (!a.resident) return;
  const uint32_t cb = __float_as_uint(c);
  const uint64_t key = ((uint64_t)res << 40) | ((uint64_t)(res == 0 ? ~cb : cb) << 8) | (uint64_t)e;
  s_key[e] = key;
  s_c[e] = c;
  const uint64_t b0 = __ballot(res == 0), b1 = __ballot(res == 1);
  if (e < 2) s_n[e] = 0;
  if (e == 0) s_fail = kTierThreads;
  __syncthreads();
  if ((e & 63) == 0) {
    atomicAdd(&s_n[0], (int)__popcll(b0));
    atomicAdd(&s_n[1], (int)__popcll(b1));
  }
  int below = 0;
#pragma unroll 8
  for (int j = 0; j < kTierThreads; j += 2) {
    const uint64_t k0 = s_key[j], k1 = s_key[j + 1];
    below += (k0 < key) + (k1 < key);
  }
  __syncthreads();
  if (res != 2) {
    const int rank = below - (res == 1 ? s_n[0] : 0);
    if (res) s_out[rank] = e; else s_in[rank] = e;
  }
  __syncthreads();
  const int limit = min(a.max_swaps, min(s_n[0], s_n[1]));
  if (e < limit) {
    const float ci = s_c[s_in[e]], co = s_c[s_out[e]];
    const float bar = a.min_gain * co;
    if (!(ci > 0.f && ci >= bar)) atomicMin(&s_fail, e);
  }
  __syncthreads();
  const int n = min(limit, s_fail);
  if (e < n) {
    const int ein = s_in[e], eout = s_out[e];
    a.swaps[2 * e] = ein;
    a.swaps[2 * e + 1] = eout;
    a.resident[ein] = 1;
    a.resident[eout] = 0;
  }
  if (e == 0) *a.n_swaps = n;
}

int launch_tier(const TierArgs& a, hipStream_t s, const Prof* p) {
  launch(k_tier, dim3(1), dim3(kTierThreads), 0, s, p, a);
  return (int)hipGetLastError();
}

int launch_route(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  const int n_hc = (a.hidden + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (a.n_experts + kRouteWaves - 1) / kRouteWaves;
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  if (a.x_dtype == 0)
    launch(k_route_logits<true>, dim3(n_hc * n_eg), dim3(256), 0, stream, p ? &p0 : nullptr, a);
  else
    launch(k_route_logits<false>, dim3(n_hc * n_eg), dim3(256), 0, stream, p ? &p0 : nullptr, a);
  if (a.n_experts <= 2 * kWave)
    launch(k_route_final<2>, dim3(1), dim3(kFinalThreads), 0, stream, p ? &p1 : nullptr, a);
  else
    launch(k_route_final<4>, dim3(1), dim3(kFinalThreads), 0, stream, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
