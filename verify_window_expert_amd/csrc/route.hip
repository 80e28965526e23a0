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
  __shared__ double xs[kMaxRows][kRouteChunk];

  const int H = a.hidden, E = a.n_experts, R = a.rows, K = a.top_k;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int hc = blockIdx.x % n_hc, eg = blockIdx.x / n_hc;
  const int h0 = hc * kRouteChunk;
  const int hn = min(kRouteChunk, H - h0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = eg * kRouteWaves + wave;

  // Every load below is unconditional with its index clamped into range, so a thread's
  // loads issue back to back; values outside the range are masked afterwards.
  // gate weights of this wave's expert: 8 loads in flight per lane
  float gv[kRouteChunk / kWave];
  const long erow = (long)min(e, E - 1) * H;
#pragma unroll
  for (int u = 0; u < kRouteChunk / kWave; u++) {
    const int h = u * kWave + lane;
    gv[u] = a.gate_w[erow + h0 + min(h, hn - 1)];
  }
  // the rows' inputs of this chunk as doubles (exact): thread handles inputs 2t, 2t+1 of
  // every row
  {
    float xv[kMaxRows][2];
#pragma unroll
    for (int r = 0; r < kMaxRows; r++)
#pragma unroll
      for (int t = 0; t < 2; t++)
        xv[r][t] = load_x<F32IN>(a.x, (long)min(r, R - 1) * H + h0 + min(2 * tid + t, hn - 1));
#pragma unroll
    for (int r = 0; r < kMaxRows; r++)
#pragma unroll
      for (int t = 0; t < 2; t++) xs[r][2 * tid + t] = (2 * tid + t < hn) ? (double)xv[r][t] : 0.0;
  }
#pragma unroll
  for (int u = 0; u < kRouteChunk / kWave; u++)
    if (u * kWave + lane >= hn) gv[u] = 0.f;
  __syncthreads();

  if (e < E) {
    double acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; r++) acc[r] = 0.0;
#pragma unroll
    for (int u = 0; u < kRouteChunk / kWave; u++) {
      const int h = u * kWave + lane;
#pragma unroll
      for (int r = 0; r < kMaxRows; r++)
        if (r < R) acc[r] = fma((double)gv[u], xs[r][h], acc[r]);
    }
#pragma unroll
    for (int r = 0; r < kMaxRows; r++) {
      if (r >= R) break;
      const double s = wave_sum(acc[r]);
      if (lane == 0) a.partials[((long)hc * R + r) * E + e] = s;
    }
  }
}

// Key order of the selection: larger logit first, then the lower expert index.
__device__ __forceinline__ bool better(double l, int e, double lb, int eb) {
  return l > lb || (l == lb && e < eb);
}

// (logit, expert) of the wave's best candidate, in every lane.
__device__ __forceinline__ void wave_argmax(double& l, int& e) {
  Words<3> v{{(uint32_t)__builtin_bit_cast(uint64_t, l), (uint32_t)(__builtin_bit_cast(uint64_t, l) >> 32),
              (uint32_t)e}};
  v = wave_allreduce_words<3>(v, [](const Words<3>& p, const Words<3>& q) {
    const double lp = double_of(Words<2>{{p.w[0], p.w[1]}}), lq = double_of(Words<2>{{q.w[0], q.w[1]}});
    return better(lq, (int)q.w[2], lp, (int)p.w[2]) ? q : p;
  });
  l = double_of(Words<2>{{v.w[0], v.w[1]}});
  e = (int)v.w[2];
}

// popcount of the bits of m held by the lanes below this one
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

constexpr int kFinalThreads = 512;   // one wave per window row

// One workgroup: wave r adds row r's partials in chunk order, then softmax and top-k for
// the row (every reduction inside the wave, without LDS); the row's selections go to LDS
// as a row mask per expert and a weight per (row, expert); waves 0..3 then list the used
// experts in ascending order with their rows (ballots give every position directly).
__global__ __launch_bounds__(kFinalThreads) void k_route_final(RouteArgs a) {
  __shared__ uint32_t s_mask[kMaxExpertsRoute + 1];
  __shared__ float s_wt[kMaxRows][kMaxExpertsRoute];
  __shared__ int s_tot[2][4];
  const int H = a.hidden, E = a.n_experts, R = a.rows, K = a.top_k;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  for (int i = tid; i <= E; i += kFinalThreads) s_mask[i] = 0u;
  __syncthreads();

  if (wave < R) {
    const int r = wave;
    // logits of experts lane + 64u: every chunk's partial loaded at once (clamped,
    // unconditional), added in chunk order, then the bias
    constexpr int MU = kMaxExpertsRoute / kWave, MC = 8;
    double part[MU][MC];
    float bias[MU];
    const float* bp = a.bias ? a.bias : a.gate_w;   // any readable array when unbiased
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = min(u * kWave + lane, E - 1);
#pragma unroll
      for (int c = 0; c < MC; c++) part[u][c] = a.partials[((long)min(c, n_hc - 1) * R + r) * E + ee];
      bias[u] = bp[ee];
    }
    double l[MU];
    int id[MU];
#pragma unroll
    for (int u = 0; u < MU; u++) {
      const int ee = u * kWave + lane;
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < MC; c++)
        if (c < n_hc) sum += part[u][c];
      for (int c = MC; c < n_hc; c++) sum += a.partials[((long)c * R + r) * E + min(ee, E - 1)];   // hidden > 4096
      const bool ok = ee < E;
      id[u] = ok ? ee : 0x7FFFFFFF;
      l[u] = ok ? sum + (a.bias ? (double)bias[u] : 0.0) : -INFINITY;
    }
    // softmax normaliser
    double mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < MU; u++) mx = fmax(mx, l[u]);
    mx = wave_max(mx);
    double z = 0.0;
#pragma unroll
    for (int u = 0; u < MU; u++)
      if (id[u] < E) z += exp(l[u] - mx);
    z = wave_sum(z);
    // the lane's candidates sorted by the selection key (network of 5 compare-exchanges),
    // so each round compares only the lanes' heads
    auto cx = [&](int i, int j) {
      if (better(l[j], id[j], l[i], id[i])) {
        const double tl = l[i]; l[i] = l[j]; l[j] = tl;
        const int ti = id[i]; id[i] = id[j]; id[j] = ti;
      }
    };
    static_assert(MU == 4, "the sorting network orders four candidates");
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
    // K rounds: the best head wins, its lane pops it; lane j keeps the j-th winner
    double my_w = 0.0;
    int my_e = 0;
    for (int j = 0; j < K; j++) {
      double bl = l[0];
      int be = id[0];
      wave_argmax(bl, be);
      if (id[0] == be) {
        l[0] = l[1]; l[1] = l[2]; l[2] = l[3]; l[3] = -INFINITY;
        id[0] = id[1]; id[1] = id[2]; id[2] = id[3]; id[3] = 0x7FFFFFFF;
      }
      if (lane == j) {
        my_e = be;
        my_w = exp(bl - mx) / z;
      }
    }
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
  if (lane == 0 && wave < 4) {
    s_tot[0][wave] = __popcll(bu);
    s_tot[1][wave] = wave_cnt;
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
  if (used) {
    const int pos = pf + rank, off = pc + before;
    a.active[pos] = e;
    a.offsets[pos] = off;
    // the expert's rows ascending, each with its weight
    uint32_t mm = m;
    for (int n = 0; mm; n++) {
      const int r = __builtin_ctz(mm);
      mm &= mm - 1u;
      a.entry_row[off + n] = r;
      a.entry_w[off + n] = s_wt[r][e];
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
  }
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
  launch(k_route_final, dim3(1), dim3(kFinalThreads), 0, stream, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
