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
#include "route_core.h"

namespace sw {

constexpr int kRouteWaves = 4;            // experts per workgroup

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

// One workgroup: the routing core (route_core.h) over the router's partials, writing the
// window's routing outputs.
template <int MU>
__global__ __launch_bounds__(kRouteCoreThreads) void k_route_final(RouteArgs a) {
  __shared__ RouteLds s;
  RouteRegs<MU> g;
  route_load<MU>(a, g);
  route_select<MU>(a, g, s, true);
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

int launch_route_logits(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  const int n_hc = (a.hidden + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (a.n_experts + kRouteWaves - 1) / kRouteWaves;
  if (a.x_dtype == 0)
    launch(k_route_logits<true>, dim3(n_hc * n_eg), dim3(256), 0, stream, p, a);
  else
    launch(k_route_logits<false>, dim3(n_hc * n_eg), dim3(256), 0, stream, p, a);
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
    launch(k_route_final<2>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p ? &p1 : nullptr, a);
  else
    launch(k_route_final<4>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
