// Router of a verify window: GEMV in double from exact products, softmax, top-k with
// the lower expert index winning ties, and the per-expert row lists of the window.
//
// Strata docs/BATCHING.md, "Several requests at once (batch slots)", opening paragraph:
// the router and each routed expert the window's rows use are fetched a single time for all of
// them; the row lists built here are what lets the expert kernels do that.
//
// Two launches. k_route_logits: workgroup (row group, expert group, input chunk), each of
// its 4 waves owns one expert and 512 inputs and writes one double partial per row of
// its row group.
// k_route_final (one workgroup) adds the partials in chunk order, then runs softmax,
// top-k and grouping for the whole window. (A completion ticket in one launch would
// serialise one device-scope atomic per workgroup, which costs more than the launch.)
// Reductions inside a wave use DPP and the permlane swaps (common.h), not LDS.
#include "route_core.h"

namespace sw {

constexpr int kRouteWaves = 4;            // experts per workgroup

constexpr int kRouteThreads = 64 * kRouteWaves;
constexpr int kRouteNU = kRouteChunk / 128;  // float2 gate weights per lane

// The gate weights of wave `wave`'s expert over the chunk [h0, h0 + hn): inputs
// 2 * lane + 128 u and the next one. Every load is unconditional, its index clamped into
// range (so a thread's loads issue back to back); route_gemv zeroes those past hn.
__device__ __forceinline__ void gate_chunk_load(const RouteArgs& a, int e, int h0, int hn, int lane,
                                                float2 (&gv)[kRouteNU]) {
  const float* grow = a.gate_w + (long)min(e, a.n_experts - 1) * a.hidden + h0;
#pragma unroll
  for (int u = 0; u < kRouteNU; u++) gv[u] = *(const float2*)(grow + min(128 * u + 2 * lane, hn - 2));
}

// One chunk of the router's GEMV, once rows r0 .. r0 + NR - 1 of the window are in xs as
// doubles (rows past R and inputs past hn zero): the wave's expert against each row, one
// wave sum per row, and one double partial per (chunk, row, expert). A row's arithmetic
// is the same whichever rows share the workgroup.
template <int NR>
__device__ __forceinline__ void route_gemv(const RouteArgs& a, const double (&xs)[NR][kRouteChunk],
                                           float2 (&gv)[kRouteNU], int hc, int hn, int e, int lane, int r0) {
#pragma unroll
  for (int u = 0; u < kRouteNU; u++)
    if (128 * u + 2 * lane >= hn) gv[u] = float2{0.f, 0.f};
  double acc[NR];
#pragma unroll
  for (int r = 0; r < NR; r++) acc[r] = 0.0;
#pragma unroll
  for (int u = 0; u < kRouteNU; u++) {
    const int h = 128 * u + 2 * lane;
#pragma unroll
    for (int r = 0; r < NR; r++) {
      const double2 xv = *(const double2*)&xs[r][h];
      acc[r] = fma((double)gv[u].x, xv.x, acc[r]);
      acc[r] = fma((double)gv[u].y, xv.y, acc[r]);
    }
  }
  double sum[NR];
#pragma unroll
  for (int r = 0; r < NR; r++) sum[r] = wave_sum(acc[r]);
  const int R = a.rows, E = a.n_experts;
  if (lane < NR && r0 + lane < R && e < E) {
    double s = sum[0];
#pragma unroll
    for (int r = 1; r < NR; r++) s = lane == r ? sum[r] : s;
    a.partials[((long)hc * R + r0 + lane) * E + e] = s;
  }
}

// N 32-bit words from p (16-byte aligned when N % 4 == 0, else 8-byte aligned), loaded
// as 16- or 8-byte vectors.
template <int N>
__device__ __forceinline__ void load_words(const void* p, uint32_t (&w)[N]) {
  static_assert(N % 2 == 0, "whole 8-byte vectors");
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; q++) {
      const u32x4 v = ((const u32x4*)p)[q];
#pragma unroll
      for (int i = 0; i < 4; i++) w[4 * q + i] = v[i];
    }
  } else {
#pragma unroll
    for (int q = 0; q < N / 2; q++) {
      const uint2 v = ((const uint2*)p)[q];
      w[2 * q] = v.x;
      w[2 * q + 1] = v.y;
    }
  }
}
template <int N>
__device__ __forceinline__ void store_words(void* p, const uint32_t (&w)[N]) {
  static_assert(N % 2 == 0, "whole 8-byte vectors");
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int q = 0; q < N / 4; q++) ((u32x4*)p)[q] = u32x4{w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]};
  } else {
#pragma unroll
    for (int q = 0; q < N / 2; q++) ((uint2*)p)[q] = uint2{w[2 * q], w[2 * q + 1]};
  }
}

// Workgroup (row group, group of 4 experts, 512-input chunk): rows r0 .. r0 + RS - 1 of
// the window as doubles in LDS, then every wave's expert against them. Fewer rows per
// workgroup: less work before each workgroup's partials, more reads of the router's
// weights (from L2 after the first).
template <bool F32IN, int RS>
__global__ __launch_bounds__(kRouteThreads) void k_route_logits(RouteArgs a) {
  constexpr int V = RS * kRouteChunk / kRouteThreads;   // inputs of the piece per thread
  constexpr int SEG = kRouteChunk / V;                   // threads per row
  static_assert(V >= 4 && V % 4 == 0, "whole 8- or 16-byte vectors of x");
  __shared__ __align__(16) double xs[RS][kRouteChunk];

  const int H = a.hidden, R = a.rows, E = a.n_experts;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (E + kRouteWaves - 1) / kRouteWaves;
  const int hc = blockIdx.x % n_hc, eg = (blockIdx.x / n_hc) % n_eg, rg = blockIdx.x / (n_hc * n_eg);
  const int h0 = hc * kRouteChunk, r0 = rg * RS;
  const int hn = min(kRouteChunk, H - h0);   // a multiple of 32 (hidden % 32 == 0), so of V
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = eg * kRouteWaves + wave;

  float2 gv[kRouteNU];
  gate_chunk_load(a, e, h0, hn, lane, gv);
  // the piece of the window's rows, as doubles (exact): thread t converts row r0 + t / SEG,
  // inputs V (t % SEG) .. + V - 1; rows past R and inputs past hn become 0
  {
    const int xr = tid / SEG, xc = V * (tid % SEG);
    const bool ok = r0 + xr < R && xc < hn;
    const long base = (long)min(r0 + xr, R - 1) * H + h0 + min(xc, hn - V);
    float v[V];
    if constexpr (F32IN) {
      uint32_t w[V];
      load_words<V>((const float*)a.x + base, w);
#pragma unroll
      for (int i = 0; i < V; i++) v[i] = __uint_as_float(w[i]);
    } else {
      uint32_t w[V / 2];
      load_words<V / 2>((const uint16_t*)a.x + base, w);
#pragma unroll
      for (int i = 0; i < V; i++) v[i] = bf16_to_f32((uint16_t)(w[i >> 1] >> (16 * (i & 1))));
    }
#pragma unroll
    for (int i = 0; i < V; i += 2)
      *(double2*)&xs[xr][xc + i] = double2{ok ? (double)v[i] : 0.0, ok ? (double)v[i + 1] : 0.0};
  }
  __syncthreads();
  route_gemv<RS>(a, xs, gv, hc, hn, e, lane, r0);
}

// A stack's hand-over between two layers in one launch: layer l's combine over one
// 512-input chunk of RS rows, which is layer l + 1's input there (x_next = bf16(residual +
// the weighted expert outputs), combine_one), and layer l + 1's router GEMV over the same
// chunk and rows. Workgroup (row group, expert group, chunk), one wave per expert as in
// the router's own kernel: every workgroup forms its piece of x_next from y (the same
// arithmetic in each, so they agree), and the first expert group of each (row group,
// chunk) also writes it (and the float output, when asked). The partials are those the
// router's own kernel computes from the stored x_next, bit for bit. Fewer rows per
// workgroup: less of y through each compute unit, more reads of the router's weights.
template <bool F32RES, int RS>
__global__ __launch_bounds__(kRouteThreads) void k_combine_route(CombineRouteArgs c) {
  constexpr int V = RS * kRouteChunk / kRouteThreads;   // values of the piece per thread
  constexpr int SEG = kRouteChunk / V;                   // threads per row
  static_assert(V >= 4 && V % 4 == 0, "whole 16-byte vectors of y");
  __shared__ __align__(16) double xs[RS][kRouteChunk];
  const RouteArgs& a = c.route;

  const int H = a.hidden, R = a.rows, E = a.n_experts, K1 = c.top_k + 1;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (E + kRouteWaves - 1) / kRouteWaves;
  const int hc = blockIdx.x % n_hc, eg = (blockIdx.x / n_hc) % n_eg, rg = blockIdx.x / (n_hc * n_eg);
  const int h0 = hc * kRouteChunk, r0 = rg * RS;
  const int hn = min(kRouteChunk, H - h0);   // a multiple of 32, so of V
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = eg * kRouteWaves + wave;

  float2 gv[kRouteNU];
  gate_chunk_load(a, e, h0, hn, lane, gv);
  {
    // thread t: row r0 + t / SEG, inputs V (t % SEG) .. + V - 1 of the chunk; every load
    // clamped into range and issued at once (the row's k + 1 expert outputs, their
    // weights, the residual)
    const int xr = tid / SEG, xc = V * (tid % SEG);
    const bool ok = r0 + xr < R && xc < hn;
    const int r = min(r0 + xr, R - 1);
    const long col = h0 + min(xc, hn - V);
    float w[kMaxTopk + 1];
    uint32_t yw[kMaxTopk + 1][V];
#pragma unroll
    for (int j = 0; j <= kMaxTopk; j++) {
      const int jj = min(j, K1 - 1);
      w[j] = c.row_w[r * K1 + jj];
      load_words<V>(c.y + (long)(r * K1 + jj) * H + col, yw[j]);
    }
    float res[V];
    if (c.x_res) {
      if constexpr (F32RES) {
        uint32_t rw[V];
        load_words<V>((const float*)c.x_res + (long)r * H + col, rw);
#pragma unroll
        for (int i = 0; i < V; i++) res[i] = __uint_as_float(rw[i]);
      } else {
        uint32_t rw[V / 2];
        load_words<V / 2>((const uint16_t*)c.x_res + (long)r * H + col, rw);
#pragma unroll
        for (int i = 0; i < V; i++) res[i] = bf16_to_f32((uint16_t)(rw[i >> 1] >> (16 * (i & 1))));
      }
    } else {
#pragma unroll
      for (int i = 0; i < V; i++) res[i] = 0.f;
    }
    uint32_t ow[V];
    uint16_t xb[V];
#pragma unroll
    for (int i = 0; i < V; i++) {
      float yi[kMaxTopk + 1];
#pragma unroll
      for (int j = 0; j <= kMaxTopk; j++) yi[j] = __uint_as_float(yw[j][i]);
      const float o = combine_one(w, yi, K1, c.x_res != nullptr, res[i]);
      ow[i] = __float_as_uint(o);
      xb[i] = f32_to_bf16(o);
    }
    if (eg == 0 && ok) {
      uint32_t pk[V / 2];
#pragma unroll
      for (int i = 0; i < V / 2; i++) pk[i] = (uint32_t)xb[2 * i] | ((uint32_t)xb[2 * i + 1] << 16);
      store_words<V / 2>(c.x_next + (long)(r0 + xr) * H + col, pk);
      if (c.out) store_words<V>(c.out + (long)(r0 + xr) * H + col, ow);
    }
#pragma unroll
    for (int i = 0; i < V; i += 2)
      *(double2*)&xs[xr][xc + i] = double2{ok ? (double)bf16_to_f32(xb[i]) : 0.0,
                                           ok ? (double)bf16_to_f32(xb[i + 1]) : 0.0};
  }
  __syncthreads();
  route_gemv<RS>(a, xs, gv, hc, hn, e, lane, r0);
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
// to (--adapt-every, --adapt-decay, --adapt-min-gain): each window's routing adds to a
// per-expert count; on a selection round, experts outside the fast tier with high counts
// replace resident experts with low counts, a pair at a time, while the incoming count
// clears min_gain times the outgoing one. One workgroup, thread e = expert e:
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

#ifndef SW_CR_ROWS
#define SW_CR_ROWS 2
#endif
constexpr int kCrRows = SW_CR_ROWS;       // window rows per workgroup of the stack's hand-over

int launch_combine_route(const CombineRouteArgs& c, int res_f32, hipStream_t stream, const Prof* p) {
  const RouteArgs& a = c.route;
  const int n_hc = (a.hidden + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (a.n_experts + kRouteWaves - 1) / kRouteWaves;
  const int n_rg = (a.rows + kCrRows - 1) / kCrRows;
  const dim3 grid(n_hc * n_eg * n_rg);
  if (res_f32)
    launch(k_combine_route<true, kCrRows>, grid, dim3(kRouteThreads), 0, stream, p, c);
  else
    launch(k_combine_route<false, kCrRows>, grid, dim3(kRouteThreads), 0, stream, p, c);
  return (int)hipGetLastError();
}

#ifndef SW_RL_ROWS
#define SW_RL_ROWS 2
#endif
constexpr int kRlRows = SW_RL_ROWS;       // window rows per workgroup of the router's GEMV

static void launch_logits(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  const int n_hc = (a.hidden + kRouteChunk - 1) / kRouteChunk;
  const int n_eg = (a.n_experts + kRouteWaves - 1) / kRouteWaves;
  const int n_rg = (a.rows + kRlRows - 1) / kRlRows;
  const dim3 grid(n_hc * n_eg * n_rg);
  if (a.x_dtype == 0)
    launch(k_route_logits<true, kRlRows>, grid, dim3(kRouteThreads), 0, stream, p, a);
  else
    launch(k_route_logits<false, kRlRows>, grid, dim3(kRouteThreads), 0, stream, p, a);
}

int launch_route_logits(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  launch_logits(a, stream, p);
  return (int)hipGetLastError();
}

int launch_route_final(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  if (a.n_experts <= 2 * kWave)
    launch(k_route_final<2>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p, a);
  else
    launch(k_route_final<4>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p, a);
  return (int)hipGetLastError();
}

int launch_route(const RouteArgs& a, hipStream_t stream, const Prof* p) {
  Prof p0, p1;
  if (p) { p0.start = p->start; p1.stop = p->stop; }
  launch_logits(a, stream, p ? &p0 : nullptr);
  if (a.n_experts <= 2 * kWave)
    launch(k_route_final<2>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p ? &p1 : nullptr, a);
  else
    launch(k_route_final<4>, dim3(1), dim3(kRouteCoreThreads), 0, stream, p ? &p1 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
