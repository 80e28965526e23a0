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
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kRouteChunk = 512;          // inputs per workgroup
constexpr int kRouteWaves = 4;            // experts per workgroup

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

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
      const double s = wave_sum_d(acc[r]);
      if (lane == 0) a.partials[((long)hc * R + r) * E + e] = s;
    }
  }
}

// Key order of the selection: larger logit first, then the lower expert index.
__device__ __forceinline__ bool better(double l, int e, double lb, int eb) {
  return l > lb || (l == lb && e < eb);
}

constexpr int kFinalThreads = 512;   // one wave per window row

__global__ __launch_bounds__(kFinalThreads) void k_route_final(RouteArgs a) {
  __shared__ double lgs[kMaxRows * 256];         // logits [R][E]
  __shared__ __align__(16) int s_idx[kMaxRows * 8];
  __shared__ float s_w[kMaxRows * 8];
  __shared__ uint32_t s_mask[257];
  __shared__ int s_wsum[2][4];
  const int H = a.hidden, E = a.n_experts, R = a.rows, K = a.top_k;
  const int n_hc = (H + kRouteChunk - 1) / kRouteChunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < kMaxRows * 8) s_idx[tid] = -1;    // entries past R*K never match an expert

  // logits: every (row, expert) pair's partials (layout [chunk][row][expert]) are read
  // with unconditional, clamped loads issued together, summed in chunk order, biased
  {
    constexpr int MP = kMaxRows * 256 / kFinalThreads, MC = 8;
    const int RE = R * E;
    double part[MP][MC];
    float bias[MP];
    const float* bp = a.bias ? a.bias : a.gate_w;   // any readable array when unbiased
#pragma unroll
    for (int i = 0; i < MP; i++) {
      const int p = min(i * kFinalThreads + tid, RE - 1);
#pragma unroll
      for (int c = 0; c < MC; c++) part[i][c] = a.partials[(long)min(c, n_hc - 1) * RE + p];
      bias[i] = bp[p % E];
    }
#pragma unroll
    for (int i = 0; i < MP; i++) {
      const int p = i * kFinalThreads + tid;
      if (p >= RE) break;
      double s = 0.0;
#pragma unroll
      for (int c = 0; c < MC; c++)
        if (c < n_hc) s += part[i][c];
      for (int c = MC; c < n_hc; c++) s += a.partials[(long)c * RE + p];   // hidden > 4096
      lgs[p] = s + (a.bias ? (double)bias[i] : 0.0);
    }
  }
  __syncthreads();

  // softmax and top-k of row r = wave; lane holds experts lane + 64u, kept sorted by the
  // selection key so that each round compares only the lanes' heads
  if (wave < R) {
    const int r = wave;
    double l[4];
    int id[4];
    double mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int ee = u * kWave + lane;
      id[u] = ee < E ? ee : 0x7FFFFFFF;
      l[u] = ee < E ? lgs[r * E + ee] : -INFINITY;
      mx = fmax(mx, l[u]);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
    double z = 0.0;
#pragma unroll
    for (int u = 0; u < 4; u++)
      if (id[u] < E) z += exp(l[u] - mx);
    z = wave_sum_d(z);
    // sort the lane's 4 candidates (network of 5 compare-exchanges)
    auto cx = [&](int i, int j) {
      if (better(l[j], id[j], l[i], id[i])) {
        const double tl = l[i]; l[i] = l[j]; l[j] = tl;
        const int ti = id[i]; id[i] = id[j]; id[j] = ti;
      }
    };
    cx(0, 1); cx(2, 3); cx(0, 2); cx(1, 3); cx(1, 2);
    int head = 0;
    for (int j = 0; j < K; j++) {
      double bl = head < 4 ? l[0] : -INFINITY;
      int be = head < 4 ? id[0] : 0x7FFFFFFF;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double ol = __shfl_xor(bl, off);
        const int oe = __shfl_xor(be, off);
        if (better(ol, oe, bl, be)) { bl = ol; be = oe; }
      }
      if (head < 4 && id[0] == be) {   // the winner pops its head
        l[0] = l[1]; l[1] = l[2]; l[2] = l[3]; l[3] = -INFINITY;
        id[0] = id[1]; id[1] = id[2]; id[2] = id[3]; id[3] = 0x7FFFFFFF;
        head++;
      }
      if (lane == j) {
        s_idx[r * K + j] = be;
        s_w[r * K + j] = (float)(exp(bl - mx) / z);   // unnormalised copy, fixed below
        lgs[r * E + be] = exp(bl - mx) / z;           // keep the double weight
      }
    }
    // weights (renormalised over the row's k when asked), in selection order
    if (lane < K) {
      const int be = s_idx[r * K + lane];
      const double w = lgs[r * E + be];
      double ssum = 0.0;
      for (int j = 0; j < K; j++) ssum += lgs[r * E + s_idx[r * K + j]];
      const double wf = a.renorm ? w / ssum : w;
      a.topk_idx[r * K + lane] = be;
      a.topk_w[r * K + lane] = (float)wf;
      s_w[r * K + lane] = (float)wf;
    }
  }
  __syncthreads();

  // grouping: row mask per expert, then compaction in expert order (threads 0..255)
  {
    int tk[kMaxRows * 8];
#pragma unroll
    for (int t = 0; t < kMaxRows * 8; t += 4) {
      const int4 v = *(const int4*)&s_idx[t];
      tk[t] = v.x; tk[t + 1] = v.y; tk[t + 2] = v.z; tk[t + 3] = v.w;
    }
    for (int ee = tid; ee <= E; ee += kFinalThreads) {
      uint32_t m = 0;
      if (ee == E) {
        m = (1u << R) - 1u;
      } else {
#pragma unroll
        for (int t = 0; t < kMaxRows * 8; t++)
          if (tk[t] == ee) m |= 1u << (t / K);
      }
      s_mask[ee] = m;
      a.row_mask[ee] = (uint8_t)m;
    }
  }
  __syncthreads();

  // exclusive scans of (used ? 1 : 0) and popcount over the routed experts (E <= 256:
  // one expert per thread of waves 0..3)
  const int ee = tid;
  const uint32_t m = ee < E ? s_mask[ee] : 0u;
  const int f = m != 0, c = __builtin_popcount(m);
  int fi = f, ci = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int tf = __shfl_up(fi, off), tc = __shfl_up(ci, off);
    if (lane >= off) { fi += tf; ci += tc; }
  }
  if (lane == 63 && wave < 4) { s_wsum[0][wave] = fi; s_wsum[1][wave] = ci; }
  __syncthreads();
  if (wave >= 4) return;
  int pf = 0, pc = 0, tot_f = 0, tot_c = 0;
  for (int w = 0; w < 4; w++) {
    if (w < wave) { pf += s_wsum[0][w]; pc += s_wsum[1][w]; }
    tot_f += s_wsum[0][w]; tot_c += s_wsum[1][w];
  }
  if (f) {
    const int pos = pf + fi - f, off = pc + ci - c;
    a.active[pos] = ee;
    a.offsets[pos] = off;
    // the expert's (row, weight) entries: top-k positions are row-major, so scanning
    // them in order lists the rows ascending
    int n = 0;
#pragma unroll
    for (int t = 0; t < kMaxRows * 8; t += 4) {
      const int4 v = *(const int4*)&s_idx[t];
      const int tv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int u = 0; u < 4; u++)
        if (tv[u] == ee) {
          a.entry_row[off + n] = (t + u) / K;
          a.entry_w[off + n] = s_w[t + u];
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
