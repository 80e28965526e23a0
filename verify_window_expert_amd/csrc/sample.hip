// Sampled draw of a verify window's rows: each row's token from its logits with the
// request's temperature, top_k, top_p and min_p, and a Philox4x32-10 draw keyed by the
// request's seed at the row's position.
//
// Strata docs/BATCHING.md, "Exactness": sampled rows are drawn one by one with the
// single-request window's counter-based draw, Philox(seed, position). A row's token
// depends on its own logits and parameters only, so it is the same alone or in any window;
// a slot's proposal is then verified by the greedy rule against these draws (k_accept).
//
// One workgroup per row. The top_k candidates come from an exact radix select over the
// row's logits (order-preserving 32-bit keys, 8 bits per pass from the top: four passes
// of a 256-bin LDS histogram find the k-th largest key), then one pass collects the keys
// above it and, of those equal to it, the lowest indices. The candidates are ranked by
// key (ties to the lower index) and one thread takes the filtered softmax and the draw in
// double: p_j = exp((l_j - l_0) / T); the shortest prefix reaching top_p of the sum; the
// prefix with p_j >= min_p; the first kept candidate whose running sum exceeds u times the
// kept sum, u the draw's 53-bit uniform.
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kSampleThreads = 1024;
constexpr int kSampleMaxK = 128;

// Order-preserving key of a finite float: larger value, larger unsigned key.
__device__ __forceinline__ uint32_t logit_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, SC'11): ten rounds over the counter with
// multipliers 0xD2511F53 and 0xCD9E8D57, the key advancing by 0x9E3779B9 and 0xBB67AE85
// between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; round++) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1, n3 = (uint32_t)p0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
  }
}

// The draw's uniform in [0, 1): counter (position low, high, 0, 0), key (seed low, high),
// the first two output words as a 53-bit fraction.
__device__ __forceinline__ double draw_uniform(uint64_t seed, uint64_t position) {
  uint32_t c[4] = {(uint32_t)position, (uint32_t)(position >> 32), 0u, 0u};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint64_t m = ((uint64_t)c[0] << 21) | (uint64_t)(c[1] >> 11);
  return ldexp((double)m, -53);
}

__global__ __launch_bounds__(kSampleThreads) void k_sample(SampleArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_state[4];            // prefix, need, count of the prefix's bin, collected
  __shared__ uint32_t ck[kSampleMaxK];
  __shared__ int ci[kSampleMaxK], s_order[kSampleMaxK];
  __shared__ double p[kSampleMaxK];        // the candidates' unnormalised probabilities
  const int r = blockIdx.x, V = a.vocab, tid = threadIdx.x, lane = tid & 63;
  const float* lg = a.logits + (long)r * V;
  const SampleParams P = a.params[r];
  const int K = min(max(P.top_k, 1), min(kSampleMaxK, V));

  // radix select of the K-th largest key
  uint32_t prefix = 0, need = (uint32_t)K, bin_count = 0;
  for (int d = 0; d < 4; d++) {
    const int shift = 24 - 8 * d;
    const uint32_t hmask = d == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    for (int v = tid; v < V; v += kSampleThreads) {
      const uint32_t k = logit_key(lg[v]);
      if ((k & hmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 255 - 4l .. 252 - 4l (largest first); a scan over the lanes
      uint32_t h[4], s = 0;
#pragma unroll
      for (int j = 0; j < 4; j++) { h[j] = hist[255 - 4 * lane - j]; s += h[j]; }
      uint32_t incl = s;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (lane >= off) incl += o;
      }
      const uint32_t excl = incl - s;
      const uint64_t hit = __ballot(incl >= need);
      const int first = (int)__builtin_ctzll(hit);   // need <= elements left, so some lane hits
      if (lane == first) {
        uint32_t c = excl;
        int j = 0;
        while (j < 3 && c + h[j] < need) { c += h[j]; j++; }
        s_state[0] = prefix | ((uint32_t)(255 - 4 * lane - j) << shift);
        s_state[1] = need - c;
        s_state[2] = h[j];
      }
    }
    __syncthreads();
    prefix = s_state[0];
    need = s_state[1];
    bin_count = s_state[2];
    __syncthreads();
  }
  // prefix is the K-th largest key T; `need` of the keys equal to T are candidates, the
  // lowest indices first. When fewer of them are wanted than exist, find the index bound B
  // with exactly `need` of them below it (a binary search, each step one counting pass).
  const uint32_t T = prefix;
  int bound = V;
  if (bin_count > need) {
    // invariant: fewer than `need` keys equal to T below lo, at least `need` below hi
    int lo = 0, hi = V;
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      if (tid == 0) s_state[3] = 0u;
      __syncthreads();
      uint32_t cnt = 0;
      for (int v = tid; v < mid; v += kSampleThreads) cnt += logit_key(lg[v]) == T ? 1u : 0u;
      if (cnt) atomicAdd(&s_state[3], cnt);
      __syncthreads();
      const uint32_t total = s_state[3];
      __syncthreads();
      if (total >= need) hi = mid; else lo = mid;
    }
    bound = hi;
  }
  if (tid == 0) s_state[3] = 0u;
  __syncthreads();
  for (int v = tid; v < V; v += kSampleThreads) {
    const uint32_t k = logit_key(lg[v]);
    if (k > T || (k == T && v < bound)) {
      const uint32_t slot = atomicAdd(&s_state[3], 1u);
      if (slot < (uint32_t)kSampleMaxK) { ck[slot] = k; ci[slot] = v; }
    }
  }
  __syncthreads();
  const int n = min((int)s_state[3], K);
  // rank: keys descending, indices ascending
  if (tid < n) {
    const uint32_t kj = ck[tid];
    const int ij = ci[tid];
    int rank = 0;
    for (int i = 0; i < n; i++) rank += (ck[i] > kj) || (ck[i] == kj && ci[i] < ij);
    s_order[min(rank, kSampleMaxK - 1)] = ij;
  }
  __syncthreads();
  if (tid == 0) {
    int pick = 0;
    const double Tm = (double)P.temperature;
    if (Tm > 0.0) {
      double all = 0.0;
      const double l0 = (double)lg[s_order[0]];
      for (int j = 0; j < n; j++) {
        p[j] = exp(((double)lg[s_order[j]] - l0) / Tm);
        all += p[j];
      }
      const double top_p = (double)P.top_p, min_p = (double)P.min_p;
      int mp = n;
      if (top_p < 1.0) {
        double c = 0.0;
        for (int j = 0; j < n; j++) {
          c += p[j];
          if (c >= top_p * all) { mp = j + 1; break; }
        }
      }
      int mm = 1;
      while (mm < n && p[mm] >= min_p) mm++;
      const int m = mp < mm ? mp : mm;
      double S = 0.0;
      for (int j = 0; j < m; j++) S += p[j];
      const double t = draw_uniform(P.seed, (uint64_t)a.position[r]) * S;
      double c = 0.0;
      pick = m - 1;
      for (int j = 0; j < m; j++) {
        c += p[j];
        if (c > t) { pick = j; break; }
      }
    }
    a.tokens[r] = s_order[pick];
  }
}

int launch_sample(const SampleArgs& a, hipStream_t s, const Prof* p) {
  launch(k_sample, dim3(a.rows), dim3(kSampleThreads), 0, s, p, a);
  return (int)hipGetLastError();
}

}  // namespace sw
