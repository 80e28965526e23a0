// Sampled draw of a verify window's rows: each row's token from its logits with the
// request's temperature, top_k, top_p and min_p, and a Philox4x32-10 draw keyed by the
// request's seed at the row's position.
//
// Strata docs/BATCHING.md, "Exactness": sampled rows are drawn one by one with the
// single-request window's counter-based draw, Philox(seed, position). A row's token
// depends on its own logits and parameters only, so it is the same alone or in any window;
// a slot's proposal is then verified by the greedy rule against these draws (k_accept).
//
// Two kernels, so that a row's vocabulary is spread over many compute units:
//   k_sample_cand: one 8-wave workgroup per (4096-logit chunk, row) keeps the chunk's exact
//     top K in the workspace. A logit among the row's top K is among its chunk's top K, so
//     nothing the row needs is dropped.
//   k_sample_draw: one 8-wave workgroup per row takes the row's top K from the chunks'
//     candidates the same way, ranks them, and wave 0 draws: p_j = exp((l_j - l_0) / T) in
//     double, the shorter of the top_p and min_p prefixes, the first kept candidate whose
//     running sum exceeds u times the kept sum.
// The order is by logit, then by the lower index. A workgroup's top K is found without
// sorting: all its waves run one bitwise search for the K-th largest order-preserving key,
// each round counting the keys at or above the trial value with ballots and adding the
// eight waves' counts in LDS (one barrier a round); the search stops at a trial value with
// exactly K keys at or above it, and only when keys equal to the K-th straddle the cut does
// the same search run over their indices.
#include "common.h"
#include "kernels.h"

namespace sw {

constexpr int kSampleMaxK = 128;
constexpr int kWaves = 8;                      // waves per workgroup, both kernels
constexpr int kThreads = 64 * kWaves;
constexpr int kCandPerLane = 8;                // logits per lane in k_sample_cand
constexpr int kCandChunk = kThreads * kCandPerLane;
constexpr int kDrawBatch = 7;                  // chunks a k_sample_draw wave takes per round

int sample_chunks(int vocab) { return (vocab + kCandChunk - 1) / kCandChunk; }

// Order-preserving key of a logit (larger value, larger unsigned key; -0 takes +0's key, as
// the two compare equal). Finite values and infinities map to 1 .. 2^32 - 1; key 0 stands
// for "no entry".
__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t b = __float_as_uint(v);
  if (b == 0x80000000u) b = 0u;
  return (b >> 31) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
  return __uint_as_float((k >> 31) ? (k & 0x7FFFFFFFu) : ~k);
}

// Candidates a row keeps: greedy rows (temperature <= 0) only the largest logit.
__device__ __forceinline__ int row_k(const SampleParams& P, int V) {
  if (!(P.temperature > 0.f)) return 1;
  return min(max(P.top_k, 1), min(kSampleMaxK, V));
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

// Lanes of the wave for which pred(j) holds, summed over the M entries of each lane.
template <int M, typename Pred>
__device__ __forceinline__ uint32_t wave_count(Pred pred) {
  uint32_t n = 0;
#pragma unroll
  for (int j = 0; j < M; j++) n += (uint32_t)__popcll(__ballot(pred(j)));
  return n;
}

// The same count over the whole workgroup: each wave's count meets the others' in LDS
// (two alternating slot sets, so one barrier a round suffices). Every thread gets the sum.
template <int M, typename Pred>
__device__ __forceinline__ uint32_t block_count(uint32_t (&s_cnt)[2][kWaves], int& phase, Pred pred) {
  const uint32_t n = wave_count<M>(pred);
  if ((threadIdx.x & 63) == 0) s_cnt[phase][threadIdx.x >> 6] = n;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; i++) t += s_cnt[phase][i];
  phase ^= 1;
  return t;
}

// Composite order of an entry: key, then the lower index (all composites are distinct).
__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint32_t)~idx;
}

// The largest of v over the workgroup (every thread gets it).
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t (&s_cnt)[2][kWaves], int& phase) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63) == 0) s_cnt[phase][threadIdx.x >> 6] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kWaves; i++) m = max(m, s_cnt[phase][i]);
  phase ^= 1;
  return m;
}

// A threshold with exactly K of the workgroup's entries at or above it in composite order,
// or lo << 32 when at most K entries qualify (all of them are kept). Entries with key 0 (none) or below
// `lo` (a bound known to be at or below the K-th largest key) do not qualify.
//
// Radix select over u = key - lo, 8 bits a pass from the top bit of the largest u (so the
// first pass spreads the keys over its 256 bins whatever their magnitude): every qualifying
// entry whose u agrees with the digits fixed so far adds 1 to its digit's bin (LDS atomics),
// and after a barrier every wave scans the 256 bins from the top for the bin holding the
// K-th largest. A bin holding exactly the entries still needed ends the search; when keys
// equal to the K-th straddle the cut, a bitwise search over their indices finds the last
// one kept. Every thread returns the same value.
template <int M>
__device__ uint64_t block_threshold(const uint32_t (&key)[M], const uint32_t (&idx)[M], int K, uint32_t lo,
                                    uint32_t (&s_hist)[4][256], uint32_t (&s_cnt)[2][kWaves], int& phase) {
  const int lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < 4 * 256; i += kThreads) (&s_hist[0][0])[i] = 0u;
  uint32_t u[M], umax = 0;
  bool q[M];
#pragma unroll
  for (int j = 0; j < M; j++) {
    q[j] = key[j] != 0u && key[j] >= lo;
    u[j] = q[j] ? key[j] - lo : 0u;
    umax = max(umax, u[j]);
  }
  umax = block_max(umax, s_cnt, phase);   // (its barrier also orders the zeroing)
  const int nb = 32 - __builtin_clz(umax | 1u);   // bits of the largest u
  const int pad = (8 - nb % 8) % 8;                 // digits cover bits nb + pad - 1 .. 0 of u << pad
  const int passes = (nb + pad) / 8;
  uint32_t need = (uint32_t)K, prefix = 0;   // prefix: the digits fixed so far, in u << pad
  for (int d = 0; d < passes; d++) {
    const int shift = nb + pad - 8 * (d + 1);
    const uint32_t hi_mask = d == 0 ? 0u : (0xFFFFFFFFu << (shift + 8));
#pragma unroll
    for (int j = 0; j < M; j++) {
      const uint32_t v = u[j] << pad;
      if (q[j] && (v & hi_mask) == prefix) atomicAdd(&s_hist[d][(v >> shift) & 255u], 1u);
    }
    __syncthreads();
    // lane l holds bins 255 - 4l .. 252 - 4l (largest first); a scan over the lanes
    uint32_t h[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      h[i] = s_hist[d][255 - 4 * lane - i];
      sum += h[i];
    }
    uint32_t incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)incl, off);
      if (lane >= off) incl += o;
    }
    if (d == 0 && (uint32_t)__shfl((int)incl, 63) <= need) return (uint64_t)lo << 32;   // at most K qualify
    const uint64_t hit = __ballot(incl >= need);
    const int fl = (int)__builtin_ctzll(hit);
    // in lane fl: the entries above its bins, then its bins in order
    uint32_t above = incl - sum, bin = 0, cnt = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const bool here = cnt == 0 && above + h[i] >= need;
      bin = here ? 255u - 4u * lane - i : bin;
      cnt = here ? h[i] : cnt;
      above += (cnt == 0) ? h[i] : 0u;
    }
    bin = (uint32_t)__shfl((int)bin, fl);
    cnt = (uint32_t)__shfl((int)cnt, fl);
    above = (uint32_t)__shfl((int)above, fl);
    prefix |= bin << shift;
    need -= above;
    if (cnt == need) return (uint64_t)(lo + (prefix >> pad)) << 32;
  }
  // the K-th largest key is t; `need` of the entries equal to it are kept, the lowest indices
  const uint32_t t = lo + (prefix >> pad);
  uint32_t imax = 0;
#pragma unroll
  for (int j = 0; j < M; j++) imax = max(imax, key[j] == t ? idx[j] : 0u);
  imax = block_max(imax, s_cnt, phase);
  uint32_t x = 0;   // the largest x with fewer than `need` of them below index x
  for (int b = 31 - __builtin_clz(imax | 1u); b >= 0; b--) {
    const uint32_t c = x | (1u << b);
    if (block_count<M>(s_cnt, phase, [&](int j) { return key[j] == t && idx[j] < c; }) < need) x = c;
  }
  return ((uint64_t)t << 32) | (uint32_t)~x;
}

// The same threshold by a bitwise search for the K-th largest key (for keys spread over
// many magnitudes, where the radix digits would crowd into a few bins): each round counts
// the keys at or above a trial value over the workgroup, and a trial value with exactly K
// keys at or above it ends the search.
template <int M>
__device__ uint64_t block_threshold_bits(const uint32_t (&key)[M], const uint32_t (&idx)[M], int K,
                                         uint32_t (&s_cnt)[2][kWaves], int& phase) {
  const uint32_t Ku = (uint32_t)K;
  if (block_count<M>(s_cnt, phase, [&](int j) { return key[j] != 0u; }) <= Ku) return 0;
  uint32_t t = 0;
  for (int b = 31; b >= 0; b--) {
    const uint32_t c = t | (1u << b);
    const uint32_t n = block_count<M>(s_cnt, phase, [&](int j) { return key[j] >= c; });
    if (n >= Ku) {
      t = c;
      if (n == Ku) return (uint64_t)t << 32;
    }
  }
  const uint32_t need = Ku - block_count<M>(s_cnt, phase, [&](int j) { return key[j] > t; });
  if (block_count<M>(s_cnt, phase, [&](int j) { return key[j] == t; }) == need) return (uint64_t)t << 32;
  uint32_t imax = 0;
#pragma unroll
  for (int j = 0; j < M; j++) imax = max(imax, key[j] == t ? idx[j] : 0u);
  imax = block_max(imax, s_cnt, phase);
  uint32_t x = 0;   // the largest x with fewer than `need` of them below index x
  for (int b = 31 - __builtin_clz(imax | 1u); b >= 0; b--) {
    const uint32_t c = x | (1u << b);
    if (block_count<M>(s_cnt, phase, [&](int j) { return key[j] == t && idx[j] < c; }) < need) x = c;
  }
  return ((uint64_t)t << 32) | (uint32_t)~x;
}

// The workgroup's entries at or above threshold T, packed at okey/oidx[0 ..) in wave order,
// then "no entry" up to slot K. Returns after a barrier, with the slots written.
template <int M>
__device__ __forceinline__ void block_store(const uint32_t (&key)[M], const uint32_t (&idx)[M], uint64_t T,
                                            uint32_t* okey, uint32_t* oidx, int K, uint32_t (&s_cnt)[2][kWaves],
                                            int& phase) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  bool sel[M];
#pragma unroll
  for (int j = 0; j < M; j++) sel[j] = key[j] != 0u && composite(key[j], idx[j]) >= T;
  const uint32_t n = wave_count<M>([&](int j) { return sel[j]; });
  if (lane == 0) s_cnt[phase][w] = n;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kWaves; i++) {
    const int v = (int)s_cnt[phase][i];
    base += i < w ? v : 0;
    total += v;
  }
  phase ^= 1;
#pragma unroll
  for (int j = 0; j < M; j++) {
    const uint64_t mk = __ballot(sel[j]);
    if (sel[j]) {
      const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
      okey[pos] = key[j];
      oidx[pos] = idx[j];
    }
    base += (int)__popcll(mk);
  }
  for (int s = total + (int)threadIdx.x; s < K; s += kThreads) {
    okey[s] = 0u;
    oidx[s] = 0u;
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void k_sample_cand(SampleArgs a) {
  __shared__ uint32_t s_cnt[2][kWaves];
  int phase = 0;
  const int c = blockIdx.x, r = blockIdx.y, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int V = a.vocab;
  const float* lg = a.logits + (size_t)r * V;
  const int K = row_k(a.params[r], V);
  const int base = c * kCandChunk + w * 64 * kCandPerLane;
  // every lane loads all its logits at once (past the row's end, from its last logit)
  float v[kCandPerLane];
#pragma unroll
  for (int j = 0; j < kCandPerLane; j++) v[j] = lg[min(base + 64 * j + lane, V - 1)];
  uint32_t key[kCandPerLane], idx[kCandPerLane];
#pragma unroll
  for (int j = 0; j < kCandPerLane; j++) {
    const int i = base + 64 * j + lane;
    idx[j] = (uint32_t)i;
    key[j] = i < V ? logit_key(v[j]) : 0u;
  }
  const uint64_t T = block_threshold_bits<kCandPerLane>(key, idx, K, s_cnt, phase);
  const size_t o = ((size_t)r * a.chunks + c) * kSampleMaxK;
  block_store<kCandPerLane>(key, idx, T, a.cand_key + o, a.cand_idx + o, K, s_cnt, phase);
  // the threshold's key: at most the chunk's K-th largest key, so at most the row's
  if (threadIdx.x == 0) a.cand_lo[(size_t)r * a.chunks + c] = (uint32_t)(T >> 32);
}

__global__ __launch_bounds__(kThreads) void k_sample_draw(SampleArgs a) {
  __shared__ uint32_t s_cnt[2][kWaves];
  __shared__ uint32_t s_hist[4][256];
  __shared__ uint32_t f_key[kSampleMaxK], f_idx[kSampleMaxK];
  __shared__ uint64_t f_comp[kSampleMaxK];
  __shared__ int s_order[kSampleMaxK];
  __shared__ float s_logit[kSampleMaxK];
  int phase = 0;
  const int r = blockIdx.x, w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int V = a.vocab, NC = a.chunks;
  const SampleParams P = a.params[r];
  const int K = row_k(P, V);
  const uint32_t* ck = a.cand_key + (size_t)r * NC * kSampleMaxK;
  const uint32_t* ci = a.cand_idx + (size_t)r * NC * kSampleMaxK;
  // lo: the largest of the chunks' bounds, at most the row's K-th largest key
  uint32_t lo = 0;
  for (int c = threadIdx.x; c < NC; c += kThreads) lo = max(lo, a.cand_lo[(size_t)r * NC + c]);
  lo = block_max(lo, s_cnt, phase);

  // the row's K best of the chunks' candidates, kWaves x kDrawBatch chunks a round (wave w
  // takes chunks w, w + 8, ...); from the second round on, wave 0 also holds the best K so far
  constexpr int MB = 2 + 2 * kDrawBatch;
  for (int c0 = 0; c0 < NC; c0 += kWaves * kDrawBatch) {
    uint32_t k[MB], id[MB];
    // all of the round's loads in flight together (chunks past the last read the last one's
    // slots), then the entries outside the row's chunks or past slot K masked
#pragma unroll
    for (int h = 0; h < 2; h++) {
      k[h] = f_key[lane + 64 * h];
      id[h] = f_idx[lane + 64 * h];
    }
#pragma unroll
    for (int q = 0; q < kDrawBatch; q++) {
      const size_t o = (size_t)min(c0 + w + kWaves * q, NC - 1) * kSampleMaxK + lane;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        k[2 + 2 * q + h] = ck[o + 64 * h];
        id[2 + 2 * q + h] = ci[o + 64 * h];
      }
    }
#pragma unroll
    for (int h = 0; h < 2; h++)
      if (w != 0 || c0 == 0 || lane + 64 * h >= K) k[h] = 0u;
#pragma unroll
    for (int q = 0; q < kDrawBatch; q++)
#pragma unroll
      for (int h = 0; h < 2; h++)
        if (c0 + w + kWaves * q >= NC || lane + 64 * h >= K) k[2 + 2 * q + h] = 0u;
    // (the threshold's first count is a barrier: wave 0 has read f_key before it is rewritten)
    const uint64_t T = block_threshold<MB>(k, id, K, lo, s_hist, s_cnt, phase);
    block_store<MB>(k, id, T, f_key, f_idx, K, s_cnt, phase);
  }

  // rank the K: thread t counts, for entry t / 4, the entries of its quarter that come first
  // (slots from K on hold composite 0, below every entry)
  if (threadIdx.x < kSampleMaxK)
    f_comp[threadIdx.x] = (int)threadIdx.x < K ? composite(f_key[threadIdx.x], f_idx[threadIdx.x]) : 0ull;
  __syncthreads();
  {
    const int e = threadIdx.x >> 2, part = threadIdx.x & 3;
    const uint64_t ce = f_comp[e];
    int rank = 0;
#pragma unroll
    for (int f = 32 * part; f < 32 * part + 32; f++) rank += f_comp[f] > ce ? 1 : 0;
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    if (part == 0 && e < K) {
      s_order[rank] = (int)f_idx[e];
      s_logit[rank] = key_logit(f_key[e]);
    }
  }
  __syncthreads();
  if (w != 0) return;
  int pick = 0;
  if (P.temperature > 0.f) {
    // lane l holds candidates 2l and 2l + 1
    const double T = (double)P.temperature, l0 = (double)s_logit[0];
    const int j0 = 2 * lane, j1 = 2 * lane + 1;
    const double p0 = j0 < K ? exp(((double)s_logit[j0] - l0) / T) : 0.0;
    const double p1 = j1 < K ? exp(((double)s_logit[j1] - l0) / T) : 0.0;
    double incl = p0 + p1;   // running sums over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    double excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0;
    const double c0 = excl + p0, c1 = c0 + p1;
    const double all = __shfl(incl, 63);
    // the first candidate j (in order) for which the two lane flags say yes, else `none`
    auto first = [&](bool f0, bool f1, int none) {
      const uint64_t b0 = __ballot(f0), b1 = __ballot(f1);
      const int i0 = b0 ? 2 * (int)__builtin_ctzll(b0) : none;
      const int i1 = b1 ? 2 * (int)__builtin_ctzll(b1) + 1 : none;
      return min(i0, i1);
    };
    int mp = K;   // top_p: the shortest prefix reaching top_p of the candidates' sum
    const double top_p = (double)P.top_p;
    if (top_p < 1.0) {
      const int f = first(j0 < K && c0 >= top_p * all, j1 < K && c1 >= top_p * all, K);
      if (f < K) mp = f + 1;
    }
    const double min_p = (double)P.min_p;   // min_p: the prefix with p_j >= min_p (p_0 = 1)
    const int mm = first(j0 >= 1 && j0 < K && p0 < min_p, j1 < K && p1 < min_p, K);
    const int m = min(mp, mm);
    const int jl = m - 1;
    const double S = __shfl((jl & 1) ? c1 : c0, jl >> 1);
    const double t = draw_uniform(P.seed, (uint64_t)a.position[r]) * S;
    const int f = first(j0 < m && c0 > t, j1 < m && c1 > t, m);
    pick = f < m ? f : m - 1;
  }
  if (lane == 0) a.tokens[r] = s_order[pick];
}

int launch_sample(const SampleArgs& a, hipStream_t s, const Prof* p) {
  Prof p1, p2;
  if (p) {
    p1.start = p->start;
    p2.stop = p->stop;
  }
  launch(k_sample_cand, dim3(a.chunks, a.rows), dim3(kThreads), 0, s, p ? &p1 : nullptr, a);
  launch(k_sample_draw, dim3(a.rows), dim3(kThreads), 0, s, p ? &p2 : nullptr, a);
  return (int)hipGetLastError();
}

}  // namespace sw
