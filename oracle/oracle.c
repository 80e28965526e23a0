/*
 * oracle.c - TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU reference of the batched verify-window MoE layer, computed
 * in double precision. Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it; the product path never does. It shares no code, header, table or
 * helper with the HIP library: it decodes the documented byte layout itself and follows
 * the per-row definition of the layer.
 *
 * Source of the method (Strata docs):
 *   - docs/BATCHING.md "Several requests at once (batch slots)", opening paragraph: a
 *     window carries one row per conversation slot and reads the router, the shared
 *     expert, the head and every routed expert the rows use once for all of them.
 *   - same page, "Exactness": batching does not change any row's arithmetic, which is
 *     that of a window holding the row alone. So the reference computes each row alone,
 *     from its definition; grouping
 *     is computed separately (oracle_group) only to check the grouping the GPU builds.
 * Where the pages leave a step open, the readings taken are:
 *   affine dequant w = scale*q + min (q unsigned), symmetric 8-bit w = scale*q;
 *   softmax over all experts, top-k selected on logits, ties to the lower expert index;
 *   top-k weights = softmax probabilities (optionally renormalised over the k chosen);
 *   shared expert ungated with weight 1; SwiGLU h = silu(gate)*up, silu(z) = z/(1+e^-z);
 *   residual and next-layer input x_next = bf16_round_nearest_even(x + moe(x)).
 *
 * Every floating-point operation is IEEE double, without fused multiply-add
 * (build with -ffp-contract=off). Inputs in bf16, binary16 and float convert to double
 * exactly; every product of a weight and an activation is exact in double.
 *
 * Parallelism: OpenMP only across independent (row, expert) evaluations; their results
 * are combined serially in a fixed order, so the output does not depend on the thread
 * count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_F32 0
#define OR_BF16 1

/* One quantized matrix (or n_mat stacked ones), as the layout documentation states. */
typedef struct {
  const uint8_t* codes;
  const void* meta;
  int32_t rows, cols, bits;
  int32_t n_mat;
  int64_t mat_stride_codes; /* bytes */
  int64_t mat_stride_meta;  /* meta elements */
} oracle_qmat;

/* ------------------------------------------------------------------ number formats */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_to_double(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_double(uint16_t h) {
  int sign = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);   /* (1 + m/1024) * 2^(e-15) */
  return sign ? -v : v;
}

/* Round a double to the nearest bfloat16 (8 significant bits), ties to even. */
uint16_t oracle_double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
  int e;
  frexp(v, &e);                      /* |v| = f * 2^e, 0.5 <= f < 1 */
  int qexp = e - 8;                  /* quantum of an 8-bit significand */
  if (qexp < -133) qexp = -133;      /* subnormal bf16 quantum 2^-133 */
  double r = rint(ldexp(v, -qexp));  /* default rounding mode: nearest, ties to even */
  double rv = ldexp(r, qexp);
  if (fabs(rv) >= ldexp(1.0, 128)) return signbit(v) ? 0xFF80 : 0x7F80;  /* overflow */
  float f = (float)rv;               /* exact: rv has <= 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return (uint16_t)(u >> 16);
}

static double act(const void* x, int dtype, long idx) {
  if (dtype == OR_F32) return (double)((const float*)x)[idx];
  return oracle_bf16_to_double(((const uint16_t*)x)[idx]);
}

/* ---------------------------------------------------------------- quantized layout */

static int group_width(int bits) { return 512 / bits; } /* inputs per k-group */

/* Code of weight (n, k) of matrix `mat`, decoded from the documented chunk layout. */
int oracle_code(const oracle_qmat* q, int mat, int n, int k) {
  const int bits = q->bits, G = group_width(bits);
  const long t = n / 16, g = k / G, beta = (k % G) / 32, j = (k % 32) / 8, i = k % 8;
  const long lane = 16 * j + n % 16;
  const long chunk = t * (q->cols / G) + g;
  const long bit = (long)bits * (8 * beta + i);
  const uint8_t* base = q->codes + (long)mat * q->mat_stride_codes;
  const uint8_t byte = base[(chunk * 64 + lane) * 16 + bit / 8];
  int code = (byte >> (bit % 8)) & ((1 << bits) - 1);
  if (bits == 8 && code >= 128) code -= 256; /* two's complement */
  return code;
}

/* Scale and min of block b (= k / 32) of row n; min is 0 for 8-bit matrices. */
void oracle_block_meta(const oracle_qmat* q, int mat, int n, int b, double* scale,
                       double* min) {
  const int G = group_width(q->bits), bpg = G / 32;
  const long t = n / 16, g = b / bpg, beta = b % bpg;
  const long chunk = t * (q->cols / G) + g;
  const long idx = (long)mat * q->mat_stride_meta + (chunk * 16 + n % 16) * bpg + beta;
  if (q->bits == 8) {
    *scale = oracle_f16_to_double(((const uint16_t*)q->meta)[idx]);
    *min = 0.0;
  } else {
    const uint32_t m = ((const uint32_t*)q->meta)[idx];
    *scale = oracle_f16_to_double((uint16_t)(m & 0xFFFF));
    *min = oracle_f16_to_double((uint16_t)(m >> 16));
  }
}

/* Dequantized weight W[n][k] of matrix `mat`. */
double oracle_weight(const oracle_qmat* q, int mat, int n, int k) {
  double s, m;
  oracle_block_meta(q, mat, n, k / 32, &s, &m);
  return s * (double)oracle_code(q, mat, n, k) + m;
}

/* Whole matrix `mat` dequantized into out[rows][cols] (used by the tests' pins). */
void oracle_dequant(const oracle_qmat* q, int mat, double* out) {
  for (int n = 0; n < q->rows; n++)
    for (int k = 0; k < q->cols; k++) out[(long)n * q->cols + k] = oracle_weight(q, mat, n, k);
}

/* ------------------------------------------------------------------------ routing */

/*
 * Router of a window: logits, softmax probabilities, top-k experts and their weights.
 *   logits[r][e] = sum_h G[e][h] * x[r][h]  (h ascending)  + bias[e]
 *   probs[r][e]  = exp(logit - max) / sum_e' exp(logit' - max)
 *   topk: the k largest logits, descending; equal logits -> lower expert index first
 *   topk_w = probs of the chosen experts, divided by their sum when renorm != 0
 */
void oracle_route(const void* x, int x_dtype, int R, int H, const float* G,
                  const float* bias, int E, int K, int renorm, double* logits,
                  double* probs, int32_t* topk_idx, double* topk_w) {
  for (int r = 0; r < R; r++) {
    double* l = logits + (long)r * E;
    for (int e = 0; e < E; e++) {
      double s = 0.0;
      for (int h = 0; h < H; h++) s += (double)G[(long)e * H + h] * act(x, x_dtype, (long)r * H + h);
      l[e] = s + (bias ? (double)bias[e] : 0.0);
    }
    double mx = l[0];
    for (int e = 1; e < E; e++)
      if (l[e] > mx) mx = l[e];
    double z = 0.0;
    for (int e = 0; e < E; e++) z += exp(l[e] - mx);
    for (int e = 0; e < E; e++) probs[(long)r * E + e] = exp(l[e] - mx) / z;

    /* selection: repeatedly take the best expert not yet taken */
    char taken[1024];
    memset(taken, 0, sizeof taken);
    for (int j = 0; j < K; j++) {
      int best = -1;
      for (int e = 0; e < E; e++) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e; /* strict '>' keeps the lower index */
      }
      taken[best] = 1;
      topk_idx[r * K + j] = best;
      topk_w[r * K + j] = probs[(long)r * E + best];
    }
    if (renorm) {
      double s = 0.0;
      for (int j = 0; j < K; j++) s += topk_w[r * K + j];
      for (int j = 0; j < K; j++) topk_w[r * K + j] /= s;
    }
  }
}

/*
 * Per-expert row lists of the window, from the top-k choice: experts ascending, each
 * with its rows ascending; the shared expert (id E) last with every row and weight 1.
 * Returns the number of active experts.
 */
int oracle_group(int R, int E, int K, const int32_t* topk_idx, const double* topk_w,
                 int32_t* active, int32_t* offsets, int32_t* entry_row,
                 double* entry_w, uint8_t* row_mask) {
  int n = 0, pos = 0;
  for (int e = 0; e <= E; e++) {
    unsigned mask = 0;
    for (int r = 0; r < R; r++) {
      if (e == E) { mask |= 1u << r; continue; }
      for (int j = 0; j < K; j++)
        if (topk_idx[r * K + j] == e) mask |= 1u << r;
    }
    row_mask[e] = (uint8_t)mask;
    if (!mask) continue;
    active[n] = e;
    offsets[n] = pos;
    for (int r = 0; r < R; r++) {
      if (!(mask >> r & 1)) continue;
      double w = 1.0;
      if (e < E)
        for (int j = 0; j < K; j++)
          if (topk_idx[r * K + j] == e) w = topk_w[r * K + j];
      entry_row[pos] = r;
      entry_w[pos] = w;
      pos++;
    }
    n++;
  }
  offsets[n] = pos;
  return n;
}

/* ------------------------------------------------------------------------ experts */

static double silu(double z) { return z / (1.0 + exp(-z)); }

/*
 * One expert on one row: h[f] = silu(sum_k Wg[f][k] x[k]) * (sum_k Wu[f][k] x[k]),
 * y[n] = sum_f Wd[n][f] h[f]; every sum with its index ascending.
 */
void oracle_expert(const oracle_qmat* gate, const oracle_qmat* up, const oracle_qmat* down,
                   int mat, const double* xr, int H, int F, double* y) {
  double* h = (double*)malloc(sizeof(double) * F);
  for (int f = 0; f < F; f++) {
    double g = 0.0, u = 0.0;
    for (int k = 0; k < H; k++) g += oracle_weight(gate, mat, f, k) * xr[k];
    for (int k = 0; k < H; k++) u += oracle_weight(up, mat, f, k) * xr[k];
    h[f] = silu(g) * u;
  }
  for (int n = 0; n < H; n++) {
    double s = 0.0;
    for (int f = 0; f < F; f++) s += oracle_weight(down, mat, n, f) * h[f];
    y[n] = s;
  }
  free(h);
}

/*
 * The experts of a window, row by row from the definition:
 *   out[r] = sum_j topk_w[r][j] * FFN_{topk_idx[r][j]}(x_r) + FFN_shared(x_r)
 *            (+ residual[r] when residual != NULL)
 * summed in the order j = 0..K-1, shared last, then the residual.
 * x_next (may be NULL) = bf16 round-to-nearest-even of out.
 */
void oracle_moe(const void* x, int x_dtype, int R, int H, int F, const oracle_qmat* gate,
                const oracle_qmat* up, const oracle_qmat* down, const oracle_qmat* sh_gate,
                const oracle_qmat* sh_up, const oracle_qmat* sh_down, int K,
                const int32_t* topk_idx, const double* topk_w, const void* residual,
                double* out, uint16_t* x_next) {
  const int per_row = K + 1;
  double* xd = (double*)malloc(sizeof(double) * R * H);
  double* y = (double*)malloc(sizeof(double) * (long)R * per_row * H);
  for (long i = 0; i < (long)R * H; i++) xd[i] = act(x, x_dtype, i);

#pragma omp parallel for schedule(dynamic, 1)
  for (int t = 0; t < R * per_row; t++) {
    const int r = t / per_row, j = t % per_row;
    double* yt = y + (long)t * H;
    if (j < K)
      oracle_expert(gate, up, down, topk_idx[r * K + j], xd + (long)r * H, H, F, yt);
    else
      oracle_expert(sh_gate, sh_up, sh_down, 0, xd + (long)r * H, H, F, yt);
  }

  for (int r = 0; r < R; r++)
    for (int n = 0; n < H; n++) {
      double s = 0.0;
      for (int j = 0; j < K; j++) s += topk_w[r * K + j] * y[((long)r * per_row + j) * H + n];
      s += y[((long)r * per_row + K) * H + n];
      if (residual) s += act(residual, x_dtype, (long)r * H + n);
      out[(long)r * H + n] = s;
      if (x_next) x_next[(long)r * H + n] = oracle_double_to_bf16(s);
    }
  free(y);
  free(xd);
}

/* --------------------------------------------------------------------------- head */

/*
 * Output head: logits[r][v] = sum_h W[v][h] x[r][h] (h ascending) for the rows' vocab
 * entries v in [v0, v1); argmax over that range, the lowest v on ties. logits is
 * [R][v1 - v0]. (A sub-range lets the tests sample a large vocabulary.)
 */
void oracle_head(const void* x, int x_dtype, int R, int H, const oracle_qmat* head, int v0,
                 int v1, double* logits, int32_t* argmax) {
  const int nv = v1 - v0;
#pragma omp parallel for schedule(static)
  for (int v = v0; v < v1; v++)
    for (int r = 0; r < R; r++) {
      double s = 0.0;
      for (int h = 0; h < H; h++) s += oracle_weight(head, 0, v, h) * act(x, x_dtype, (long)r * H + h);
      logits[(long)r * nv + (v - v0)] = s;
    }
  for (int r = 0; r < R; r++) {
    int best = 0;
    for (int v = 1; v < nv; v++)
      if (logits[(long)r * nv + v] > logits[(long)r * nv + best]) best = v;
    argmax[r] = v0 + best;
  }
}

/* ------------------------------------------------------------------ verify/accept */

/*
 * Greedy verification of a window's MTP proposals (Strata docs/BATCHING.md, the
 * --batch-mtp paragraph: each slot verifies one proposal alongside its current token, so
 * a window carries two rows per slot; docs/MULTI_GPU.md, the --pipeline-windows
 * paragraph: a window accepted whole also yields a bonus token).
 *
 * Rows: with mtp, slot s owns rows 2s (its current token) and 2s + 1 (its proposal);
 * without, row s. argmax[r] is the model's next token after row r (the head's argmax).
 * A slot's proposal is kept when it equals the next token after the slot's token row;
 * the slot then emits the proposal and the next token after the proposal row (two
 * tokens), otherwise the next token after its token row alone (one token). tokens is
 * [n_slots][2] (-1 where unused), n_tokens [n_slots]. Returns the number of kept
 * proposals.
 */
int oracle_accept(int n_slots, int mtp, const int32_t* argmax, const int32_t* proposal,
                  int32_t* tokens, int32_t* n_tokens) {
  int kept = 0;
  for (int s = 0; s < n_slots; s++) {
    const int32_t next_after_token = argmax[mtp ? 2 * s : s];
    tokens[2 * s] = next_after_token;
    tokens[2 * s + 1] = -1;
    n_tokens[s] = 1;
    if (mtp && proposal[s] == next_after_token) {
      tokens[2 * s + 1] = argmax[2 * s + 1];
      n_tokens[s] = 2;
      kept++;
    }
  }
  return kept;
}

/* ------------------------------------------------------------------ sampled draw */

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel
 * random numbers: as easy as 1, 2, 3", SC'11), written from the paper's definition: ten
 * rounds over a 128-bit counter (c0, c1, c2, c3) with a 64-bit key (k0, k1). A round takes
 * the two 64-bit products M0 * c0 and M1 * c2 (M0 = 0xD2511F53, M1 = 0xCD9E8D57) and
 * forms (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); between rounds
 * the key advances by the Weyl constants (0x9E3779B9, 0xBB67AE85).
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
  uint32_t k0 = key[0], k1 = key[1];
  for (int round = 0; round < 10; round++) {
    if (round > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0, n1 = (uint32_t)p1;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1, n3 = (uint32_t)p0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * The draw of one row (Strata docs/BATCHING.md, "Exactness": sampled rows are drawn one
 * by one with the single-request window's counter-based draw, Philox(seed, position)).
 * Reading: the key is the request's 64-bit seed (low word first), the counter the row's
 * 64-bit position (low word first) and two zero words; the uniform is the first two output
 * words as a 53-bit fraction, u = (out0 * 2^21 + out1 / 2^11) / 2^53 in [0, 1).
 */
double oracle_uniform(uint64_t seed, uint64_t position) {
  const uint32_t ctr[4] = {(uint32_t)position, (uint32_t)(position >> 32), 0u, 0u};
  const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t o[4];
  oracle_philox4x32_10(ctr, key, o);
  const uint64_t m = ((uint64_t)o[0] << 21) | (uint64_t)(o[1] >> 11);
  return ldexp((double)m, -53);
}

/*
 * A sampled token from one row's logits [V] (the head's output), with the request's
 * temperature, top_k, top_p, min_p and seed, at the row's position. Readings where the
 * pages name the parameters only:
 *   1. candidates: the top_k largest logits (ties to the lower index), top_k clamped to
 *      1 .. min(128, V), listed by logit descending, then index ascending;
 *   2. temperature <= 0: the first candidate (greedy: the lowest index of the largest
 *      logit); else p_j = exp((l_j - l_0) / T) (l_0 the largest), unnormalised;
 *   3. top_p: the shortest prefix of the list whose sum reaches top_p times the sum of
 *      all candidates (top_p >= 1: the whole list);
 *   4. min_p: the prefix of candidates with p_j >= min_p (min_p times the largest, which
 *      is 1); the kept prefix is the shorter of the two, at least one candidate;
 *   5. with S the sum of the kept p_j and u = oracle_uniform(seed, position), the token is
 *      the first kept candidate whose running sum exceeds u * S.
 * All in double, j ascending. *margin (may be NULL) receives the smallest relative
 * distance of a decision to its boundary (the running sum against u * S, the top_p and
 * min_p cuts), so a test can tell the decisions another summation order might flip.
 */
int oracle_sample(const float* logits, int V, double temperature, int top_k, double top_p, double min_p,
                  uint64_t seed, uint64_t position, double* margin) {
  int K = top_k < 1 ? 1 : top_k;
  if (K > 128) K = 128;
  if (K > V) K = V;
  int cand[128];
  char* taken = (char*)calloc((size_t)V, 1);
  for (int j = 0; j < K; j++) {
    int best = -1;
    for (int v = 0; v < V; v++) {
      if (taken[v]) continue;
      if (best < 0 || logits[v] > logits[best]) best = v; /* strict '>' keeps the lower index */
    }
    taken[best] = 1;
    cand[j] = best;
  }
  free(taken);
  double mg = INFINITY;
  if (!(temperature > 0.0)) {
    if (margin) *margin = mg;
    return cand[0];
  }
  double p[128], all = 0.0;
  for (int j = 0; j < K; j++) {
    p[j] = exp(((double)logits[cand[j]] - (double)logits[cand[0]]) / temperature);
    all += p[j];
  }
  int mp = K;
  if (top_p < 1.0) {
    double c = 0.0;
    for (int j = 0; j < K; j++) {
      c += p[j];
      if (c >= top_p * all) {
        mp = j + 1;
        mg = fmin(mg, fabs(c - top_p * all) / all);
        if (j > 0) mg = fmin(mg, fabs(c - p[j] - top_p * all) / all);
        break;
      }
    }
  }
  int mm = 1;
  while (mm < K && p[mm] >= min_p) mm++;
  if (min_p > 0.0) {
    mg = fmin(mg, fabs(p[mm - 1] - min_p));
    if (mm < K) mg = fmin(mg, fabs(p[mm] - min_p));
  }
  const int m = mp < mm ? mp : mm;
  double S = 0.0;
  for (int j = 0; j < m; j++) S += p[j];
  const double t = oracle_uniform(seed, position) * S;
  double c = 0.0;
  int pick = m - 1;
  for (int j = 0; j < m; j++) {
    c += p[j];
    if (c > t) {
      pick = j;
      break;
    }
  }
  /* the running sums on either side of the pick */
  c = 0.0;
  for (int j = 0; j < m; j++) {
    c += p[j];
    if (j == pick - 1 || j == pick) mg = fmin(mg, fabs(c - t) / S);
  }
  if (margin) *margin = mg;
  return cand[pick];
}

/* ---------------------------------------------------------- routing counts and tier */

/*
 * Expert routing counts and the adaptive tier's swap choice (Strata docs/BATCHING.md,
 * the paragraph on batch windows counting the experts they route to, with --adapt-every,
 * --adapt-decay and --adapt-min-gain F, whose default is 1.5): the windows' routing builds
 * per-expert counts; a periodic round exchanges heavily used experts outside the fast tier
 * for lightly used resident ones, and an exchange needs the incoming count to reach F
 * times the outgoing one.
 *
 * Readings where the pages leave the step open: a window adds, for each routed expert e,
 * the number of its rows that route to e (row_mask[e]'s bits), after scaling the running
 * count by decay: counts[e] = fmaf(counts[e], decay, rows_e), in float (the same
 * precision on every side, since the comparisons below decide integers).
 */
void oracle_tier_count(int E, const uint8_t* row_mask, float* counts, float decay) {
  for (int e = 0; e < E; e++) {
    int n = 0;
    for (int r = 0; r < 8; r++) n += (row_mask[e] >> r) & 1;
    counts[e] = fmaf(counts[e], decay, (float)n);
  }
}

typedef struct { float c; int e; } tier_key;
static int by_count_desc(const void* a, const void* b) {
  const tier_key *x = a, *y = b;
  if (x->c != y->c) return x->c > y->c ? -1 : 1;
  return x->e - y->e;
}
static int by_count_asc(const void* a, const void* b) {
  const tier_key *x = a, *y = b;
  if (x->c != y->c) return x->c < y->c ? -1 : 1;
  return x->e - y->e;
}

/*
 * The swap choice of one round: the experts outside the tier ordered by count, largest
 * first, and the resident ones ordered by count, smallest first (ties: the lower expert
 * index first, in both lists); pair i swaps in_i for out_i while in_i's count is positive
 * and at least min_gain * out_i's count (the product in float), for at most max_swaps
 * pairs. resident[] is updated; swaps receives (in, out) pairs. Returns the swap count.
 */
int oracle_tier_select(int E, const float* counts, uint8_t* resident, int max_swaps, float min_gain,
                       int32_t* swaps) {
  tier_key* in = malloc(sizeof(tier_key) * (E > 0 ? E : 1));
  tier_key* out = malloc(sizeof(tier_key) * (E > 0 ? E : 1));
  int n_in = 0, n_out = 0;
  for (int e = 0; e < E; e++) {
    tier_key k = {counts[e], e};
    if (resident[e]) out[n_out++] = k; else in[n_in++] = k;
  }
  qsort(in, n_in, sizeof(tier_key), by_count_desc);
  qsort(out, n_out, sizeof(tier_key), by_count_asc);
  int n = 0;
  while (n < max_swaps && n < n_in && n < n_out) {
    const float bar = min_gain * out[n].c;
    if (!(in[n].c > 0.0f && in[n].c >= bar)) break;
    swaps[2 * n] = in[n].e;
    swaps[2 * n + 1] = out[n].e;
    n++;
  }
  for (int i = 0; i < n; i++) {
    resident[swaps[2 * i]] = 1;
    resident[swaps[2 * i + 1]] = 0;
  }
  free(in);
  free(out);
  return n;
}

/* Threads for the parallel loops above (n >= 1; no effect without OpenMP). */
void oracle_set_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  if (n >= 1) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Threads OpenMP would use for the parallel loops above (1 without OpenMP). */
int oracle_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
