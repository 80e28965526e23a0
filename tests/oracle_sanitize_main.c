/*
 * TEST INFRASTRUCTURE ONLY: a driver that runs the CPU oracle (oracle/oracle.c, compiled
 * into the same binary with AddressSanitizer and UndefinedBehaviorSanitizer) on one small
 * window read from files, and writes every result to one file, so that a test can check
 * that the oracle touches no memory outside its buffers and hits no undefined behaviour,
 * and that its results equal those of the normal build bit for bit.
 *
 * usage: oracle_sanitize <dir> R H F E K V
 *   <dir>/in.bin: x float32 [R][H]; G float32 [E][H]; then for gate, up (E x [F][H]),
 *   down (E x [H][F]), sh_gate, sh_up ([F][H]), sh_down ([H][F]) the codes (4-bit) and the
 *   meta words (uint32); then the head's codes (int8 [V][H]) and meta (uint16 [V][H/32]);
 *   then argmax/proposal int32 [R] and [R/2], then row_mask uint8 [E+1], counts float [E],
 *   resident uint8 [E].
 *   <dir>/out.bin: logits, probs [R][E] double, topk_idx [R][K] int32, topk_w double,
 *   group (n, active [A], offsets [A+1], entry_row, entry_w), out [R][H] double, x_next
 *   [R][H] uint16, head logits [R][V] double, argmax [R] int32, accept tokens [R/2][2],
 *   n_tokens [R/2], kept, tier counts [E], resident [E], swaps [2E], n_swaps.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  const uint8_t* codes;
  const void* meta;
  int32_t rows, cols, bits;
  int32_t n_mat;
  int64_t mat_stride_codes;
  int64_t mat_stride_meta;
} oracle_qmat;

void oracle_route(const void* x, int x_dtype, int R, int H, const float* G, const float* bias, int E, int K,
                  int renorm, double* logits, double* probs, int32_t* topk_idx, double* topk_w);
int oracle_group(int R, int E, int K, const int32_t* topk_idx, const double* topk_w, int32_t* active,
                 int32_t* offsets, int32_t* entry_row, double* entry_w, uint8_t* row_mask);
void oracle_moe(const void* x, int x_dtype, int R, int H, int F, const oracle_qmat* gate, const oracle_qmat* up,
                const oracle_qmat* down, const oracle_qmat* sh_gate, const oracle_qmat* sh_up,
                const oracle_qmat* sh_down, int K, const int32_t* topk_idx, const double* topk_w,
                const void* residual, double* out, uint16_t* x_next);
void oracle_head(const void* x, int x_dtype, int R, int H, const oracle_qmat* head, int v0, int v1, double* logits,
                 int32_t* argmax);
int oracle_accept(int n_slots, int mtp, const int32_t* argmax, const int32_t* proposal, int32_t* tokens,
                  int32_t* n_tokens);
void oracle_tier_count(int E, const uint8_t* row_mask, float* counts, float decay);
int oracle_tier_select(int E, const float* counts, uint8_t* resident, int max_swaps, float min_gain, int32_t* swaps);
void oracle_set_threads(int n);

static FILE* in;
static void* take(size_t n) {
  void* p = malloc(n ? n : 1);
  if (fread(p, 1, n, in) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

static oracle_qmat qm(int n_mat, int rows, int cols, int bits) {
  oracle_qmat q;
  const size_t nc = (size_t)rows * cols * bits / 8, nm = (size_t)rows * cols / 32;
  q.codes = take(n_mat * nc);
  q.meta = take(n_mat * nm * (bits == 8 ? 2 : 4));
  q.rows = rows; q.cols = cols; q.bits = bits; q.n_mat = n_mat;
  q.mat_stride_codes = (int64_t)nc; q.mat_stride_meta = (int64_t)nm;
  return q;
}

int main(int argc, char** argv) {
  if (argc != 8) return 2;
  char path[4096];
  const int R = atoi(argv[2]), H = atoi(argv[3]), F = atoi(argv[4]), E = atoi(argv[5]), K = atoi(argv[6]),
            V = atoi(argv[7]);
  snprintf(path, sizeof path, "%s/in.bin", argv[1]);
  in = fopen(path, "rb");
  if (!in) return 2;
  float* x = take(sizeof(float) * R * H);
  float* G = take(sizeof(float) * E * H);
  oracle_qmat gate = qm(E, F, H, 4), up = qm(E, F, H, 4), down = qm(E, H, F, 4);
  oracle_qmat sg = qm(1, F, H, 4), su = qm(1, F, H, 4), sd = qm(1, H, F, 4);
  oracle_qmat head = qm(1, V, H, 8);
  const int S = R / 2;
  int32_t* am_in = take(sizeof(int32_t) * R);
  int32_t* prop = take(sizeof(int32_t) * S);
  uint8_t* rmask = take(E + 1);
  float* counts = take(sizeof(float) * E);
  uint8_t* resident = take(E);
  fclose(in);

  oracle_set_threads(2);
  double* logits = malloc(sizeof(double) * R * E);
  double* probs = malloc(sizeof(double) * R * E);
  int32_t* idx = malloc(sizeof(int32_t) * R * K);
  double* w = malloc(sizeof(double) * R * K);
  oracle_route(x, 0, R, H, G, NULL, E, K, 0, logits, probs, idx, w);
  const int A = (E < R * K ? E : R * K) + 1, NE = R * K + R;
  int32_t* active = calloc(A, sizeof(int32_t));
  int32_t* offsets = calloc(A + 1, sizeof(int32_t));
  int32_t* entry_row = calloc(NE, sizeof(int32_t));
  double* entry_w = calloc(NE, sizeof(double));
  uint8_t* row_mask = calloc(E + 1, 1);
  const int n = oracle_group(R, E, K, idx, w, active, offsets, entry_row, entry_w, row_mask);
  double* out = malloc(sizeof(double) * R * H);
  uint16_t* xn = malloc(sizeof(uint16_t) * R * H);
  oracle_moe(x, 0, R, H, F, &gate, &up, &down, &sg, &su, &sd, K, idx, w, x, out, xn);
  double* hl = malloc(sizeof(double) * R * V);
  int32_t* am = malloc(sizeof(int32_t) * R);
  oracle_head(x, 0, R, H, &head, 0, V, hl, am);
  int32_t* tokens = malloc(sizeof(int32_t) * 2 * (S > 0 ? S : 1));
  int32_t* ntok = malloc(sizeof(int32_t) * (S > 0 ? S : 1));
  const int kept = oracle_accept(S, 1, am_in, prop, tokens, ntok);
  oracle_tier_count(E, rmask, counts, 0.875f);
  int32_t* swaps = malloc(sizeof(int32_t) * 2 * E);
  const int n_swaps = oracle_tier_select(E, counts, resident, E / 4, 1.5f, swaps);

  snprintf(path, sizeof path, "%s/out.bin", argv[1]);
  FILE* o = fopen(path, "wb");
  if (!o) return 2;
  fwrite(logits, sizeof(double), (size_t)R * E, o);
  fwrite(probs, sizeof(double), (size_t)R * E, o);
  fwrite(idx, sizeof(int32_t), (size_t)R * K, o);
  fwrite(w, sizeof(double), (size_t)R * K, o);
  fwrite(&n, sizeof(int), 1, o);
  fwrite(active, sizeof(int32_t), A, o);
  fwrite(offsets, sizeof(int32_t), A + 1, o);
  fwrite(entry_row, sizeof(int32_t), NE, o);
  fwrite(entry_w, sizeof(double), NE, o);
  fwrite(out, sizeof(double), (size_t)R * H, o);
  fwrite(xn, sizeof(uint16_t), (size_t)R * H, o);
  fwrite(hl, sizeof(double), (size_t)R * V, o);
  fwrite(am, sizeof(int32_t), R, o);
  fwrite(tokens, sizeof(int32_t), 2 * S, o);
  fwrite(ntok, sizeof(int32_t), S, o);
  fwrite(&kept, sizeof(int), 1, o);
  fwrite(counts, sizeof(float), E, o);
  fwrite(resident, 1, E, o);
  fwrite(swaps, sizeof(int32_t), 2 * n_swaps, o);
  fwrite(&n_swaps, sizeof(int), 1, o);
  fclose(o);
  free(x); free(G); free(logits); free(probs); free(idx); free(w); free(active); free(offsets);
  free(entry_row); free(entry_w); free(row_mask); free(out); free(xn); free(hl); free(am); free(tokens);
  free(ntok); free(swaps); free(am_in); free(prop); free(rmask); free(counts); free(resident);
  free((void*)gate.codes); free((void*)gate.meta); free((void*)up.codes); free((void*)up.meta);
  free((void*)down.codes); free((void*)down.meta); free((void*)sg.codes); free((void*)sg.meta);
  free((void*)su.codes); free((void*)su.meta); free((void*)sd.codes); free((void*)sd.meta);
  free((void*)head.codes); free((void*)head.meta);
  return 0;
}
