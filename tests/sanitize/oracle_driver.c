/*
 * Drives every entry point of oracle/rr_oracle.c on small seeded inputs, for
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer (the test that
 * builds it: tests/test_sanitizers_cpu.py). Shapes cover whole and ragged
 * lengths, causal and not, G = 1 and G > 1, tau < 1 and tau = 1, a row mask,
 * thresholds per head, sampled attention rows and a decode step. Exit status 0
 * when every call returns 0 and the basic invariants hold.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef struct {
  int32_t L, Hq, Hkv, d, S, B;
  float tau;
  int32_t causal;
  int32_t round_bf16;
} rro_problem;

float rro_round_bf16(float x);
int rro_pool(const rro_problem* p, const float* K, float* Kbar);
int rro_search(const rro_problem* p, const float* Q, const float* K, int32_t* row_count, int32_t* col_idx,
               float* mass, float* cminus, float* cplus, int32_t* rank, float* total, float* kbar_out,
               const uint8_t* row_mask, const float* tau_heads, int nthreads);
int rro_attention(const rro_problem* p, const float* Q, const float* K, const float* V, const int32_t* row_count,
                  const int32_t* col_idx, const int32_t* rows, long long n_rows, double* out, int nthreads);
int rro_recall(const rro_problem* p, const float* Q, const float* K, const int32_t* row_count,
               const int32_t* col_idx, const int32_t* rows, long long n_rows, double* out, int nthreads);
int rro_decode(const rro_problem* p, const float* q, const float* K, const float* V, int32_t* row_count,
               int32_t* col_idx, float* mass, double* out, int nthreads);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static float uniform(void) { /* xorshift64*, values in [-1, 1) */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (float)((state * 2685821657736338717ull) >> 40) / (float)(1u << 23) - 1.0f;
}

static float* randn(size_t n, int bf16) {
  float* a = malloc(n * sizeof(float));
  for (size_t i = 0; i < n; ++i) a[i] = bf16 ? rro_round_bf16(uniform()) : uniform();
  return a;
}

static int fail(const char* what, int rc) {
  fprintf(stderr, "FAILED: %s (%d)\n", what, rc);
  return 1;
}

static int run(int L, int Hq, int Hkv, int d, int S, int B, float tau, int causal, int bf16) {
  rro_problem p = {L, Hq, Hkv, d, S, B, tau, causal, bf16};
  const int nb = (L + B - 1) / B, ns = (L + S - 1) / S;
  float* Q = randn((size_t)L * Hq * d, bf16);
  float* K = randn((size_t)L * Hkv * d, bf16);
  float* V = randn((size_t)L * Hkv * d, bf16);
  int32_t* rc = calloc((size_t)Hq * nb, sizeof(int32_t));
  int32_t* ci = calloc((size_t)Hq * nb * nb, sizeof(int32_t));
  float* mass = calloc((size_t)Hq * nb * nb, sizeof(float));
  float* cm = calloc((size_t)Hq * nb * nb, sizeof(float));
  float* cp = calloc((size_t)Hq * nb * nb, sizeof(float));
  int32_t* rank = calloc((size_t)Hq * nb * nb, sizeof(int32_t));
  float* total = calloc((size_t)Hq * nb, sizeof(float));
  float* kbar = calloc((size_t)ns * Hkv * d, sizeof(float));
  uint8_t* mask = calloc((size_t)Hq * nb, 1);
  float* th = malloc((size_t)Hq * sizeof(float));
  double* out = calloc((size_t)L * Hq * d, sizeof(double));
  double* rec = calloc((size_t)Hq * nb, sizeof(double));
  int bad = 0, rcode;
  if ((rcode = rro_pool(&p, K, kbar))) bad |= fail("pool", rcode);
  if ((rcode = rro_search(&p, Q, K, rc, ci, mass, cm, cp, rank, total, kbar, NULL, NULL, 2)))
    bad |= fail("search", rcode);
  for (int h = 0; h < Hq && !bad; ++h)
    for (int i = 0; i < nb; ++i) {
      const int ncand = causal ? i + 1 : nb;
      if (rc[h * nb + i] < 1 || rc[h * nb + i] > ncand) bad |= fail("row count", rc[h * nb + i]);
      if (i == nb - 1 && rc[h * nb + i] != ncand) bad |= fail("last row kept whole", i);
    }
  if ((rcode = rro_attention(&p, Q, K, V, rc, ci, NULL, 0, out, 2))) bad |= fail("attention", rcode);
  for (size_t n = 0; n < (size_t)L * Hq * d; ++n)
    if (!isfinite(out[n])) {
      bad |= fail("attention output finite", (int)n);
      break;
    }
  int32_t rows[8] = {0, 0, L - 1, Hq - 1, L / 2, 0, L > 1 ? L - 2 : 0, Hq > 1 ? 1 : 0};
  if ((rcode = rro_attention(&p, Q, K, V, rc, ci, rows, 4, out, 1))) bad |= fail("attention rows", rcode);
  if ((rcode = rro_recall(&p, Q, K, rc, ci, NULL, 0, rec, 2))) bad |= fail("recall", rcode);
  int32_t rrows[4] = {0, 0, Hq - 1, nb - 1};
  if ((rcode = rro_recall(&p, Q, K, rc, ci, rrows, 2, rec, 1))) bad |= fail("recall rows", rcode);
  for (int n = 0; n < Hq * nb; ++n) mask[n] = (uint8_t)(n % 3 == 0);
  for (int h = 0; h < Hq; ++h) th[h] = h % 2 ? 0.5f : NAN;
  if ((rcode = rro_search(&p, Q, K, rc, ci, mass, NULL, NULL, NULL, NULL, NULL, mask, th, 1)))
    bad |= fail("search with a row mask and thresholds per head", rcode);
  if (causal) {
    int32_t drc[64], dci[64 * 64];
    float dmass[64 * 64];
    double dout[64 * 128];
    if (Hq <= 64 && nb <= 64 && d <= 128) {
      if ((rcode = rro_decode(&p, Q + (size_t)(L - 1) * Hq * d, K, V, drc, dci, dmass, dout, 2)))
        bad |= fail("decode", rcode);
    }
  }
  free(Q); free(K); free(V); free(rc); free(ci); free(mass); free(cm); free(cp); free(rank);
  free(total); free(kbar); free(mask); free(th); free(out); free(rec);
  return bad;
}

int main(void) {
  int bad = 0;
  bad |= run(512, 4, 2, 64, 8, 64, 0.9f, 1, 1);     /* whole blocks, bf16 values, G = 2 */
  bad |= run(1000, 3, 3, 64, 16, 128, 0.8f, 1, 0);  /* ragged length, fp32, G = 1 */
  bad |= run(300, 4, 1, 128, 4, 64, 0.95f, 0, 1);   /* non-causal, short last block and stride */
  bad |= run(256, 2, 1, 64, 8, 64, 1.0f, 1, 1);     /* tau = 1 */
  bad |= run(37, 2, 2, 64, 8, 64, 0.9f, 1, 0);      /* a single short block */
  if (!bad) printf("oracle driver ok\n");
  return bad;
}
