/*
 * rr_oracle.c -- plain, slow CPU oracle for RRAttention's prefill hot path.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the package smoke check and the CPU
 * baseline leg of the benchmark call this; the GPU library never does, and the
 * two share no code, header or constant.
 *
 * What it computes, following "RRAttention: Dynamic Block Sparse Attention via
 * Per-Head Round-Robin Shifts for Long-Context Inference" (abstract and TL;DR;
 * three stages in the Figure 2 caption, stride S and block B):
 *   pool    keys are aggregated per stride of S tokens (stride-level
 *           aggregation). Reading taken: the mean of the S keys, summed in
 *           float32 in token order, divided by S once, then rounded to the
 *           input dtype (bfloat16 round-to-nearest-even, or kept as float32).
 *   sample  head h samples, in every stride s, the query at in-stride offset
 *           h mod S (head round-robin sampling: the offset rotates across
 *           heads within each stride).
 *   score   each sampled query is scored against the pooled keys of its KV
 *           head, scaled by 1/sqrt(d); with the causal flag, stride t is
 *           visible to sampled stride s when t <= s. This is the
 *           O(L^2/S^2) estimate.
 *   mass    per sampled query a softmax over its visible strides; the
 *           probabilities of the strides inside key block j are summed and
 *           the r = B/S sampled queries of query block i are averaged, giving
 *           the block mass m[h][i][j] (each row sums to 1).
 *   select  adaptive Top-tau: order the row's candidate blocks by (mass
 *           descending, block index ascending) and keep the shortest prefix
 *           whose cumulative mass reaches tau times the row total: block k of
 *           the order is kept when the mass before it is < tau * total. With
 *           tau >= 1 every candidate block is kept. The last query block row
 *           is statically protected: it keeps all candidate blocks and is not
 *           searched (its masses are reported as 0).
 *   attend  exact softmax attention restricted to the keys of the selected
 *           blocks (and key <= query with the causal flag), two-pass softmax,
 *           float64 arithmetic.
 * The search runs in float32, the precision the GPU kernels take the same
 * integer decisions in; the attention runs in float64.
 *
 * Layout: Q [L][Hq][d], K and V [L][Hkv][d], batch 1; query head h reads KV
 * head h / (Hq / Hkv). Block lists: row_count [Hq][nb], col_idx [Hq][nb][nb]
 * holding the selected key blocks of row (h, i) in ascending order.
 *
 * Ragged lengths (not on the pages; the plainest extension): L need not be a
 * multiple of B or S. nb = ceil(L / B) and ns = ceil(L / S); the last stride
 * pools the tokens it has (their mean), the last key block holds the strides
 * and keys that exist, keys at or past L are never attended, and the last
 * query block (kept whole) has L - (nb - 1) B queries. A threshold per query
 * head may replace tau.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int32_t L, Hq, Hkv, d, S, B;
  float tau;
  int32_t causal;
  int32_t round_bf16; /* 1: inputs are bfloat16 values, pooled keys are rounded to bfloat16 */
} rro_problem;

/* Round a float32 to the nearest bfloat16 (ties to even), returned as float32. */
float rro_round_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7f800000u) == 0x7f800000u) { /* inf or NaN: keep, quiet the NaN */
    if (u & 0x007fffffu) u |= 0x00400000u;
    u &= 0xffff0000u;
  } else {
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    u &= 0xffff0000u;
  }
  float y;
  memcpy(&y, &u, 4);
  return y;
}

static int check_problem(const rro_problem* p) {
  if (!p) return 1;
  if (p->L <= 0 || p->Hq <= 0 || p->Hkv <= 0 || p->d <= 0 || p->S <= 0 || p->B <= 0) return 1;
  if (p->Hq % p->Hkv) return 1;
  if (p->B % p->S) return 1; /* L need not be a multiple of B or S: the last block and stride may be short */
  if (!(p->tau > 0.0f)) return 1;
  return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

int rro_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* strides and blocks of a sequence of L tokens; the last of each may be short */
static int n_strides(const rro_problem* p) { return (p->L + p->S - 1) / p->S; }
static int n_blocks(const rro_problem* p) { return (p->L + p->B - 1) / p->B; }

/* Stride pooling: Kbar[t][k][e] = mean over the tokens u of stride t
 * (u < S, and t*S + u < L for a short last stride) of K[t*S+u][k][e]. */
int rro_pool(const rro_problem* p, const float* K, float* Kbar) {
  if (check_problem(p) || !K || !Kbar) return 1;
  const int S = p->S, H = p->Hkv, d = p->d, ns = n_strides(p);
  for (int t = 0; t < ns; ++t) {
    const int cnt = p->L - t * S < S ? p->L - t * S : S;
    for (int k = 0; k < H; ++k)
      for (int e = 0; e < d; ++e) {
        float acc = 0.0f;
        for (int u = 0; u < cnt; ++u) acc += K[((size_t)(t * S + u) * H + k) * d + e];
        float mean = acc / (float)cnt;
        Kbar[((size_t)t * H + k) * d + e] = p->round_bf16 ? rro_round_bf16(mean) : mean;
      }
  }
  return 0;
}

/* ordering of candidate blocks: mass descending, then block index ascending */
typedef struct {
  float m;
  int32_t j;
} mass_idx;

static int by_mass_desc(const void* a, const void* b) {
  const mass_idx* x = (const mass_idx*)a;
  const mass_idx* y = (const mass_idx*)b;
  if (x->m > y->m) return -1;
  if (x->m < y->m) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

/*
 * Pattern search. Outputs (caller-allocated):
 *   row_count [Hq][nb], col_idx [Hq][nb][nb] (unused tail entries set to -1),
 *   mass [Hq][nb][nb]   block masses (0 outside the candidates and on the last row),
 * optional (may be NULL):
 *   cminus, cplus [Hq][nb][nb]  mass before / including block j in the ordering,
 *   rank [Hq][nb][nb]           position of block j in the ordering (-1 if no candidate),
 *   total [Hq][nb]              the row total used for the cut,
 *   kbar [L/S][Hkv][d]          the pooled keys,
 *   row_mask [Hq][nb]           compute only rows with a nonzero entry (others
 *                               get row_count 0 and are otherwise untouched),
 *   tau_heads [Hq]              a threshold per query head in place of p->tau.
 * With L not a multiple of B the last key block holds fewer strides; the
 * searched rows (every query block but the last) are full blocks, so their
 * sampled queries always exist.
 */
int rro_search(const rro_problem* p, const float* Q, const float* K, int32_t* row_count,
               int32_t* col_idx, float* mass, float* cminus, float* cplus, int32_t* rank,
               float* total, float* kbar_out, const uint8_t* row_mask, const float* tau_heads,
               int nthreads) {
  if (check_problem(p) || !Q || !K || !row_count || !col_idx || !mass) return 1;
  const int L = p->L, Hq = p->Hq, Hkv = p->Hkv, d = p->d, S = p->S, B = p->B;
  const int ns = n_strides(p), nb = n_blocks(p), r = B / S, G = Hq / Hkv;
  (void)L;
  const float sigma = 1.0f / sqrtf((float)d);
  float* Kbar = (float*)malloc(sizeof(float) * (size_t)ns * Hkv * d);
  if (!Kbar) return 2;
  rro_pool(p, K, Kbar);
  if (kbar_out) memcpy(kbar_out, Kbar, sizeof(float) * (size_t)ns * Hkv * d);
  int status = 0;
  set_threads(nthreads);

#pragma omp parallel
  {
    float* z = (float*)malloc(sizeof(float) * (size_t)ns);
    float* acc = (float*)malloc(sizeof(float) * (size_t)nb);
    mass_idx* order = (mass_idx*)malloc(sizeof(mass_idx) * (size_t)nb);
    char* keep = (char*)malloc((size_t)nb);
    if (!z || !acc || !order || !keep) {
#pragma omp atomic write
      status = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long long hi = 0; hi < (long long)Hq * nb; ++hi) {
        const int h = (int)(hi / nb), i = (int)(hi % nb);
        const int g = h / G;
        const int off = h % S; /* round-robin offset of head h */
        const int ncand = p->causal ? i + 1 : nb;
        const size_t row = (size_t)h * nb + i;
        if (row_mask && !row_mask[row]) {
          row_count[row] = 0;
          continue;
        }
        float* m = mass + row * nb;
        for (int j = 0; j < nb; ++j) m[j] = 0.0f;

        if (i < nb - 1) {
          for (int j = 0; j < nb; ++j) acc[j] = 0.0f;
          for (int a = 0; a < r; ++a) {
            const int s = i * r + a;                 /* sampled stride */
            const float* qv = Q + ((size_t)(s * S + off) * Hq + h) * d;
            const int nt = p->causal ? s + 1 : ns;   /* visible strides t <= s */
            float mu = -INFINITY;
            for (int t = 0; t < nt; ++t) {
              const float* kv = Kbar + ((size_t)t * Hkv + g) * d;
              float dot = 0.0f;
              for (int e = 0; e < d; ++e) dot += qv[e] * kv[e];
              z[t] = sigma * dot;
              if (z[t] > mu) mu = z[t];
            }
            float l = 0.0f;
            for (int t = 0; t < nt; ++t) l += expf(z[t] - mu);
            for (int t = 0; t < nt; ++t) acc[t / r] += expf(z[t] - mu) / l;
          }
          for (int j = 0; j < ncand; ++j) m[j] = acc[j] / (float)r;
        }

        /* order the candidates and take the Top-tau prefix */
        for (int j = 0; j < ncand; ++j) {
          order[j].m = m[j];
          order[j].j = j;
        }
        qsort(order, (size_t)ncand, sizeof(mass_idx), by_mass_desc);
        float run = 0.0f;
        for (int k = 0; k < ncand; ++k) {
          const int j = order[k].j;
          if (cminus) cminus[row * nb + j] = run;
          run += order[k].m;
          if (cplus) cplus[row * nb + j] = run;
          if (rank) rank[row * nb + j] = k;
        }
        const float T = run;
        if (total) total[row] = T;
        const float tau = tau_heads ? tau_heads[h] : p->tau;
        const float thr = tau * T;
        for (int j = 0; j < nb; ++j) keep[j] = 0;
        if (rank)
          for (int j = ncand; j < nb; ++j) rank[row * nb + j] = -1;
        if (i == nb - 1 || tau >= 1.0f) {
          for (int j = 0; j < ncand; ++j) keep[j] = 1;
        } else {
          float before = 0.0f;
          for (int k = 0; k < ncand; ++k) {
            if (before < thr) keep[order[k].j] = 1;
            before += order[k].m;
          }
        }
        int cnt = 0;
        int32_t* out = col_idx + row * nb;
        for (int j = 0; j < nb; ++j)
          if (keep[j]) out[cnt++] = j;
        for (int j = cnt; j < nb; ++j) out[j] = -1;
        row_count[row] = cnt;
      }
    }
    free(z);
    free(acc);
    free(order);
    free(keep);
  }
  free(Kbar);
  return status;
}

/* Lists must be ascending, in range and (causal) at most the query block. */
static int check_lists(const rro_problem* p, const int32_t* row_count, const int32_t* col_idx) {
  const int nb = n_blocks(p);
  for (long long row = 0; row < (long long)p->Hq * nb; ++row) {
    const int i = (int)(row % nb);
    const int cnt = row_count[row];
    if (cnt < 1 || cnt > nb) return 1;
    int prev = -1;
    for (int c = 0; c < cnt; ++c) {
      const int j = col_idx[row * nb + c];
      if (j <= prev || j >= nb || (p->causal && j > i)) return 1;
      prev = j;
    }
  }
  return 0;
}

/*
 * Block-sparse attention in float64. rows: NULL for every (x, h) with output
 * [L][Hq][d]; otherwise n_rows pairs (x, h) and output [n_rows][d].
 */
int rro_attention(const rro_problem* p, const float* Q, const float* K, const float* V,
                  const int32_t* row_count, const int32_t* col_idx, const int32_t* rows,
                  long long n_rows, double* out, int nthreads) {
  if (check_problem(p) || !Q || !K || !V || !row_count || !col_idx || !out) return 1;
  if (check_lists(p, row_count, col_idx)) return 3;
  const int L = p->L, Hq = p->Hq, Hkv = p->Hkv, d = p->d, B = p->B;
  const int nb = n_blocks(p), G = Hq / Hkv;
  const double sigma = 1.0 / sqrt((double)d);
  const long long total_rows = rows ? n_rows : (long long)L * Hq;
  int status = 0;
  set_threads(nthreads);

#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)L);
    int32_t* ys = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
    if (!a || !ys || !acc) {
#pragma omp atomic write
      status = 2;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (long long n = 0; n < total_rows; ++n) {
        int x, h;
        if (rows) {
          x = rows[2 * n];
          h = rows[2 * n + 1];
        } else {
          x = (int)(n / Hq);
          h = (int)(n % Hq);
        }
        double* o = out + (size_t)n * d;
        if (x < 0 || x >= L || h < 0 || h >= Hq) {
          for (int e = 0; e < d; ++e) o[e] = NAN;
          continue;
        }
        const int i = x / B, g = h / G;
        const size_t row = (size_t)h * nb + i;
        const float* qv = Q + ((size_t)x * Hq + h) * d;
        int ny = 0;
        double mx = -INFINITY;
        for (int c = 0; c < row_count[row]; ++c) {
          const int j = col_idx[row * nb + c];
          for (int y = j * B; y < (j + 1) * B && y < L; ++y) {
            if (p->causal && y > x) break;
            const float* kv = K + ((size_t)y * Hkv + g) * d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += (double)qv[e] * (double)kv[e];
            a[ny] = sigma * dot;
            ys[ny] = y;
            if (a[ny] > mx) mx = a[ny];
            ++ny;
          }
        }
        for (int e = 0; e < d; ++e) acc[e] = 0.0;
        double l = 0.0;
        for (int c = 0; c < ny; ++c) {
          const double w = exp(a[c] - mx);
          l += w;
          const float* vv = V + ((size_t)ys[c] * Hkv + g) * d;
          for (int e = 0; e < d; ++e) acc[e] += w * (double)vv[e];
        }
        for (int e = 0; e < d; ++e) o[e] = ny ? acc[e] / l : NAN;
      }
    }
    free(a);
    free(ys);
    free(acc);
  }
  return status;
}

/*
 * Mass recall of the selection against full attention: the quantity behind
 * the Figure 4 and Figure 5 captions (full-attention ground truth next to
 * the blocks RRAttention selects). For query x of head h with logits
 * a_y = Q[x,h] . K[y,g] / sqrt(d) over every admissible key y (y <= x with the
 * causal flag), the full-attention softmax mass that falls on keys of the
 * row's selected blocks is
 *   r(x) = sum_{y selected} exp(a_y - max) / sum_{y admissible} exp(a_y - max).
 * out[n] is the mean of r(x) over the B queries x of query block i for the
 * n-th requested row (h, i) (rows: n_rows pairs h, i; NULL = every row, in
 * [Hq][nb] order); a short last block averages over the queries it has.
 * float64, two passes (maximum, then the two sums).
 */
int rro_recall(const rro_problem* p, const float* Q, const float* K, const int32_t* row_count,
               const int32_t* col_idx, const int32_t* rows, long long n_rows, double* out,
               int nthreads) {
  if (check_problem(p) || !Q || !K || !row_count || !col_idx || !out) return 1;
  if (check_lists(p, row_count, col_idx)) return 3;
  const int L = p->L, Hq = p->Hq, Hkv = p->Hkv, d = p->d, B = p->B;
  const int nb = n_blocks(p), G = Hq / Hkv;
  const double sigma = 1.0 / sqrt((double)d);
  const long long total_rows = rows ? n_rows : (long long)Hq * nb;
  int status = 0;
  set_threads(nthreads);

#pragma omp parallel
  {
    double* a = (double*)malloc(sizeof(double) * (size_t)L);
    char* sel = (char*)malloc((size_t)nb);
    if (!a || !sel) {
#pragma omp atomic write
      status = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long long n = 0; n < total_rows; ++n) {
        int h, i;
        if (rows) {
          h = rows[2 * n];
          i = rows[2 * n + 1];
        } else {
          h = (int)(n / nb);
          i = (int)(n % nb);
        }
        if (h < 0 || h >= Hq || i < 0 || i >= nb) {
          out[n] = NAN;
          continue;
        }
        const int g = h / G;
        const size_t row = (size_t)h * nb + i;
        for (int j = 0; j < nb; ++j) sel[j] = 0;
        for (int c = 0; c < row_count[row]; ++c) sel[col_idx[row * nb + c]] = 1;
        double mean = 0.0;
        const int xend = (i + 1) * B < L ? (i + 1) * B : L;
        for (int x = i * B; x < xend; ++x) {
          const float* qv = Q + ((size_t)x * Hq + h) * d;
          const int ny = p->causal ? x + 1 : L;
          double mx = -INFINITY;
          for (int y = 0; y < ny; ++y) {
            const float* kv = K + ((size_t)y * Hkv + g) * d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += (double)qv[e] * (double)kv[e];
            a[y] = sigma * dot;
            if (a[y] > mx) mx = a[y];
          }
          double all = 0.0, in = 0.0;
          for (int y = 0; y < ny; ++y) {
            const double w = exp(a[y] - mx);
            all += w;
            if (sel[y / B]) in += w;
          }
          mean += in / all;
        }
        out[n] = mean / (xend - i * B);
      }
    }
    free(a);
    free(sel);
  }
  return status;
}

/*
 * Decode step (the TL;DR names decode-stage sparsification as future work;
 * the readings below are the plainest ones the prefill definition supports):
 * the cache holds L tokens, the new token's own key and value included at
 * position L - 1, and q[h] is the new query of head h (it sees every cached
 * key). Block selection reuses the prefill's pieces with the query itself in
 * place of the round-robin samples:
 *   scores  z_t = q[h] . Kbar[t][g(h)] / sqrt(d) over every stride t of the
 *           cache (Kbar as in rro_pool, the last stride possibly short);
 *   mass    m_j = sum over the strides t of key block j of softmax_t(z);
 *   select  the Top-tau prefix of the (mass desc, index asc) order, as in
 *           prefill, plus the last key block (the one holding the query),
 *           which is always kept; tau >= 1 keeps every block.
 * Attention: out[h] = softmax over the keys of the selected blocks (y < L)
 * of q[h] . K[y] / sqrt(d), applied to V; float64, two passes.
 * Outputs: row_count [Hq], col_idx [Hq][nb] (ascending, tail -1), mass
 * [Hq][nb] (float32), out [Hq][d] (float64). Search in float32 like prefill.
 */
int rro_decode(const rro_problem* p, const float* q, const float* K, const float* V, int32_t* row_count,
               int32_t* col_idx, float* mass, double* out, int nthreads) {
  if (check_problem(p) || !q || !K || !V || !row_count || !col_idx || !mass || !out) return 1;
  const int L = p->L, Hq = p->Hq, Hkv = p->Hkv, d = p->d, B = p->B;
  const int ns = n_strides(p), nb = n_blocks(p), r = B / p->S, G = Hq / Hkv;
  const float sigma = 1.0f / sqrtf((float)d);
  float* Kbar = (float*)malloc(sizeof(float) * (size_t)ns * Hkv * d);
  if (!Kbar) return 2;
  rro_pool(p, K, Kbar);
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    float* z = (float*)malloc(sizeof(float) * (size_t)ns);
    mass_idx* order = (mass_idx*)malloc(sizeof(mass_idx) * (size_t)nb);
    char* keep = (char*)malloc((size_t)nb);
    double* a = (double*)malloc(sizeof(double) * (size_t)L);
    if (!z || !order || !keep || !a) {
#pragma omp atomic write
      status = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int h = 0; h < Hq; ++h) {
        const int g = h / G;
        const float* qv = q + (size_t)h * d;
        float* m = mass + (size_t)h * nb;
        /* block masses of the query's stride softmax */
        float mu = -INFINITY;
        for (int t = 0; t < ns; ++t) {
          const float* kv = Kbar + ((size_t)t * Hkv + g) * d;
          float dot = 0.0f;
          for (int e = 0; e < d; ++e) dot += qv[e] * kv[e];
          z[t] = sigma * dot;
          if (z[t] > mu) mu = z[t];
        }
        float l = 0.0f;
        for (int t = 0; t < ns; ++t) l += expf(z[t] - mu);
        for (int j = 0; j < nb; ++j) m[j] = 0.0f;
        for (int t = 0; t < ns; ++t) m[t / r] += expf(z[t] - mu) / l;
        /* Top-tau prefix of the order, plus the last block */
        for (int j = 0; j < nb; ++j) {
          order[j].m = m[j];
          order[j].j = j;
          keep[j] = 0;
        }
        qsort(order, (size_t)nb, sizeof(mass_idx), by_mass_desc);
        float T = 0.0f;
        for (int k = 0; k < nb; ++k) T += order[k].m;
        if (p->tau >= 1.0f) {
          for (int j = 0; j < nb; ++j) keep[j] = 1;
        } else {
          float before = 0.0f;
          const float thr = p->tau * T;
          for (int k = 0; k < nb; ++k) {
            if (before < thr) keep[order[k].j] = 1;
            before += order[k].m;
          }
        }
        keep[nb - 1] = 1;
        int cnt = 0;
        int32_t* lst = col_idx + (size_t)h * nb;
        for (int j = 0; j < nb; ++j)
          if (keep[j]) lst[cnt++] = j;
        for (int j = cnt; j < nb; ++j) lst[j] = -1;
        row_count[h] = cnt;
        /* attention over the selected blocks' keys */
        int ny = 0;
        double mx = -INFINITY;
        for (int c = 0; c < cnt; ++c)
          for (int y = lst[c] * B; y < (lst[c] + 1) * B && y < L; ++y) {
            const float* kv = K + ((size_t)y * Hkv + g) * d;
            double dot = 0.0;
            for (int e = 0; e < d; ++e) dot += (double)qv[e] * (double)kv[e];
            a[ny] = dot / sqrt((double)d);
            if (a[ny] > mx) mx = a[ny];
            ++ny;
          }
        double* o = out + (size_t)h * d;
        for (int e = 0; e < d; ++e) o[e] = 0.0;
        double lsum = 0.0;
        int n = 0;
        for (int c = 0; c < cnt; ++c)
          for (int y = lst[c] * B; y < (lst[c] + 1) * B && y < L; ++y) {
            const double w = exp(a[n++] - mx);
            lsum += w;
            const float* vv = V + ((size_t)y * Hkv + g) * d;
            for (int e = 0; e < d; ++e) o[e] += w * (double)vv[e];
          }
        for (int e = 0; e < d; ++e) o[e] /= lsum;
      }
    }
    free(z);
    free(order);
    free(keep);
    free(a);
  }
  free(Kbar);
  return status;
}
