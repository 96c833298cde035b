/*
 * kascade_oracle.c -- fp64 reference for Kascade's cross-layer top-k sparse
 * attention. TEST INFRASTRUCTURE ONLY (see kascade_oracle.h): it is called by
 * the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
 * GPU library.
 *
 * Every step is the plain definition, computed in double precision with
 * natural j-ascending summation, one independent unit per OpenMP iteration.
 * There is no blocking, fusion or reordering beyond that.
 */
#include "kascade_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ERR_PROBLEM (-1)
#define ERR_UNIT (-2)
#define ERR_INDEX (-3)
#define ERR_NOMEM (-4)

/* Record a failure from inside a parallel loop. */
static void fail(int* status, int code) {
#pragma omp atomic write
  *status = code;
}

/* One stored element as an exact double. bfloat16 is the upper half of an
 * IEEE float32, so widening the 16 bits into the top of a 32-bit word is exact. */
static double element(const void* base, int dtype, size_t i) {
  if (dtype == 0) return (double)((const float*)base)[i];
  uint32_t bits = (uint32_t)((const uint16_t*)base)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int problem_ok(const oracle_problem* p) {
  if (!p) return 0;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1) return 0;
  if (p->num_q_heads % p->num_kv_heads != 0) return 0;
  if (p->q_len < 1 || p->kv_len < 1 || p->top_k < 1) return 0;
  if (p->dtype != 0 && p->dtype != 1) return 0;
  if (p->shared_index_set != 0 && p->shared_index_set != 1) return 0;
  return 1;
}

/* Index sets per batch row: one per KV head (head-aware selection), or one
 * shared by every head (the non-head-aware ablation). */
static int index_sets(const oracle_problem* p) {
  return p->shared_index_set ? 1 : p->num_kv_heads;
}

/* The index set that query head h attends through. */
static int set_of_head(const oracle_problem* p, int h) {
  return p->shared_index_set ? 0 : h / (p->num_q_heads / p->num_kv_heads);
}

/* The query heads whose probabilities are pooled into index set `set`:
 * heads h0 .. h0+nh-1 (the KV head's group, or all heads for a shared set). */
static void pooled_heads(const oracle_problem* p, int set, int* h0, int* nh) {
  const int G = p->num_q_heads / p->num_kv_heads;
  if (p->shared_index_set) {
    *h0 = 0;
    *nh = p->num_q_heads;
  } else {
    *h0 = set * G;
    *nh = G;
  }
}

static size_t q_offset(const oracle_problem* p, int b, int h, int i) {
  return (((size_t)b * p->num_q_heads + h) * p->q_len + i) * p->head_dim;
}

static size_t kv_offset(const oracle_problem* p, int b, int kvh, int j) {
  return (((size_t)b * p->num_kv_heads + kvh) * p->kv_len + j) * p->head_dim;
}

/* Attention logit of query row (b, h, i) against key j of KV head kvh:
 * scale * <q, k_j>. */
static double logit(const oracle_problem* p, const void* q, const void* k,
                    int b, int h, int i, int kvh, int j) {
  size_t qo = q_offset(p, b, h, i), ko = kv_offset(p, b, kvh, j);
  double acc = 0.0;
  for (int c = 0; c < p->head_dim; ++c)
    acc += element(q, p->dtype, qo + c) * element(k, p->dtype, ko + c);
  return p->scale * acc;
}

/* Softmax of s[0..n) in place: s[j] <- exp(s[j] - m) / sum. Returns the
 * log-sum-exp m + log(sum). */
static double softmax_inplace(double* s, int n) {
  double m = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (s[j] > m) m = s[j];
  double l = 0.0;
  for (int j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    l += s[j];
  }
  for (int j = 0; j < n; ++j) s[j] /= l;
  return m + log(l);
}

/* ---- exact top-k -------------------------------------------------------- */

typedef struct {
  double value;
  int32_t j;
} ranked_key;

/* Larger pooled value first; equal values go to the lower key index. */
static int rank_order(const void* a, const void* b) {
  const ranked_key* x = (const ranked_key*)a;
  const ranked_key* y = (const ranked_key*)b;
  if (x->value > y->value) return -1;
  if (x->value < y->value) return 1;
  return (x->j > y->j) - (x->j < y->j);
}

static int ascending(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* The min(k, n) keys with the largest score[0..n), written ascending into
 * out[0..), followed by -1 up to slot k. Full sort, no partial selection. */
static int select_top_k(const double* score, int n, int k, int32_t* out) {
  ranked_key* r = (ranked_key*)malloc((size_t)n * sizeof *r);
  if (!r) return ERR_NOMEM;
  for (int j = 0; j < n; ++j) {
    r[j].value = score[j];
    r[j].j = j;
  }
  qsort(r, (size_t)n, sizeof *r, rank_order);
  int kt = k < n ? k : n;
  for (int s = 0; s < kt; ++s) out[s] = r[s].j;
  qsort(out, (size_t)kt, sizeof *out, ascending);
  for (int s = kt; s < k; ++s) out[s] = -1;
  free(r);
  return 0;
}

static void set_threads(int nthreads) {
  if (nthreads > 0) omp_set_num_threads(nthreads);
}

/* ---- anchor, decode ------------------------------------------------------ */

int oracle_anchor_decode(const oracle_problem* p, const void* q, const void* k,
                         const int32_t* units, int nunits,
                         int32_t* idx_out, double* pooled_out, int nthreads) {
  if (!problem_ok(p) || p->q_len != 1 || p->top_k > p->kv_len || !q || !k || !idx_out)
    return ERR_PROBLEM;
  const int G = p->num_q_heads / p->num_kv_heads, N = p->kv_len, S = index_sets(p);
  const int total = p->batch * S;
  const int n = units ? nunits : total;
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)N * sizeof(double));
    double* pooled = (double*)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
      int b = units ? units[2 * u] : u / S;
      int set = units ? units[2 * u + 1] : u % S;
      if (!s || !pooled) { fail(&status, ERR_NOMEM); continue; }
      if (b < 0 || b >= p->batch || set < 0 || set >= S) { fail(&status, ERR_UNIT); continue; }
      int h0, nh;
      pooled_heads(p, set, &h0, &nh);
      for (int j = 0; j < N; ++j) pooled[j] = 0.0;
      for (int h = h0; h < h0 + nh; ++h) {
        /* query head h reads KV head h / G; a group's heads are contiguous */
        for (int j = 0; j < N; ++j) s[j] = logit(p, q, k, b, h, 0, h / G, j);
        softmax_inplace(s, N);
        for (int j = 0; j < N; ++j) pooled[j] += s[j];
      }
      for (int j = 0; j < N; ++j) pooled[j] /= nh;
      if (select_top_k(pooled, N, p->top_k, idx_out + (size_t)u * p->top_k)) fail(&status, ERR_NOMEM);
      if (pooled_out) memcpy(pooled_out + (size_t)u * N, pooled, (size_t)N * sizeof(double));
    }
    free(s);
    free(pooled);
  }
  return status;
}

/* ---- anchor, causal prefill --------------------------------------------- */

int oracle_anchor_prefill(const oracle_problem* p, const void* q, const void* k,
                          const int32_t* units, int nunits,
                          int32_t* idx_out, double* pooled_out, int nthreads) {
  if (!problem_ok(p) || p->q_len != p->kv_len || p->q_tile < 1 || !q || !k || !idx_out)
    return ERR_PROBLEM;
  const int G = p->num_q_heads / p->num_kv_heads, N = p->kv_len, T = p->q_tile, S = index_sets(p);
  const int tiles = (N + T - 1) / T;
  const int total = p->batch * S * tiles;
  const int n = units ? nunits : total;
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)N * sizeof(double));
    double* pooled = (double*)malloc((size_t)N * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
      int b, set, t;
      if (units) {
        b = units[3 * u]; set = units[3 * u + 1]; t = units[3 * u + 2];
      } else {
        b = u / (S * tiles);
        set = (u / tiles) % S;
        t = u % tiles;
      }
      if (!s || !pooled) { fail(&status, ERR_NOMEM); continue; }
      if (b < 0 || b >= p->batch || set < 0 || set >= S || t < 0 || t >= tiles) {
        fail(&status, ERR_UNIT);
        continue;
      }
      const int row0 = t * T;
      const int prefix = (t + 1) * T < N ? (t + 1) * T : N; /* rows of the tile end here too */
      const int rows = prefix - row0;
      int h0, nh;
      pooled_heads(p, set, &h0, &nh);
      for (int j = 0; j < N; ++j) pooled[j] = 0.0;
      for (int h = h0; h < h0 + nh; ++h) {
        for (int i = row0; i < prefix; ++i) {
          /* causal row i sees keys 0..i */
          for (int j = 0; j <= i; ++j) s[j] = logit(p, q, k, b, h, i, h / G, j);
          softmax_inplace(s, i + 1);
          for (int j = 0; j <= i; ++j) pooled[j] += s[j];
        }
      }
      for (int j = 0; j < prefix; ++j) pooled[j] /= (double)nh * rows;
      if (select_top_k(pooled, prefix, p->top_k, idx_out + (size_t)u * p->top_k)) fail(&status, ERR_NOMEM);
      if (pooled_out) memcpy(pooled_out + (size_t)u * N, pooled, (size_t)N * sizeof(double));
    }
    free(s);
    free(pooled);
  }
  return status;
}

/* ---- softmax attention over an explicit key list ------------------------- */

/* out[0..d) = sum_{j in keys} softmax_j(logits) * v_j for query row (b, h, i).
 * An empty list gives zeros. Returns the log-sum-exp (or -inf if empty). */
static double attend(const oracle_problem* p, const void* q, const void* k, const void* v,
                     int b, int h, int i, const int32_t* keys, int nkeys,
                     double* s, double* out) {
  const int kvh = h / (p->num_q_heads / p->num_kv_heads), d = p->head_dim;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  if (nkeys == 0) return -INFINITY;
  for (int a = 0; a < nkeys; ++a) s[a] = logit(p, q, k, b, h, i, kvh, keys[a]);
  double lse = softmax_inplace(s, nkeys);
  if (v) {
    for (int a = 0; a < nkeys; ++a) {
      size_t vo = kv_offset(p, b, kvh, keys[a]);
      for (int c = 0; c < d; ++c) out[c] += s[a] * element(v, p->dtype, vo + c);
    }
  }
  return lse;
}

/* ---- reuse, decode ------------------------------------------------------- */

int oracle_reuse_decode(const oracle_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* units, int nunits,
                        double* out, int nthreads) {
  if (!problem_ok(p) || p->q_len != 1 || !q || !k || !v || !idx || !out) return ERR_PROBLEM;
  const int N = p->kv_len, K = p->top_k;
  const int total = p->batch * p->num_q_heads;
  const int n = units ? nunits : total;
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)K * sizeof(double));
    int32_t* keys = (int32_t*)malloc((size_t)K * sizeof(int32_t));
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
      int b = units ? units[2 * u] : u / p->num_q_heads;
      int h = units ? units[2 * u + 1] : u % p->num_q_heads;
      if (!s || !keys) { fail(&status, ERR_NOMEM); continue; }
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_q_heads) { fail(&status, ERR_UNIT); continue; }
      const int32_t* list = idx + ((size_t)b * index_sets(p) + set_of_head(p, h)) * K;
      int nk = 0;
      for (int a = 0; a < K; ++a) {
        if (list[a] == -1) continue;             /* padding */
        if (list[a] < 0 || list[a] >= N) { fail(&status, ERR_INDEX); nk = -1; break; }
        keys[nk++] = list[a];
      }
      if (nk < 0) continue;
      attend(p, q, k, v, b, h, 0, keys, nk, s, out + (size_t)u * p->head_dim);
    }
    free(s);
    free(keys);
  }
  return status;
}

/* ---- reuse, causal prefill ------------------------------------------------ */

int oracle_reuse_prefill(const oracle_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* units, int nunits,
                         double* out, int nthreads) {
  if (!problem_ok(p) || p->q_len != p->kv_len || p->q_tile < 1 || !q || !k || !v || !idx || !out)
    return ERR_PROBLEM;
  const int N = p->kv_len, K = p->top_k, T = p->q_tile;
  const int tiles = (N + T - 1) / T;
  const int total = p->batch * p->num_q_heads * N;
  const int n = units ? nunits : total;
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)K * sizeof(double));
    int32_t* keys = (int32_t*)malloc((size_t)K * sizeof(int32_t));
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
      int b, h, i;
      if (units) {
        b = units[3 * u]; h = units[3 * u + 1]; i = units[3 * u + 2];
      } else {
        b = u / (p->num_q_heads * N);
        h = (u / N) % p->num_q_heads;
        i = u % N;
      }
      if (!s || !keys) { fail(&status, ERR_NOMEM); continue; }
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_q_heads || i < 0 || i >= N) {
        fail(&status, ERR_UNIT);
        continue;
      }
      const int t = i / T;
      const int32_t* list = idx + (((size_t)b * index_sets(p) + set_of_head(p, h)) * tiles + t) * K;
      int nk = 0;
      for (int a = 0; a < K; ++a) {
        if (list[a] == -1) continue;
        if (list[a] < 0 || list[a] >= N) { fail(&status, ERR_INDEX); nk = -1; break; }
        if (list[a] <= i) keys[nk++] = list[a];  /* causal restriction */
      }
      if (nk < 0) continue;
      attend(p, q, k, v, b, h, i, keys, nk, s, out + (size_t)u * p->head_dim);
    }
    free(s);
    free(keys);
  }
  return status;
}

/* ---- dense --------------------------------------------------------------- */

int oracle_dense(const oracle_problem* p, const void* q, const void* k, const void* v,
                 int causal, const int32_t* units, int nunits,
                 double* out, double* lse, int nthreads) {
  if (!problem_ok(p) || !q || !k || (out && !v)) return ERR_PROBLEM;
  if (causal && p->q_len != p->kv_len) return ERR_PROBLEM;
  const int N = p->kv_len, L = p->q_len, d = p->head_dim;
  const int total = p->batch * p->num_q_heads * L;
  const int n = units ? nunits : total;
  int status = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double* s = (double*)malloc((size_t)N * sizeof(double));
    int32_t* keys = (int32_t*)malloc((size_t)N * sizeof(int32_t));
    double* o = (double*)malloc((size_t)d * sizeof(double));
#pragma omp for schedule(dynamic, 1)
    for (int u = 0; u < n; ++u) {
      int b, h, i;
      if (units) {
        b = units[3 * u]; h = units[3 * u + 1]; i = units[3 * u + 2];
      } else {
        b = u / (p->num_q_heads * L);
        h = (u / L) % p->num_q_heads;
        i = u % L;
      }
      if (!s || !keys || !o) { fail(&status, ERR_NOMEM); continue; }
      if (b < 0 || b >= p->batch || h < 0 || h >= p->num_q_heads || i < 0 || i >= L) {
        fail(&status, ERR_UNIT);
        continue;
      }
      int nk = causal ? i + 1 : N;
      for (int a = 0; a < nk; ++a) keys[a] = a;
      double r = attend(p, q, k, out ? v : NULL, b, h, i, keys, nk, s, o);
      if (out) memcpy(out + (size_t)u * d, o, (size_t)d * sizeof(double));
      if (lse) lse[u] = r;
    }
    free(s);
    free(keys);
    free(o);
  }
  return status;
}

/* ---- thread count --------------------------------------------------------- */

int oracle_threads(int nthreads) {
  int used = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
#pragma omp single
    used = omp_get_num_threads();
  }
  return used;
}
