/*
 * kascade_oracle.h -- plain, slow fp64 CPU oracle for Kascade's cross-layer
 * top-k sparse attention.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists so that the tests, the smoke
 * check and the CPU leg of the benchmark can tell whether the GPU library
 * computes the right thing. It shares no code, header, table or helper with
 * the GPU library, and the GPU library must never call it.
 *
 * What is computed (sources: "Kascade: A Practical Sparse Attention Method for
 * Long-Context LLM Inference"; the arXiv abstract as reproduced on the
 * opentrain.ai review page, section "Abstract"; the euno.news summary,
 * sections "Key Contributions" and "Methodology"):
 *
 *  - Anchor layer: dense attention scores, softmax per query row, then the
 *    exact top-k key indices ("exact Top-k indices in a small set of anchor
 *    layers"). Selection is head-aware. Reading used here: one index set per
 *    KV head, ranking the mean of the post-softmax probabilities of the G
 *    query heads that share the KV head (G = 1 is the pages' "per head" case).
 *    Prefill selects one set per query tile ("tile-level operations"): the
 *    mean is also taken over the tile's rows, and only keys < prefix_t are
 *    candidates, prefix_t = min((t+1)*T, N), k_t = min(k, prefix_t).
 *  - Reuse layer: softmax attention restricted to the saved index set, with
 *    the reuse layer's own Q, K and V (summary, Methodology step 3). Prefill
 *    rows also obey causality: row i uses only saved keys j <= i.
 *  - Non-head-aware variant (shared_index_set = 1), the ablation the pages
 *    compare head-aware selection against (summary, "Key Contributions" and
 *    "Results & Findings"): one index set per batch row (and tile), ranking the mean of
 *    the post-softmax probabilities of all Hq query heads, and every head
 *    reuses that one set. With Hkv = 1 it is the head-aware case.
 *  - Dense: textbook softmax attention (causal for prefill), used for the
 *    k = N identity and for the anchor layer's optional dense output.
 *
 * Parity pins: every function here is checked against something other than
 * itself by the CPU tests (torch scaled_dot_product_attention in float64,
 * brute-force subset enumeration, closed forms and invariants). No function
 * is "parity unpinned".
 *
 * Conventions shared with the GPU library by specification only (no code):
 *   Q, O : [B, Hq, q_len, d] row-major    K, V : [B, Hkv, kv_len, d]
 *   idx  : [B, S, tiles, k] int32, ascending, -1 after the first k_t slots,
 *          S = Hkv (one set per KV head) or 1 (one shared set)
 *   query head h reads KV head h / G, G = Hq / Hkv.
 * Element type: dtype 0 = float32, dtype 1 = bfloat16 stored as uint16 bits.
 * Everything is converted exactly to double and computed in double.
 */
#ifndef KASCADE_ORACLE_H
#define KASCADE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int batch;         /* B */
  int num_q_heads;   /* Hq */
  int num_kv_heads;  /* Hkv, must divide Hq */
  int head_dim;      /* d */
  int q_len;         /* decode: 1; prefill: equal to kv_len */
  int kv_len;        /* N */
  int top_k;         /* k */
  int q_tile;        /* T (prefill); ignored for decode */
  double scale;      /* logit scale, usually 1/sqrt(d) */
  int dtype;         /* 0 = float32, 1 = bfloat16 bits */
  int shared_index_set; /* 0: one index set per KV head; 1: one set shared by all heads */
} oracle_problem;

/* All functions return 0 on success and a negative value on a bad argument.
 * "units" is a flat list of unit coordinates; NULL means every unit in
 * row-major order. nthreads <= 0 means the OpenMP default. */

/* Anchor, decode. Unit = (b, s): 2 ints each, s the index set (the KV head,
 * or 0 for a shared set).
 * idx_out    [nunits][k]   selected key indices, ascending.
 * pooled_out [nunits][N]   mean post-softmax probability over the set's heads (nullable). */
int oracle_anchor_decode(const oracle_problem* p, const void* q, const void* k,
                         const int32_t* units, int nunits,
                         int32_t* idx_out, double* pooled_out, int nthreads);

/* Anchor, causal prefill. Unit = (b, s, t): 3 ints each.
 * idx_out    [nunits][k]   ascending, -1 after k_t entries.
 * pooled_out [nunits][N]   mean over the set's heads and the tile's rows; 0 for j >= prefix_t (nullable). */
int oracle_anchor_prefill(const oracle_problem* p, const void* q, const void* k,
                          const int32_t* units, int nunits,
                          int32_t* idx_out, double* pooled_out, int nthreads);

/* Reuse, decode. Unit = (b, h): 2 ints. idx is [B, S, 1, k], S = Hkv or 1 (shared).
 * out [nunits][d]. */
int oracle_reuse_decode(const oracle_problem* p, const void* q, const void* k, const void* v,
                        const int32_t* idx, const int32_t* units, int nunits,
                        double* out, int nthreads);

/* Reuse, causal prefill. Unit = (b, h, i): 3 ints. idx is [B, S, tiles, k].
 * out [nunits][d]; a row whose restricted set is empty gets zeros. */
int oracle_reuse_prefill(const oracle_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, const int32_t* units, int nunits,
                         double* out, int nthreads);

/* Dense attention. Unit = (b, h, i): 3 ints (i = 0 for decode).
 * causal != 0: row i sees keys j <= i (prefill); otherwise all N keys.
 * out [nunits][d] (nullable), lse [nunits] natural-log sum-exp of the logits (nullable). */
int oracle_dense(const oracle_problem* p, const void* q, const void* k, const void* v,
                 int causal, const int32_t* units, int nunits,
                 double* out, double* lse, int nthreads);

/* Threads an OpenMP parallel region of the oracle runs with when asked for
 * nthreads (0 = the OpenMP default). No arithmetic; for reporting only. */
int oracle_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
