/*
 * kascade.h -- C ABI of the MI355X (gfx950) library for Kascade's cross-layer
 * top-k sparse attention hot path.
 *
 * Method (Kascade: A Practical Sparse Attention Method for Long-Context LLM
 * Inference, arXiv 2512.16391; arXiv abstract as shown on the opentrain.ai
 * review page, section "Abstract"; euno.news summary, sections "Key
 * Contributions" and "Methodology" steps 2, 3, 5 and 6):
 *   - an ANCHOR layer computes dense attention scores and reduces them to the
 *     exact top-k key indices, head-aware, once per decode query or once per
 *     prefill query tile;
 *   - the following REUSE layers attend only to the keys at those saved
 *     indices, with their own Q, K and V and a softmax restricted to the set.
 *
 * Readings of the pages used throughout:
 *   - Head-aware selection under grouped-query attention: one index set per
 *     KV head. Query head h reads KV head h / G (G = Hq / Hkv); the ranking
 *     score of key j is the mean over the G heads of the group (and, in
 *     prefill, over the rows of the query tile) of the post-softmax attention
 *     probability of j. With G = 1 this is the pages' per-head selection.
 *   - Prefill tile t covers query rows [t*T, min((t+1)*T, N)); its candidate
 *     keys are j < prefix_t = min((t+1)*T, N); it keeps k_t = min(k, prefix_t)
 *     keys. Causal rows see keys j <= i, the diagonal included.
 *   - Exactly equal scores are ranked lower key index first.
 *   - The saved set is used as is: no extra window, sink or diagonal keys.
 *   - Non-head-aware variant (shared_index_set = 1), the ablation baseline the
 *     pages compare head-aware selection against (euno.news summary, "Key
 *     Contributions" and "Results & Findings"): the ranking score is the mean
 *     over ALL Hq query heads (each against its own KV head) of the
 *     post-softmax probabilities, one set per batch row (and prefill tile),
 *     and every head's reuse attends through that one set. With Hkv = 1 it is
 *     the head-aware selection.
 *
 * Layouts (all row-major, contiguous, caller-owned device memory):
 *   Q, O : [B, Hq,  q_len,  d]    (decode: q_len = 1)
 *   K, V : [B, Hkv, kv_len, d]    (prefill: q_len == kv_len == N)
 *   idx  : int32 [B, S, tiles, k]; S = Hkv, or 1 with shared_index_set;
 *          tiles = 1 for decode, ceil(N/T) for prefill. Entries [0, k_t) are
 *          the selected key positions in ascending order; entries [k_t, k)
 *          are -1.
 *   lse  : float32 [B, Hq, q_len], natural-log sum of exp of the scaled logits
 *          over the keys the row attends to in the anchor (dense) pass.
 * Element type: dtype KASCADE_F32 (float32) or KASCADE_BF16 (bfloat16) for Q,
 * K, V and O. Accumulation is float32; bfloat16 outputs are rounded to nearest
 * even.
 *
 * Ownership and execution: every pointer is a device pointer owned by the
 * caller. The library allocates nothing; scratch memory is the caller's
 * workspace, sized by kascade_workspace_bytes(). A decode workspace (either
 * decode op) begins with arrival counters that must be zero before its first
 * use: zero-fill it once when it is allocated. Decode calls leave the counters
 * zero again, so the same workspace serves any sequence of decode calls
 * (including replays of a captured graph); do not hand a decode workspace to
 * a prefill call in between. Calls enqueue kernels on the
 * given HIP stream (a hipStream_t passed as void*, NULL = the null stream) and
 * return without synchronising. Outputs are valid once the stream reaches
 * them. The idx buffer written by an anchor call is read by later reuse calls;
 * the caller keeps it alive. Calls are reentrant; two calls must not share a
 * workspace concurrently.
 *
 * Errors: each call returns a kascade_status. Argument errors are reported
 * before anything is enqueued. Device faults surface at the caller's next
 * synchronisation. Nothing is thrown across the ABI.
 *
 * Values: Q, K and V are expected to be finite. With NaN or infinite inputs
 * the scores and outputs are undefined, but every index set an anchor call
 * writes is still well formed (exactly min(k, candidates) distinct keys in
 * range, ascending, then -1), so reuse calls stay in bounds.
 */
#ifndef KASCADE_H
#define KASCADE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KASCADE_OK = 0,
  KASCADE_ERR_INVALID = 1,     /* inconsistent shape or argument, null or misaligned pointer */
  KASCADE_ERR_UNSUPPORTED = 2, /* well-formed but not provided (head_dim, dtype, tile size) */
  KASCADE_ERR_WORKSPACE = 3,   /* workspace null or smaller than kascade_workspace_bytes() */
  KASCADE_ERR_HIP = 4,         /* a HIP launch or runtime call failed */
  KASCADE_ERR_SCRATCH = 5      /* kascade_reuse_decode_noalloc: the problem needs more scratch
                                  than the library's array holds (KASCADE_NOALLOC_SCRATCH_BYTES) */
} kascade_status;

typedef enum { KASCADE_F32 = 0, KASCADE_BF16 = 1 } kascade_dtype;

typedef enum {
  KASCADE_OP_ANCHOR_DECODE = 0,
  KASCADE_OP_REUSE_DECODE = 1,
  KASCADE_OP_ANCHOR_PREFILL = 2,
  KASCADE_OP_REUSE_PREFILL = 3
} kascade_op;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t num_q_heads;  /* Hq, a multiple of Hkv */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* d: 64 or 128 */
  int32_t q_len;        /* decode: 1; prefill: equal to kv_len */
  int32_t kv_len;       /* N >= 1 */
  int32_t top_k;        /* k >= 1; decode requires k <= N */
  int32_t q_tile;       /* T (prefill only): 64 or 128 */
  float scale;          /* logit scale; <= 0 selects 1/sqrt(d) */
  int32_t dtype;        /* kascade_dtype; prefill requires KASCADE_BF16 */
  int32_t shared_index_set; /* 0: one index set per KV head (head-aware, the
                               method); 1: one set per batch row (and tile)
                               shared by every head, the non-head-aware
                               ablation. Any other value is invalid. */
} kascade_problem;

/* Check a problem for an op without touching the GPU. Returns KASCADE_OK,
 * KASCADE_ERR_INVALID or KASCADE_ERR_UNSUPPORTED. Supported: decode with
 * float32 or bfloat16 and d in {64, 128}; prefill with bfloat16, d in
 * {64, 128} and T in {64, 128}. */
int kascade_validate(const kascade_problem* p, int op);

/* Bytes of device workspace the op needs for this problem (0 for an invalid
 * problem). The workspace must be 256-byte aligned; decode workspaces must be
 * zero-filled once when allocated (see above). */
size_t kascade_workspace_bytes(const kascade_problem* p, int op);

/* Anchor layer, one decode query per (batch, query head).
 * Defined by: the anchor layer's dense attention pass, post-softmax scores
 * reduced to exact top-k indices per head (Kascade abstract, opentrain.ai
 * page, "Abstract"; euno.news summary, "Methodology" steps 2 and 5).
 * Computes dense scores of q against all N keys, the per-KV-head pooled
 * post-softmax score, and its exact top-k into idx [B, S, 1, k].
 * out (nullable): dense attention output [B, Hq, 1, d] (reads V; v may be
 * NULL when out is NULL). lse (nullable): [B, Hq, 1].
 * idx (nullable): when NULL the call is plain dense attention -- no scores
 * are kept and nothing is selected -- for layers that attend densely without
 * refreshing an index set; out or lse must then be given.
 * Workspace: kascade_workspace_bytes(p, KASCADE_OP_ANCHOR_DECODE). */
int kascade_anchor_decode(const kascade_problem* p, const void* q, const void* k,
                          const void* v, void* out, int32_t* idx, float* lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Reuse layer, decode. Defined by: a reuse layer attends only to the keys
 * saved by the preceding anchor, softmax restricted to that set, with its own
 * Q, K and V (euno.news summary, "Methodology" step 3; Kascade abstract,
 * opentrain.ai page, "Abstract").
 * For each (b, h): softmax attention of q over the keys idx[b, h/G, 0, :]
 * (idx[b, 0, 0, :] with a shared set) with this layer's K and V, written to
 * out [B, Hq, 1, d].
 * Entries -1 (and any entry outside [0, N)) are skipped; a row whose list has
 * no usable entry gets zeros. */
int kascade_reuse_decode(const kascade_problem* p, const void* q, const void* k,
                         const void* v, const int32_t* idx, void* out,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Reuse layer, decode, allocating nothing: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Same computation, arguments and results as
 * kascade_reuse_decode, without the workspace: the scratch is a device array
 * inside the library of KASCADE_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * kept until the process ends. The first call on a GPU looks up that array's
 * address and clears it with a kernel on `stream`; make that first call
 * outside graph capture if the lookup must not happen during capture.
 * Returns KASCADE_ERR_SCRATCH, before anything is enqueued, for a problem
 * whose kascade_workspace_bytes(p, KASCADE_OP_REUSE_DECODE) exceeds the
 * array. Every call on a GPU shares that GPU's array: calls that may overlap
 * on one GPU (other streams, other host threads) race and must be serialised
 * by the caller. */
#define KASCADE_NOALLOC_SCRATCH_BYTES (8u << 20)
int kascade_reuse_decode_noalloc(const kascade_problem* p, const void* q, const void* k,
                                 const void* v, const int32_t* idx, void* out, void* stream);

/* Anchor layer, causal prefill. Defined by: exact top-k selection in the
 * anchor layer, done per query tile in prefill (Kascade abstract, opentrain.ai
 * page, "Abstract": tile-level operations; euno.news summary, "Methodology"
 * steps 2, 5 and 6).
 * For each (b, KV head, query tile t): the mean
 * over the tile's rows and the group's heads of the causal post-softmax
 * probabilities (all heads' with a shared set), and its exact top-k_t among
 * keys < prefix_t into idx [B, S, ceil(N/T), k]. out (nullable): dense causal attention output
 * [B, Hq, N, d]. lse (nullable): [B, Hq, N].
 * idx (nullable): when NULL the call is plain dense causal attention (no
 * pooled scores, no selection); out or lse must then be given.
 * Workspace: kascade_workspace_bytes(p, KASCADE_OP_ANCHOR_PREFILL). */
int kascade_anchor_prefill(const kascade_problem* p, const void* q, const void* k,
                           const void* v, void* out, int32_t* idx, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Reuse layer, causal prefill. Defined by: each query tile of a reuse layer
 * attends only to its tile's saved index set, causally, with the layer's own
 * Q, K and V (euno.news summary, "Methodology" steps 3 and 6; Kascade
 * abstract, opentrain.ai page, "Abstract").
 * Row i of tile t attends to the keys
 * j in idx[b, h/G, t, 0:k_t] (set 0 when shared) with 0 <= j <= i (entries -1, or outside the
 * sequence, are skipped); a row with no such key gets zeros. Output
 * out [B, Hq, N, d]. Slots at or past k_t = min(k, prefix_t) are not read. */
int kascade_reuse_prefill(const kascade_problem* p, const void* q, const void* k,
                          const void* v, const int32_t* idx, void* out,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Static text for a status code. */
const char* kascade_status_string(int status);

/* ---- optional per-kernel timing (tracing) ----------------------------------
 * While enabled, every kernel the library enqueues is bracketed by a pair of
 * HIP events recorded on the call's stream. kascade_timing_collect() waits
 * for the recorded events, adds their elapsed times per kernel name into
 * out[0..max_entries) and clears the record. Timing is process-wide and off
 * by default; the events are created by the library on first use and reused.
 * kascade_timing_enable returns the previous setting. kascade_timing_collect
 * returns the number of entries written, or -1 on a HIP error. */
typedef struct {
  char name[40];       /* kernel name, NUL-terminated */
  double total_ms;     /* summed duration of its launches */
  int64_t launches;    /* number of launches summed */
} kascade_kernel_time;

int kascade_timing_enable(int on);
int kascade_timing_collect(kascade_kernel_time* out, int max_entries);

#ifdef __cplusplus
}
#endif
#endif /* KASCADE_H */
