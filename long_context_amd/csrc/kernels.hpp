// Internal launch interface between the C ABI (kascade_api.hip) and the
// kernels. Not installed; the public interface is include/kascade.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kascade {

// ---- decode -----------------------------------------------------------------

// One decode attention pass over a key list, split across wavefronts.
// Dense mode walks keys 0..N-1; gather mode walks idx rows (entries -1 skipped).
struct DecodeArgs {
  const void* q;         // [B, Hq, 1, d]
  const void* k;         // [B, Hkv, N, d]
  const void* v;         // [B, Hkv, N, d] (only read when with_pv)
  const int32_t* idx;    // gather mode: [B, idx_sets, 1, list_len]
  int idx_sets;          // Hkv (a set per KV head) or 1 (one set for all heads)
  int batch, hq, hkv, group, n, list_len, d;
  int keys_per_split, splits;
  float scale_log2;      // logit scale times log2(e)
  float* part_ml;        // [B*Hq*splits][2]: running max (log2 units) and sum
  float* part_o;         // [B*Hq*splits][d]: unnormalised partial output
  float* logits;         // dense mode, optional: [B, Hq, logits_ld] scaled logits, log2 units
  int logits_ld;         // row stride of logits: N rounded up to a multiple of 4
  // Gather with the split merge fused in (bf16): the workgroups of a (b, KV
  // head) each merge their wavefronts in LDS; with more than one workgroup per
  // (b, KV head) they leave partials in part_ml / part_o, laid out
  // [unit][workgroup][head of the group] (x2, xd), and the last to arrive on
  // counters[unit] merges them into out and sets the counter back to 0.
  int* counters;         // [B*Hkv] arrival counters, zero between calls
  void* out;             // [B, Hq, 1, d] bf16
};

// Wavefronts per workgroup of the fused gather; splits are a multiple of it.
constexpr int kGatherWaves = 8;
__host__ __device__ inline size_t gather_merge_lds_bytes(int group, int d) {
  return (size_t)kGatherWaves * group * (d + 2) * sizeof(float);
}
hipError_t launch_decode_gather_merged(const DecodeArgs& a, hipStream_t s);

__host__ __device__ inline int decode_logits_ld(int n) { return (n + 3) & ~3; }

hipError_t launch_decode_attn(const DecodeArgs& a, bool bf16, bool gather, bool with_pv,
                              hipStream_t s);

// Merge split partials into the output rows, the natural-log lse and/or the
// log2-domain lse2 (each optional).
hipError_t launch_decode_combine(const float* part_ml, const float* part_o, int rows, int splits,
                                 int d, bool bf16, void* out, float* lse, float* lse2,
                                 hipStream_t s);

// ---- selection --------------------------------------------------------------

// Exact top-k of non-negative float scores per segment, ascending indices,
// lower index first among equal scores, -1 padding up to k.
// Decode: segment (b, kv) is pooled here from the group's logits [., ld] and
// lse2, in sub-segments of 32768 keys; above one sub-segment the per-sub
// selections go through candidate arrays of topk_decode_candidates(n, k)
// entries per segment (cand_val float, cand_idx int32), then a merge.
int topk_decode_subsegments(int n);
size_t topk_decode_candidates(int n, int k);
hipError_t launch_topk_decode(const float* logits, int ld, const float* lse2, int batch, int hq,
                              int hkv, int group, int n, int k, float* cand_val, int32_t* cand_idx,
                              int32_t* idx, hipStream_t s);
// Rows of n scores each, one selection per row: [rows, n] -> idx [rows, k];
// rows longer than one sub-segment use candidate arrays of
// topk_decode_candidates(n, k) entries per row.
hipError_t launch_topk_rows(const float* scores, int rows, int n, int k, float* cand_val, int32_t* cand_idx,
                            int32_t* idx, hipStream_t s);
// Decode, one set for all heads: pooled[b][j] = sum over the Hq heads of
// exp2(logit - lse2) from the logits [B*Hq, ld] and lse2 [B*Hq].
hipError_t launch_pool_all_heads(const float* logits, int ld, const float* lse2, int batch, int hq,
                                 int n, float* pooled, hipStream_t s);
// Prefill, one set for all heads: out[b][e] = sum over the Hkv ragged rows of
// batch b of pooled[(b*Hkv + kv)*len + e].
hipError_t launch_sum_sets(const float* pooled, int batch, int hkv, size_t len, float* out,
                           hipStream_t s);
// Prefill: segment (b, kv, t) covers prefix_t = min((t+1)*T, N) scores stored
// ragged: base (b*Hkv + kv) * ragged_len + T*t*(t+1)/2.
hipError_t launch_topk_prefill(const float* scores, int batch, int hkv, int n, int tile, int k,
                               int32_t* idx, hipStream_t s);

// Elements of one (b, kv) ragged pooled row: tiles 0..tiles-2 are full and
// hold (t+1)*tile candidates, the last one holds n; tile t starts at
// tile*t*(t+1)/2.
__host__ __device__ inline size_t prefill_ragged_len(int n, int tile) {
  const size_t tiles = (size_t)(n + tile - 1) / tile;
  return (size_t)tile * (tiles - 1) * tiles / 2 + (size_t)n;
}

// ---- prefill ----------------------------------------------------------------

struct PrefillArgs {
  const uint16_t* q;     // [B, Hq, N, d] bf16
  const uint16_t* k;     // [B, Hkv, N, d]
  const uint16_t* v;
  const int32_t* idx;    // reuse: [B, idx_sets, tiles, topk]
  int idx_sets;          // Hkv (a set per KV head) or 1 (one set for all heads)
  int batch, hq, hkv, group, n, d, tile, tiles, topk;
  float scale_log2;
  uint16_t* out;         // [B, Hq, N, d] bf16 (optional in the anchor)
  float* lse2;           // [B, Hq, N] log2-domain log-sum-exp (anchor pass 1 output)
  float* pooled;         // ragged pooled scores (anchor pass 2 output)
};

hipError_t launch_prefill_dense(const PrefillArgs& a, hipStream_t s);   // pass 1: lse2 (+ out)
hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s);    // pass 2: pooled
hipError_t launch_prefill_reuse(const PrefillArgs& a, hipStream_t s);   // reuse attention
// Reuse attention with the gathered rows loaded straight into a ring of LDS
// buffers (d 64 or 128, tile 64 or 128, four wavefronts of 32 rows per
// workgroup: one head at tile 128, two at tile 64, whose group must be even).
bool prefill_reuse_ring_supported(const PrefillArgs& a);
hipError_t launch_prefill_reuse_ring(const PrefillArgs& a, hipStream_t s);
hipError_t launch_lse2_to_lse(const float* lse2, float* lse, size_t count, hipStream_t s);

}  // namespace kascade
