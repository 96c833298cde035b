// C ABI of the library (declared in include/kascade.h): argument validation,
// workspace layout and the kernel sequence of each call. Validation is pure
// host code and runs before anything is enqueued.
#include <math.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "api_internal.hpp"
#include "kascade.h"
#include "kernels.hpp"

namespace {

using namespace kascade;

constexpr size_t kAlign = 256;
#ifndef KASCADE_TARGET_WAVES
#define KASCADE_TARGET_WAVES 2048
#endif
#ifndef KASCADE_TARGET_WAVES_DENSE
#define KASCADE_TARGET_WAVES_DENSE 4096
#endif
// Split-K decode: wavefronts to aim for: about eight per compute unit for the
// gathered lists, sixteen for the anchor's sweep over the whole cache.
constexpr int kTargetWaves = KASCADE_TARGET_WAVES;
constexpr int kTargetWavesDense = KASCADE_TARGET_WAVES_DENSE;
constexpr int kMaxGroup = 16;       // query heads per KV head handled together

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_decode(int op) { return op == KASCADE_OP_ANCHOR_DECODE || op == KASCADE_OP_REUSE_DECODE; }

int validate(const kascade_problem* p, int op) {
  if (!p) return KASCADE_ERR_INVALID;
  if (op < KASCADE_OP_ANCHOR_DECODE || op > KASCADE_OP_REUSE_PREFILL) return KASCADE_ERR_INVALID;
  if (p->batch < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 ||
      p->q_len < 1 || p->kv_len < 1 || p->top_k < 1)
    return KASCADE_ERR_INVALID;
  if (p->num_q_heads % p->num_kv_heads != 0) return KASCADE_ERR_INVALID;
  if (p->dtype != KASCADE_F32 && p->dtype != KASCADE_BF16) return KASCADE_ERR_INVALID;
  if (p->shared_index_set != 0 && p->shared_index_set != 1) return KASCADE_ERR_INVALID;
  // NaN scale, tested on the bit pattern (the library is built assuming no NaN
  // operands, so a floating-point comparison could be folded away).
  uint32_t scale_bits;
  memcpy(&scale_bits, &p->scale, sizeof scale_bits);
  if ((scale_bits & 0x7f800000u) == 0x7f800000u && (scale_bits & 0x007fffffu) != 0u) return KASCADE_ERR_INVALID;
  // Index arithmetic inside the kernels uses 32-bit row numbers.
  if ((long long)p->batch * p->num_q_heads * p->q_len >= (1ll << 31) ||
      (long long)p->batch * p->num_kv_heads * p->kv_len >= (1ll << 31))
    return KASCADE_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128) return KASCADE_ERR_UNSUPPORTED;
  if (p->batch > 65535) return KASCADE_ERR_UNSUPPORTED;  // a grid dimension in places
  if (p->num_q_heads / p->num_kv_heads > kMaxGroup) return KASCADE_ERR_UNSUPPORTED;
  if (is_decode(op)) {
    if (p->q_len != 1) return KASCADE_ERR_INVALID;
    if (p->top_k > p->kv_len) return KASCADE_ERR_INVALID;
  } else {
    if (p->q_len != p->kv_len) return KASCADE_ERR_INVALID;
    if (p->q_tile < 1) return KASCADE_ERR_INVALID;
    if (p->q_tile != 64 && p->q_tile != 128) return KASCADE_ERR_UNSUPPORTED;
    if (p->dtype != KASCADE_BF16) return KASCADE_ERR_UNSUPPORTED;
  }
  return KASCADE_OK;
}

struct DecodeSplit {
  int splits, keys_per_split;
};

#ifndef KASCADE_GATHER_GRAIN
#define KASCADE_GATHER_GRAIN 64
#endif
// Spread a list of `len` keys per (b, KV head) over enough wavefronts to fill
// the chip; each wavefront gets a multiple of `grain` keys.
DecodeSplit decode_split(const kascade_problem* p, int len, bool dense, int grain = 64) {
  const int units = p->batch * p->num_kv_heads;
  const int max_splits = (len + grain - 1) / grain;
  const int target = dense ? kTargetWavesDense : kTargetWaves;
  int splits = (target + units - 1) / units;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  int kps = (len + splits - 1) / splits;
  kps = (kps + grain - 1) / grain * grain;
  return {(len + kps - 1) / kps, kps};
}

struct DecodeWorkspace {
  DecodeSplit split;
  bool merged;  // bf16 reuse: split merge fused into the gather (workgroup partials)
  size_t counters, part_ml, part_o, logits, lse2, pooled, cand_val, cand_idx, total;  // byte offsets
};

// bf16 reuse decode fuses the split merge into the gather: the splits come in
// workgroups of kGatherWaves wavefronts, and the partials are per workgroup.
DecodeSplit gather_split(const kascade_problem* p) {
  DecodeSplit s = decode_split(p, p->top_k, false, KASCADE_GATHER_GRAIN);
  s.splits = (s.splits + kGatherWaves - 1) / kGatherWaves * kGatherWaves;
  return s;
}

// Every decode workspace begins with the reuse gather's arrival counters
// (B*Hkv int32). They must be zero before a reuse call; the reuse call leaves
// them zero, and the anchor call never writes them, so one zero-filled decode
// workspace serves any sequence of decode calls.
size_t counters_bytes(const kascade_problem* p) {
  return align_up((size_t)p->batch * p->num_kv_heads * sizeof(int32_t));
}

DecodeWorkspace decode_workspace(const kascade_problem* p, int op) {
  DecodeWorkspace w{};
  const bool anchor = op == KASCADE_OP_ANCHOR_DECODE;
  w.merged = !anchor && p->dtype == KASCADE_BF16;
  w.split = w.merged ? gather_split(p) : decode_split(p, anchor ? p->kv_len : p->top_k, anchor);
  const size_t rows = (size_t)p->batch * p->num_q_heads;
  // partial slots: per (row, split), or per (row, workgroup) when merged
  const size_t slots = rows * (w.merged ? w.split.splits / kGatherWaves : w.split.splits);
  size_t off = 0;
  w.counters = off;
  off += counters_bytes(p);
  w.part_ml = off;
  off += align_up(slots * 2 * sizeof(float));
  w.part_o = off;
  off += align_up(slots * p->head_dim * sizeof(float));
  if (anchor) {
    w.logits = off;
    off += align_up(rows * decode_logits_ld(p->kv_len) * sizeof(float));
    w.lse2 = off;
    off += align_up(rows * sizeof(float));
    // Selection segments: one per (b, KV head), or one per batch row (shared set,
    // whose pooled row is kept here); long segments need sub-segment candidates.
    const size_t segments = (size_t)p->batch * (p->shared_index_set ? 1 : p->num_kv_heads);
    if (p->shared_index_set) {
      w.pooled = off;
      off += align_up((size_t)p->batch * p->kv_len * sizeof(float));
    }
    const size_t cand = segments * topk_decode_candidates(p->kv_len, p->top_k);
    w.cand_val = off;
    off += align_up(cand * sizeof(float));
    w.cand_idx = off;
    off += align_up(cand * sizeof(int32_t));
  }
  w.total = off;
  return w;
}

struct PrefillWorkspace {
  size_t lse2, pooled, shared, total;
};

PrefillWorkspace prefill_workspace(const kascade_problem* p, int op) {
  PrefillWorkspace w{};
  if (op == KASCADE_OP_ANCHOR_PREFILL) {
    size_t off = 0;
    w.lse2 = off;
    off += align_up((size_t)p->batch * p->num_q_heads * p->kv_len * sizeof(float));
    w.pooled = off;
    off += align_up((size_t)p->batch * p->num_kv_heads * prefill_ragged_len(p->kv_len, p->q_tile) *
                    sizeof(float));
    if (p->shared_index_set) {
      w.shared = off;
      off += align_up((size_t)p->batch * prefill_ragged_len(p->kv_len, p->q_tile) * sizeof(float));
    }
    w.total = off;
  }
  return w;
}

size_t workspace_bytes(const kascade_problem* p, int op) {
  if (validate(p, op) != KASCADE_OK) return 0;
  return is_decode(op) ? decode_workspace(p, op).total : prefill_workspace(p, op).total;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool aligned4(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

int check_workspace(const kascade_problem* p, int op, void* ws, size_t ws_bytes) {
  const size_t need = workspace_bytes(p, op);
  if (need == 0) return KASCADE_OK;
  if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0)
    return KASCADE_ERR_WORKSPACE;
  return KASCADE_OK;
}

float scale_log2(const kascade_problem* p) {
  const float scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
  return scale * 1.4426950408889634f;
}

int status_of(hipError_t e) { return e == hipSuccess ? KASCADE_OK : KASCADE_ERR_HIP; }

// ---- optional per-kernel timing ---------------------------------------------

struct TimedLaunch {
  const char* name;
  hipEvent_t start, stop;
};

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> spare;

  hipEvent_t event() {
    if (!spare.empty()) {
      hipEvent_t e = spare.back();
      spare.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
  }
};

Timing& timing() {
  static Timing t;
  return t;
}

// Run one launch; when timing is on, bracket it with events on its stream.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  Timing& t = timing();
  std::unique_lock<std::mutex> lock(t.mu);
  if (!t.on) {
    lock.unlock();
    return launch();
  }
  hipEvent_t a = t.event(), b = t.event();
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, s);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, s);
  t.pending.push_back({name, a, b});
  return e;
}

#define KASCADE_TRY(name, expr)                                   \
  do {                                                            \
    const hipError_t e_ = timed(name, s, [&] { return (expr); }); \
    if (e_ != hipSuccess) return status_of(e_);                   \
  } while (0)

DecodeArgs decode_args(const kascade_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* idx, const DecodeWorkspace& w, char* ws) {
  DecodeArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.idx = idx;
  a.idx_sets = p->shared_index_set ? 1 : p->num_kv_heads;
  a.batch = p->batch;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.n = p->kv_len;
  a.d = p->head_dim;
  a.keys_per_split = w.split.keys_per_split;
  a.splits = w.split.splits;
  a.scale_log2 = scale_log2(p);
  a.part_ml = reinterpret_cast<float*>(ws + w.part_ml);
  a.part_o = reinterpret_cast<float*>(ws + w.part_o);
  a.counters = reinterpret_cast<int*>(ws + w.counters);
  a.logits = nullptr;
  a.logits_ld = decode_logits_ld(p->kv_len);
  return a;
}

PrefillArgs prefill_args(const kascade_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, void* out) {
  PrefillArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.idx = idx;
  a.idx_sets = p->shared_index_set ? 1 : p->num_kv_heads;
  a.batch = p->batch;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.group = p->num_q_heads / p->num_kv_heads;
  a.n = p->kv_len;
  a.d = p->head_dim;
  a.tile = p->q_tile;
  a.tiles = (p->kv_len + p->q_tile - 1) / p->q_tile;
  a.topk = p->top_k;
  a.scale_log2 = scale_log2(p);
  a.out = static_cast<uint16_t*>(out);
  return a;
}

}  // namespace

namespace kascade {

int reuse_decode_check(const kascade_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* idx, const void* out) {
  const int rc = validate(p, KASCADE_OP_REUSE_DECODE);
  if (rc) return rc;
  if (!q || !k || !v || !idx || !out) return KASCADE_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(idx))
    return KASCADE_ERR_INVALID;
  return KASCADE_OK;
}

int reuse_decode_enqueue(const kascade_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, void* out, char* ws, hipStream_t s) {
  const DecodeWorkspace w = decode_workspace(p, KASCADE_OP_REUSE_DECODE);
  DecodeArgs a = decode_args(p, q, k, v, idx, w, ws);
  a.list_len = p->top_k;
  a.out = out;
  if (w.merged) {
    KASCADE_TRY("decode_attn_gather", launch_decode_gather_merged(a, s));
    return KASCADE_OK;
  }
  KASCADE_TRY("decode_attn_gather", launch_decode_attn(a, false, true, true, s));
  KASCADE_TRY("decode_combine", launch_decode_combine(a.part_ml, a.part_o, p->batch * a.hq,
                                                      a.splits, a.d, false, out, nullptr, nullptr, s));
  return KASCADE_OK;
}

}  // namespace kascade

extern "C" {

int kascade_validate(const kascade_problem* p, int op) { return validate(p, op); }

size_t kascade_workspace_bytes(const kascade_problem* p, int op) { return workspace_bytes(p, op); }

const char* kascade_status_string(int status) {
  switch (status) {
    case KASCADE_OK: return "ok";
    case KASCADE_ERR_INVALID: return "invalid argument";
    case KASCADE_ERR_UNSUPPORTED: return "unsupported problem";
    case KASCADE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case KASCADE_ERR_HIP: return "HIP launch or runtime error";
    case KASCADE_ERR_SCRATCH: return "problem exceeds the allocation-free entry point's scratch";
    default: return "unknown status";
  }
}

int kascade_anchor_decode(const kascade_problem* p, const void* q, const void* k, const void* v,
                          void* out, int32_t* idx, float* lse, void* workspace,
                          size_t workspace_bytes, void* stream) {
  int rc = validate(p, KASCADE_OP_ANCHOR_DECODE);
  if (rc) return rc;
  // idx NULL: dense attention only (out and/or lse), no scores kept, no selection.
  if (!q || !k || (out && !v) || (!idx && !out && !lse)) return KASCADE_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || (out && !aligned16(out)) ||
      (idx && !aligned4(idx)) || (lse && !aligned4(lse)))
    return KASCADE_ERR_INVALID;
  rc = check_workspace(p, KASCADE_OP_ANCHOR_DECODE, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const DecodeWorkspace w = decode_workspace(p, KASCADE_OP_ANCHOR_DECODE);
  char* ws = static_cast<char*>(workspace);
  DecodeArgs a = decode_args(p, q, k, v, nullptr, w, ws);
  a.list_len = p->kv_len;
  const bool bf16 = p->dtype == KASCADE_BF16;
  if (!idx) {
    KASCADE_TRY("decode_attn_dense_only", launch_decode_attn(a, bf16, false, out != nullptr, s));
    KASCADE_TRY("decode_combine", launch_decode_combine(a.part_ml, a.part_o, p->batch * a.hq, a.splits,
                                                        a.d, bf16, out, lse, nullptr, s));
    return KASCADE_OK;
  }
  a.logits = reinterpret_cast<float*>(ws + w.logits);
  float* pooled = reinterpret_cast<float*>(ws + w.pooled);
  float* lse2 = reinterpret_cast<float*>(ws + w.lse2);
  KASCADE_TRY("decode_attn_dense", launch_decode_attn(a, bf16, false, out != nullptr, s));
  KASCADE_TRY("decode_combine", launch_decode_combine(a.part_ml, a.part_o, p->batch * a.hq,
                                                      a.splits, a.d, bf16, out, lse, lse2, s));
  if (p->shared_index_set) {
    KASCADE_TRY("pool_all_heads", launch_pool_all_heads(a.logits, a.logits_ld, lse2, p->batch, a.hq,
                                                        a.n, pooled, s));
    KASCADE_TRY("topk_rows", launch_topk_rows(pooled, p->batch, a.n, p->top_k,
                                              reinterpret_cast<float*>(ws + w.cand_val),
                                              reinterpret_cast<int32_t*>(ws + w.cand_idx), idx, s));
  } else {
    KASCADE_TRY("topk_decode", launch_topk_decode(a.logits, a.logits_ld, lse2, p->batch, a.hq, a.hkv,
                                                  a.group, a.n, p->top_k,
                                                  reinterpret_cast<float*>(ws + w.cand_val),
                                                  reinterpret_cast<int32_t*>(ws + w.cand_idx), idx, s));
  }
  return KASCADE_OK;
}

int kascade_reuse_decode(const kascade_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, void* out, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int rc = kascade::reuse_decode_check(p, q, k, v, idx, out);
  if (rc) return rc;
  rc = check_workspace(p, KASCADE_OP_REUSE_DECODE, workspace, workspace_bytes);
  if (rc) return rc;
  return kascade::reuse_decode_enqueue(p, q, k, v, idx, out, static_cast<char*>(workspace),
                                       static_cast<hipStream_t>(stream));
}

int kascade_anchor_prefill(const kascade_problem* p, const void* q, const void* k, const void* v,
                           void* out, int32_t* idx, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc = validate(p, KASCADE_OP_ANCHOR_PREFILL);
  if (rc) return rc;
  // idx NULL: dense causal attention only (out and/or lse), no pooled scores, no selection.
  if (!q || !k || (out && !v) || (!idx && !out && !lse)) return KASCADE_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || (v && !aligned16(v)) || (out && !aligned16(out)) ||
      (idx && !aligned4(idx)) || (lse && !aligned4(lse)))
    return KASCADE_ERR_INVALID;
  rc = check_workspace(p, KASCADE_OP_ANCHOR_PREFILL, workspace, workspace_bytes);
  if (rc) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const PrefillWorkspace w = prefill_workspace(p, KASCADE_OP_ANCHOR_PREFILL);
  char* ws = static_cast<char*>(workspace);
  // Without a dense output only K is read; V is never touched.
  PrefillArgs a = prefill_args(p, q, k, out ? v : k, nullptr, out);
  a.lse2 = reinterpret_cast<float*>(ws + w.lse2);
  a.pooled = reinterpret_cast<float*>(ws + w.pooled);
  KASCADE_TRY(idx ? "prefill_dense" : "prefill_dense_only", launch_prefill_dense(a, s));
  if (idx) {
    KASCADE_TRY("prefill_pool", launch_prefill_pool(a, s));
    if (p->shared_index_set) {
      float* shared = reinterpret_cast<float*>(ws + w.shared);
      KASCADE_TRY("sum_sets", launch_sum_sets(a.pooled, p->batch, a.hkv,
                                              prefill_ragged_len(a.n, a.tile), shared, s));
      KASCADE_TRY("topk_prefill", launch_topk_prefill(shared, p->batch, 1, a.n, a.tile, p->top_k, idx, s));
    } else {
      KASCADE_TRY("topk_prefill", launch_topk_prefill(a.pooled, p->batch, a.hkv, a.n, a.tile, p->top_k,
                                                      idx, s));
    }
  }
  if (lse)
    KASCADE_TRY("lse_convert", launch_lse2_to_lse(a.lse2, lse, (size_t)p->batch * a.hq * a.n, s));
  return KASCADE_OK;
}

int kascade_reuse_prefill(const kascade_problem* p, const void* q, const void* k, const void* v,
                          const int32_t* idx, void* out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int rc = validate(p, KASCADE_OP_REUSE_PREFILL);
  if (rc) return rc;
  if (!q || !k || !v || !idx || !out) return KASCADE_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(idx))
    return KASCADE_ERR_INVALID;
  rc = check_workspace(p, KASCADE_OP_REUSE_PREFILL, workspace, workspace_bytes);
  if (rc) return rc;
  PrefillArgs a = prefill_args(p, q, k, v, idx, out);
  hipStream_t s = static_cast<hipStream_t>(stream);
  KASCADE_TRY("prefill_gather", launch_prefill_reuse(a, s));
  return KASCADE_OK;
}

int kascade_timing_enable(int on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  const int prev = t.on ? 1 : 0;
  t.on = on != 0;
  return prev;
}

int kascade_timing_collect(kascade_kernel_time* out, int max_entries) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lock(t.mu);
  int n = 0, rc = 0;
  for (const TimedLaunch& l : t.pending) {
    float ms = 0.f;
    if (hipEventSynchronize(l.stop) != hipSuccess || hipEventElapsedTime(&ms, l.start, l.stop) != hipSuccess) {
      rc = -1;
    } else {
      int i = 0;
      while (i < n && strncmp(out[i].name, l.name, sizeof out[i].name) != 0) ++i;
      if (i == n && n < max_entries) {
        memset(&out[n], 0, sizeof out[n]);
        strncpy(out[n].name, l.name, sizeof out[n].name - 1);
        ++n;
      }
      if (i < n) {
        out[i].total_ms += ms;
        out[i].launches += 1;
      }
    }
    t.spare.push_back(l.start);
    t.spare.push_back(l.stop);
  }
  t.pending.clear();
  return rc ? rc : n;
}

}  // extern "C"
