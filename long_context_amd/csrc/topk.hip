// Exact top-k selection for the anchor layer ("exact Top-k indices", Kascade
// abstract on the opentrain.ai page, "Abstract").
//
// Input: non-negative float32 scores (pooled post-softmax probabilities). For
// non-negative IEEE floats the 32-bit pattern orders like the value and bit 31
// is clear, so the k-th largest score is found by an MSB-first radix select
// over bits 30..0: digit histograms in LDS over bits 30..20 (the exponent and
// three mantissa bits, so that probabilities, which cluster in a few
// octaves, still spread over many bins and the histogram atomics rarely
// collide), then bits 19..10 and 9..0, each pass narrowing to the bucket that
// holds the k-th element. That gives the exact threshold
// pattern and how many keys equal to it are still needed. A final ordered
// pass then writes, in ascending key order, every key above the threshold and
// the lowest-indexed keys equal to it (block-wide ballot scans keep the order),
// then pads with -1. No sort is needed, and the result is deterministic.
//
// One 1024-thread workgroup per segment. Segments of up to 32768 keys are held
// in registers (32 per thread), so the passes only touch the LDS histogram,
// and an LDS copy lets two prefix sums over threads order the output;
// longer ones are re-read from memory each pass. Histogram atomics are
// aggregated per wavefront for the most common digit, since the exponents of
// probabilities cluster.
//
// Decode fuses the pooling: the segment of KV head kv is produced here from
// the group's scaled logits and row log-sum-exps, sum over heads of
// exp2(logit - lse2), straight into registers. Heads are summed in order; a
// thread issues eight 16-byte loads per head and requests the next head's
// before summing the current one, which keeps enough bytes moving per
// compute unit to stream the logits.
//
// One set shared by all heads (the non-head-aware ablation) pools first, in a
// separate pass: decode sums exp2(logit - lse2) over all Hq heads per key;
// prefill sums the per-KV-head pooled rows of a batch row. The selection then
// runs on those rows. Sums rank keys as the means do.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kascade {

namespace {

constexpr int kThreads = 1024;  // decode segments and long prefill segments
constexpr int kSmallThreads = 256;  // prefill segments of at most kRegs * 256 keys
constexpr int kPasses = 3;  // digits: bits 30..20, 19..10, 9..0
constexpr int kMaxBins = 2048;
__device__ __forceinline__ int pass_shift(int pass) { return 20 - 10 * pass; }
__device__ __forceinline__ int pass_bins(int pass) { return pass == 0 ? 2048 : 1024; }

__device__ __forceinline__ void hist_add(unsigned* hist, unsigned digit, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const unsigned d0 = __builtin_amdgcn_readlane(digit, leader);
  const bool same = active && digit == d0;
  const uint64_t same_mask = __ballot(same);
  const int lane = threadIdx.x & 63;
  if (lane == leader) atomicAdd(&hist[d0], (unsigned)__popcll(same_mask));
  if (active && !same) atomicAdd(&hist[digit], 1u);
}

// Exclusive block-wide prefix count of `flag` over thread order (NT threads);
// returns the rank of this thread among flagged threads and the block total.
template <int NT>
__device__ __forceinline__ unsigned block_rank(bool flag, unsigned* wave_tot, unsigned& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t mask = __ballot(flag);
  const unsigned below = (unsigned)__popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = (unsigned)__popcll(mask);
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const unsigned c = wave_tot[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + below;
}

// Exclusive prefix sum of v over thread order (NT threads); `total` gets the sum.
template <int NT>
__device__ __forceinline__ unsigned block_scan(unsigned v, unsigned* wave_tot, unsigned& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const unsigned t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const unsigned c = wave_tot[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// After a histogram pass over `bins` buckets of the digit at `shift`: find the
// bucket holding the krem-th largest candidate, counting from the top bucket
// down, and extend prefix / reduce krem to it. Thread t scans the per = bins/NT
// buckets bins-1-per*t downwards. Every thread returns the same prefix and krem.
template <int NT>
__device__ __forceinline__ void narrow(const unsigned* hist, int bins, int shift, unsigned* wave_tot,
                                       unsigned* sh, unsigned& prefix, unsigned& krem) {
  const int tid = threadIdx.x;
  const int per = bins / NT;
  const int top = bins - 1 - per * tid;
  unsigned local = 0;
  for (int i = 0; i < per; ++i) local += hist[top - i];
  unsigned total;
  const unsigned above = block_scan<NT>(local, wave_tot, total);  // candidates in higher buckets
  if (above < krem && krem <= above + local) {
    unsigned run = above;
    for (int i = 0; i < per; ++i) {
      const unsigned c = hist[top - i];
      if (krem <= run + c) {
        sh[0] = prefix | ((unsigned)(top - i) << shift);
        sh[1] = krem - run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  prefix = sh[0];
  krem = sh[1];
}

// Where a selected position j of a segment goes: the key written to the output
// is remap[j] when a remap table is given, else key_base + j; vals (optional)
// receives the selected scores in the same order.
template <bool REMAP, bool VALS>
struct SelectOut {
  int32_t* idx;
  int key_base;
  const int32_t* remap;
  float* vals;
  __device__ __forceinline__ void put(unsigned pos, int j, unsigned bits) const {
    idx[pos] = REMAP ? remap[j] : key_base + j;
    if (VALS) vals[pos] = __uint_as_float(bits);
  }
};
using PlainOut = SelectOut<false, false>;   // positions are the keys
using CandOut = SelectOut<false, true>;     // keys offset by key_base, scores kept
using RemapOut = SelectOut<true, false>;    // keys looked up from a table

// Selection key of a score: its float bit pattern with the sign bit cleared.
// Pooled scores are sums of probabilities, hence non-negative, and their
// patterns order like their values. Clearing the sign keeps every key below
// 2^31 whatever the inputs were (a NaN of either sign included), which the
// radix passes (bits 30..0) rely on to select exactly k keys.
__device__ __forceinline__ unsigned score_key(float v) { return __float_as_uint(v) & 0x7fffffffu; }
__device__ __forceinline__ unsigned score_key(unsigned bits) { return bits & 0x7fffffffu; }

// Selection over a segment read from memory (any length).
template <int NT, class Out>
__device__ __forceinline__ void select_segment(const unsigned* keys, int n, int kt, int k, Out so) {
  int32_t* out = so.idx;
  __shared__ unsigned hist[kMaxBins];
  __shared__ unsigned wave_tot[NT / 64];
  __shared__ unsigned sh[2];
  const int tid = threadIdx.x;

  if (kt >= n) {  // every candidate is kept
    for (int s = tid; s < k; s += NT) {
      if (s < n) so.put(s, s, score_key(keys[s]));
      else out[s] = -1;
    }
    return;
  }

  unsigned prefix = 0, mask = 0, krem = (unsigned)kt;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int shift = pass_shift(pass), bins = pass_bins(pass);
    const unsigned dmask = (unsigned)bins - 1u;
    for (int i = tid; i < bins; i += NT) hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += NT) {
      const int j = j0 + tid;
      const unsigned u = j < n ? score_key(keys[j]) : 0u;
      const bool match = j < n && (u & mask) == prefix;
      hist_add(hist, (u >> shift) & dmask, match);
    }
    __syncthreads();
    narrow<NT>(hist, bins, shift, wave_tot, sh, prefix, krem);
    mask |= dmask << shift;
  }

  // prefix is the k-th largest pattern; krem keys equal to it are still needed.
  unsigned base = 0, eq_seen = 0;
  for (int j0 = 0; j0 < n; j0 += NT) {
    const int j = j0 + tid;
    const unsigned u = j < n ? score_key(keys[j]) : 0u;
    const bool gt = j < n && u > prefix;
    const bool eq = j < n && u == prefix;
    unsigned eq_total;
    const unsigned eq_rank = eq_seen + block_rank<NT>(eq, wave_tot, eq_total);
    const bool sel = gt || (eq && eq_rank < krem);
    unsigned sel_total;
    const unsigned pos = base + block_rank<NT>(sel, wave_tot, sel_total);
    if (sel && pos < (unsigned)kt) so.put(pos, j, u);  // bound holds by construction; kept as a guard
    base += sel_total;
    eq_seen += eq_total;
  }
  for (int s = kt + tid; s < k; s += NT) out[s] = -1;
}

// Same selection with the segment held in registers, for segments of at most
// kRegs * NT keys. Register i of thread tid holds key key_of<NT>(i, tid): four
// consecutive keys per group of four registers, so loads can be 16 bytes
// wide; the histogram passes do not depend on order. The segment is also
// staged in LDS, one padding word per 32 keys, so that in the final pass
// thread tid reads its contiguous keys 32*tid .. 32*tid+31 without bank
// conflicts and two prefix sums over threads order the output.
constexpr int kRegs = 32;
template <int NT>
constexpr int stage_len() { return kRegs * NT + NT; }  // staged keys plus padding

__device__ __forceinline__ int stage_index(int j) { return j + (j >> 5); }
template <int NT>
__device__ __forceinline__ int key_of(int i, int tid) { return 4 * (NT * (i >> 2) + tid) + (i & 3); }

template <int NT, class Out>
__device__ __forceinline__ void select_registers(const unsigned (&u)[kRegs], const unsigned* staged, int n,
                                                 int kt, int k, Out so) {
  int32_t* out = so.idx;
  __shared__ unsigned hist[kMaxBins];
  __shared__ unsigned wave_tot[NT / 64];
  __shared__ unsigned sh[2];
  const int tid = threadIdx.x;
  if (kt >= n) {
    for (int s = tid; s < k; s += NT) {
      if (s < n) so.put(s, s, staged[stage_index(s)]);
      else out[s] = -1;
    }
    return;
  }
  unsigned prefix = 0, mask = 0, krem = (unsigned)kt;
#pragma unroll
  for (int pass = 0; pass < kPasses; ++pass) {
    const int shift = pass_shift(pass), bins = pass_bins(pass);
    const unsigned dmask = (unsigned)bins - 1u;
    for (int i = tid; i < bins; i += NT) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRegs; ++i)
      hist_add(hist, (u[i] >> shift) & dmask, key_of<NT>(i, tid) < n && (u[i] & mask) == prefix);
    __syncthreads();
    narrow<NT>(hist, bins, shift, wave_tot, sh, prefix, krem);
    mask |= dmask << shift;
  }
  // prefix is the k-th largest pattern; krem keys equal to it are still needed,
  // taken lowest index first.
  const int j0 = kRegs * tid;
  unsigned v[kRegs];
  unsigned gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kRegs; ++i) {
    v[i] = j0 + i < n ? staged[stage_index(j0 + i)] : 0u;
    gt += (j0 + i < n && v[i] > prefix) ? 1u : 0u;
    eq += (j0 + i < n && v[i] == prefix) ? 1u : 0u;
  }
  unsigned total;
  const unsigned eq_before = block_scan<NT>(eq, wave_tot, total);
  const unsigned take = krem > eq_before ? min(krem - eq_before, eq) : 0u;
  unsigned pos = block_scan<NT>(gt + take, wave_tot, total);
  unsigned taken = 0;
#pragma unroll
  for (int i = 0; i < kRegs; ++i) {
    const bool in = j0 + i < n;
    bool sel = in && v[i] > prefix;
    if (in && v[i] == prefix && taken < take) {
      sel = true;
      ++taken;
    }
    if (sel && pos < (unsigned)kt) so.put(pos++, j0 + i, v[i]);  // bound holds by construction
  }
  for (int s = kt + tid; s < k; s += NT) out[s] = -1;
}

// Decode selection in sub-segments of kSub = kRegs * 1024 keys, one workgroup
// each:
// workgroup (seg, sub) pools keys [sub * kSub, ...) of segment seg = (b, KV
// head) into registers and selects their exact top-k. With one sub-segment
// that is the answer; otherwise the selected keys and scores go to the
// candidate arrays (sub-segment sub at offset sub * min(k, kSub), in key
// order) and topk_merge_kernel selects among them. Every key of the
// segment's top-k is among its own sub-segment's top-k (fewer than k keys
// precede it there), so the merge is exact.
constexpr int kDecodeThreads = kThreads;
constexpr int kSub = kRegs * kDecodeThreads;

template <bool WHOLE>
__global__ __launch_bounds__(kDecodeThreads) void topk_decode_kernel(const float* logits, int ld,
                                                                 const float* lse2, int hq,
                                                                 int hkv, int group, int n, int k,
                                                                 int nsub, float* cand_val,
                                                                 int32_t* cand_idx, int32_t* idx) {
  constexpr int NT = kDecodeThreads;
  __shared__ float l2[16];
  const int seg = (int)blockIdx.x / nsub, sub = (int)blockIdx.x % nsub;
  const int b = seg / hkv, kvh = seg % hkv;
  const int tid = threadIdx.x;
  const int base = sub * kSub;
  const int n_sub = min(kSub, n - base);
  if (tid < group) l2[tid] = lse2[b * hq + kvh * group + tid];
  __syncthreads();
  const float* lg = logits + (size_t)(b * hq + kvh * group) * ld;
  // Pooled scores of keys base + key_of(i, tid) into p[i]: the sum over heads
  // (it ranks keys exactly as the mean does), heads in order. Rows are ld
  // floats, a multiple of four, so a 16-byte load that starts below n stays
  // inside its row; keys at or past n get 0.
  __shared__ unsigned staged[stage_len<NT>()];
  float p[kRegs];
#pragma unroll
  for (int i = 0; i < kRegs; ++i) p[i] = 0.f;
  // Two heads' rows in flight: head g + 1 is requested before head g is
  // summed, so each head's load latency hides behind the previous head.
  auto load_head = [&](int g, float4 (&x)[kRegs / 4]) __attribute__((always_inline)) {
    const float* row = lg + (size_t)g * ld + base;
#pragma unroll
    for (int q = 0; q < kRegs / 4; ++q) {
      const int j4 = key_of<NT>(4 * q, tid);
      x[q] = j4 < n_sub ? *reinterpret_cast<const float4*>(row + j4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto add_head = [&](int g, const float4 (&x)[kRegs / 4]) __attribute__((always_inline)) {
    const float m = l2[g];
#pragma unroll
    for (int q = 0; q < kRegs / 4; ++q) {
      p[4 * q + 0] += fast_exp2(x[q].x - m);
      p[4 * q + 1] += fast_exp2(x[q].y - m);
      p[4 * q + 2] += fast_exp2(x[q].z - m);
      p[4 * q + 3] += fast_exp2(x[q].w - m);
    }
  };
  float4 xa[kRegs / 4], xb[kRegs / 4];
  load_head(0, xa);
  for (int g = 0; g < group; g += 2) {
    if (g + 1 < group) load_head(g + 1, xb);
    add_head(g, xa);
    if (g + 1 >= group) break;
    if (g + 2 < group) load_head(g + 2, xa);
    add_head(g + 1, xb);
  }
  unsigned u[kRegs];
#pragma unroll
  for (int i = 0; i < kRegs; ++i) {
    const int j = key_of<NT>(i, tid);
    u[i] = j < n_sub ? score_key(p[i]) : 0u;
    if (j < n_sub) staged[stage_index(j)] = u[i];
  }
  __syncthreads();
  // One sub-segment (WHOLE): the final sets. Several: this sub-segment's candidates.
  if constexpr (WHOLE) {
    select_registers<NT>(u, staged, n_sub, k, k, PlainOut{idx + (size_t)seg * k, 0, nullptr, nullptr});
  } else {
    const size_t off = ((size_t)seg * nsub + sub) * min(k, kSub);
    const int kc = min(k, n_sub);
    select_registers<NT>(u, staged, n_sub, kc, kc, CandOut{cand_idx + off, base, nullptr, cand_val + off});
  }
}

// Final selection of segment seg among its candidates (see topk_decode_kernel):
// m = (nsub - 1) * min(k, kSub) + min(k, keys of the last sub-segment)
// candidates, stored in key order; NT threads (256 while m fits their
// registers, else 1024).
__host__ __device__ inline int merge_candidates(int n, int k, int nsub) {
  const int kmax = k < kSub ? k : kSub, last = n - (nsub - 1) * kSub;
  return (nsub - 1) * kmax + (k < last ? k : last);
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_merge_kernel(const float* cand_val, const int32_t* cand_idx,
                                                        int n, int k, int nsub, int32_t* idx) {
  const int seg = blockIdx.x;
  const int kmax = min(k, kSub);
  const int m = merge_candidates(n, k, nsub);
  const float* vals = cand_val + (size_t)seg * nsub * kmax;
  const int32_t* keys = cand_idx + (size_t)seg * nsub * kmax;
  int32_t* out = idx + (size_t)seg * k;
  if (m <= kRegs * NT) {
    __shared__ unsigned staged[stage_len<NT>()];
    unsigned u[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int j = key_of<NT>(i, threadIdx.x);
      u[i] = j < m ? score_key(vals[j]) : 0u;
      if (j < m) staged[stage_index(j)] = u[i];
    }
    __syncthreads();
    select_registers<NT>(u, staged, m, k, k, RemapOut{out, 0, keys, nullptr});
  } else {
    select_segment<NT>(reinterpret_cast<const unsigned*>(vals), m, k, k, RemapOut{out, 0, keys, nullptr});
  }
}

// Rows of scores in memory longer than one sub-segment: workgroup
// (row, sub) selects the exact top-k of keys [sub * kSub, ...) of its row into
// the candidate arrays, laid out as for topk_decode_kernel.
__global__ __launch_bounds__(kThreads) void topk_rows_sub_kernel(const float* scores, int n, int k, int nsub,
                                                                   float* cand_val, int32_t* cand_idx) {
  constexpr int NT = kThreads;
  const int row = (int)blockIdx.x / nsub, sub = (int)blockIdx.x % nsub;
  const int base = sub * kSub;
  const int n_sub = min(kSub, n - base);
  const float* src = scores + (size_t)row * n + base;
  __shared__ unsigned staged[stage_len<NT>()];
  unsigned u[kRegs];
#pragma unroll
  for (int i = 0; i < kRegs; ++i) {
    const int j = key_of<NT>(i, threadIdx.x);
    u[i] = j < n_sub ? score_key(src[j]) : 0u;
    if (j < n_sub) staged[stage_index(j)] = u[i];
  }
  __syncthreads();
  const size_t off = ((size_t)row * nsub + sub) * min(k, kSub);
  const int kc = min(k, n_sub);
  select_registers<NT>(u, staged, n_sub, kc, kc, CandOut{cand_idx + off, base, nullptr, cand_val + off});
}

// Tiles t0 + blockIdx.x of every (b, KV head); NT threads per segment.
template <int NT>
__global__ __launch_bounds__(NT) void topk_prefill_kernel(const float* pooled, int hkv, int n, int tile,
                                                          int tiles, int t0, size_t ragged, int k,
                                                          int32_t* idx) {
  const int t = t0 + (int)blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int prefix = min((t + 1) * tile, n);
  const size_t base = (size_t)(b * hkv + kvh) * ragged + (size_t)tile * t * (t + 1) / 2;
  int32_t* out = idx + ((size_t)(b * hkv + kvh) * tiles + t) * k;
  const float* src = pooled + base;
  if (prefix <= kRegs * NT) {
    __shared__ unsigned staged[stage_len<NT>()];
    unsigned u[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int j = key_of<NT>(i, threadIdx.x);
      u[i] = j < prefix ? score_key(src[j]) : 0u;
      if (j < prefix) staged[stage_index(j)] = u[i];
    }
    __syncthreads();
    select_registers<NT>(u, staged, prefix, min(k, prefix), k, PlainOut{out, 0, nullptr, nullptr});
  } else {
    select_segment<NT>(reinterpret_cast<const unsigned*>(src), prefix, min(k, prefix), k,
                       PlainOut{out, 0, nullptr, nullptr});
  }
}

// Segments (b, kv, t) of one ragged pooled layout: tiles whose candidates fit
// a small workgroup's registers go to 256-thread workgroups (several per
// compute unit), the longer ones to 1024-thread workgroups.
hipError_t launch_select_tiles(const float* scores, int batch, int hkv, int n, int tile, size_t ragged,
                               int k, int32_t* idx, hipStream_t s) {
  const int tiles = (n + tile - 1) / tile;
  const int small = min(tiles, (kRegs * kSmallThreads) / tile);  // tiles t < small have prefix <= 8192
  if (tiles > small) {
    hipLaunchKernelGGL(topk_prefill_kernel<kThreads>, dim3(tiles - small, hkv, batch), dim3(kThreads), 0, s,
                       scores, hkv, n, tile, tiles, small, ragged, k, idx);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (small > 0) {
    hipLaunchKernelGGL(topk_prefill_kernel<kSmallThreads>, dim3(small, hkv, batch), dim3(kSmallThreads), 0,
                       s, scores, hkv, n, tile, tiles, 0, ragged, k, idx);
  }
  return hipGetLastError();
}

constexpr int kPoolThreads = 256;

// pooled[b][j] = sum over the hq heads of batch row b of exp2(logit - lse2);
// one thread per key, heads walked in order, loads coalesced over keys.
__global__ __launch_bounds__(kPoolThreads) void pool_all_heads_kernel(const float* logits, int ld,
                                                                        const float* lse2, int hq,
                                                                        int n, float* pooled) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * kPoolThreads + threadIdx.x;
  if (j >= n) return;
  const float* lg = logits + (size_t)b * hq * ld + j;
  const float* l2 = lse2 + (size_t)b * hq;
  float acc = 0.f;
  for (int h = 0; h < hq; ++h) acc += fast_exp2(lg[(size_t)h * ld] - l2[h]);
  pooled[(size_t)b * n + j] = acc;
}

// out[b][e] = sum over kv of pooled[(b*hkv + kv)*len + e].
__global__ __launch_bounds__(kPoolThreads) void sum_sets_kernel(const float* pooled, int hkv,
                                                                  size_t len, float* out) {
  const int b = blockIdx.y;
  const float* src = pooled + (size_t)b * hkv * len;
  for (size_t e = (size_t)blockIdx.x * kPoolThreads + threadIdx.x; e < len;
       e += (size_t)gridDim.x * kPoolThreads) {
    float acc = 0.f;
    for (int kv = 0; kv < hkv; ++kv) acc += src[(size_t)kv * len + e];
    out[(size_t)b * len + e] = acc;
  }
}

}  // namespace

static hipError_t launch_topk_merge(const float* cand_val, const int32_t* cand_idx, int segments, int n, int k,
                                    int nsub, int32_t* idx, hipStream_t s) {
  if (merge_candidates(n, k, nsub) <= kRegs * kSmallThreads)
    hipLaunchKernelGGL(topk_merge_kernel<kSmallThreads>, dim3(segments), dim3(kSmallThreads), 0, s, cand_val,
                       cand_idx, n, k, nsub, idx);
  else
    hipLaunchKernelGGL(topk_merge_kernel<kThreads>, dim3(segments), dim3(kThreads), 0, s, cand_val, cand_idx, n,
                       k, nsub, idx);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const float* scores, int rows, int n, int k, float* cand_val, int32_t* cand_idx,
                            int32_t* idx, hipStream_t s) {
  const int nsub = topk_decode_subsegments(n);
  // Up to one sub-segment a row is a single prefill segment whose tile spans
  // all n keys; longer rows go through sub-segment candidates and a merge.
  if (nsub == 1) return launch_select_tiles(scores, rows, 1, n, n, (size_t)n, k, idx, s);
  hipLaunchKernelGGL(topk_rows_sub_kernel, dim3(rows * nsub), dim3(kThreads), 0, s, scores, n, k, nsub, cand_val,
                     cand_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_topk_merge(cand_val, cand_idx, rows, n, k, nsub, idx, s);
}

hipError_t launch_pool_all_heads(const float* logits, int ld, const float* lse2, int batch, int hq,
                                 int n, float* pooled, hipStream_t s) {
  hipLaunchKernelGGL(pool_all_heads_kernel, dim3((n + kPoolThreads - 1) / kPoolThreads, batch),
                     dim3(kPoolThreads), 0, s, logits, ld, lse2, hq, n, pooled);
  return hipGetLastError();
}

hipError_t launch_sum_sets(const float* pooled, int batch, int hkv, size_t len, float* out,
                           hipStream_t s) {
  const size_t want = (len + kPoolThreads - 1) / kPoolThreads;
  const int blocks = (int)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(sum_sets_kernel, dim3(blocks, batch), dim3(kPoolThreads), 0, s, pooled, hkv, len,
                     out);
  return hipGetLastError();
}

int topk_decode_subsegments(int n) { return (n + kSub - 1) / kSub; }


size_t topk_decode_candidates(int n, int k) {
  const int nsub = topk_decode_subsegments(n);
  return nsub > 1 ? (size_t)nsub * (size_t)min(k, kSub) : 0;
}

hipError_t launch_topk_decode(const float* logits, int ld, const float* lse2, int batch, int hq,
                              int hkv, int group, int n, int k, float* cand_val, int32_t* cand_idx,
                              int32_t* idx, hipStream_t s) {
  const int nsub = topk_decode_subsegments(n);
  if (nsub == 1)
    hipLaunchKernelGGL(topk_decode_kernel<true>, dim3(batch * hkv), dim3(kDecodeThreads), 0, s, logits, ld,
                       lse2, hq, hkv, group, n, k, nsub, cand_val, cand_idx, idx);
  else
    hipLaunchKernelGGL(topk_decode_kernel<false>, dim3(batch * hkv * nsub), dim3(kDecodeThreads), 0, s, logits,
                       ld, lse2, hq, hkv, group, n, k, nsub, cand_val, cand_idx, idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nsub == 1) return e;
  return launch_topk_merge(cand_val, cand_idx, batch * hkv, n, k, nsub, idx, s);
}

hipError_t launch_topk_prefill(const float* scores, int batch, int hkv, int n, int tile, int k,
                               int32_t* idx, hipStream_t s) {
  return launch_select_tiles(scores, batch, hkv, n, tile, prefill_ragged_len(n, tile), k, idx, s);
}

}  // namespace kascade
