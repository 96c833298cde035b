// Exact top-k selection for the anchor layer ("exact Top-k indices", Kascade
// abstract on the opentrain.ai page, "Abstract").
//
// Input: non-negative float32 scores (pooled post-softmax probabilities). For
// non-negative IEEE floats the 32-bit pattern orders like the value and bit 31
// is clear, so the k-th largest score is found by an MSB-first radix select
// over bits 30..0: digit histograms in LDS over the exponent (bits 30..23),
// then bits 22..15, 14..7 and 6..0, each pass narrowing to the bucket that
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
// exp2(logit - lse2), straight into registers.
//
// One set shared by all heads (the non-head-aware ablation) pools first, in a
// separate pass: decode sums exp2(logit - lse2) over all Hq heads per key;
// prefill sums the per-KV-head pooled rows of a batch row. The selection then
// runs on those rows. Sums rank keys as the means do.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kascade {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kShift[4] = {23, 15, 7, 0};
constexpr unsigned kDigitMask[4] = {0xffu, 0xffu, 0xffu, 0x7fu};

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

// Exclusive block-wide prefix count of `flag` over thread order; returns the
// rank of this thread among flagged threads and the block total.
__device__ __forceinline__ unsigned block_rank(bool flag, unsigned* wave_tot, unsigned& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t mask = __ballot(flag);
  const unsigned below = (unsigned)__popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[wave] = (unsigned)__popcll(mask);
  __syncthreads();
  unsigned before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const unsigned c = wave_tot[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + below;
}

__device__ void select_segment(const unsigned* keys, int n, int kt, int k, int32_t* out) {
  __shared__ unsigned hist[256];
  __shared__ unsigned wave_tot[kWaves];
  __shared__ unsigned sh_prefix, sh_krem;
  const int tid = threadIdx.x;

  if (kt >= n) {  // every candidate is kept
    for (int s = tid; s < k; s += kThreads) out[s] = s < n ? s : -1;
    return;
  }

  unsigned prefix = 0, mask = 0, krem = (unsigned)kt;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = kShift[pass];
    const unsigned dmask = kDigitMask[pass];
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += kThreads) {
      const int j = j0 + tid;
      const unsigned u = j < n ? keys[j] : 0u;
      const bool match = j < n && (u & mask) == prefix;
      hist_add(hist, (u >> shift) & dmask, match);
    }
    __syncthreads();
    if (tid < 64) {
      // Lane L covers buckets 255-4L .. 252-4L, i.e. lanes walk from the top.
      unsigned c[4], local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * tid - i];
        local += c[i];
      }
      unsigned incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(incl, o);
        if (tid >= o) incl += t;
      }
      const unsigned excl = incl - local;
      if (excl < krem && krem <= incl) {
        unsigned run = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run + c[i] >= krem) {
            sh_prefix = prefix | ((unsigned)(255 - 4 * tid - i) << shift);
            sh_krem = krem - run;
            break;
          }
          run += c[i];
        }
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    krem = sh_krem;
    mask |= dmask << shift;
    __syncthreads();
  }

  // prefix is the k-th largest pattern; krem keys equal to it are still needed.
  unsigned base = 0, eq_seen = 0;
  for (int j0 = 0; j0 < n; j0 += kThreads) {
    const int j = j0 + tid;
    const unsigned u = j < n ? keys[j] : 0u;
    const bool gt = j < n && u > prefix;
    const bool eq = j < n && u == prefix;
    unsigned eq_total;
    const unsigned eq_rank = eq_seen + block_rank(eq, wave_tot, eq_total);
    const bool sel = gt || (eq && eq_rank < krem);
    unsigned sel_total;
    const unsigned pos = base + block_rank(sel, wave_tot, sel_total);
    if (sel && pos < (unsigned)kt) out[pos] = j;  // bound holds by construction; kept as a guard
    base += sel_total;
    eq_seen += eq_total;
  }
  for (int s = kt + tid; s < k; s += kThreads) out[s] = -1;
}

// Exclusive prefix sum of v over thread order (1024 threads); `total` gets the sum.
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
  for (int w = 0; w < kWaves; ++w) {
    const unsigned c = wave_tot[w];
    before += w < wave ? c : 0u;
    all += c;
  }
  __syncthreads();
  total = all;
  return before + incl - v;
}

// Same selection with the segment held in registers, for segments of at most
// 32768 keys. Thread tid holds keys tid + 1024*i (coalesced loads) for the
// histogram passes, whose counts do not depend on order. The segment is also
// staged in LDS, one padding word per 32 keys, so that in the final pass
// thread tid reads its contiguous keys 32*tid .. 32*tid+31 without bank
// conflicts and two prefix sums over threads order the output.
constexpr int kRegs = 32;
constexpr int kStage = kRegs * kThreads + kThreads;  // staged keys plus padding

__device__ __forceinline__ int stage_index(int j) { return j + (j >> 5); }

__device__ void select_registers(const unsigned (&u)[kRegs], const unsigned* staged, int n, int kt,
                                 int k, int32_t* out) {
  __shared__ unsigned hist[256];
  __shared__ unsigned wave_tot[kWaves];
  __shared__ unsigned sh_prefix, sh_krem;
  const int tid = threadIdx.x;
  if (kt >= n) {
    for (int s = tid; s < k; s += kThreads) out[s] = s < n ? s : -1;
    return;
  }
  unsigned prefix = 0, mask = 0, krem = (unsigned)kt;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = kShift[pass];
    const unsigned dmask = kDigitMask[pass];
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRegs; ++i)
      hist_add(hist, (u[i] >> shift) & dmask, i * kThreads + tid < n && (u[i] & mask) == prefix);
    __syncthreads();
    if (tid < 64) {
      unsigned c[4], local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * tid - i];
        local += c[i];
      }
      unsigned incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned t = __shfl_up(incl, o);
        if (tid >= o) incl += t;
      }
      const unsigned excl = incl - local;
      if (excl < krem && krem <= incl) {
        unsigned run = excl;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (run + c[i] >= krem) {
            sh_prefix = prefix | ((unsigned)(255 - 4 * tid - i) << shift);
            sh_krem = krem - run;
            break;
          }
          run += c[i];
        }
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    krem = sh_krem;
    mask |= dmask << shift;
    __syncthreads();
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
  const unsigned eq_before = block_scan(eq, wave_tot, total);
  const unsigned take = krem > eq_before ? min(krem - eq_before, eq) : 0u;
  unsigned pos = block_scan(gt + take, wave_tot, total);
  unsigned taken = 0;
#pragma unroll
  for (int i = 0; i < kRegs; ++i) {
    const bool in = j0 + i < n;
    bool sel = in && v[i] > prefix;
    if (in && v[i] == prefix && taken < take) {
      sel = true;
      ++taken;
    }
    if (sel && pos < (unsigned)kt) out[pos++] = j0 + i;  // bound holds by construction
  }
  for (int s = kt + tid; s < k; s += kThreads) out[s] = -1;
}

__global__ __launch_bounds__(kThreads) void topk_decode_kernel(const float* logits, int ld,
                                                                 const float* lse2, int hq,
                                                                 int hkv, int group, int n, int k,
                                                                 float* spill, int32_t* idx) {
  __shared__ float l2[16];
  const int seg = blockIdx.x, b = seg / hkv, kvh = seg % hkv;
  const int tid = threadIdx.x;
  if (tid < group) l2[tid] = lse2[b * hq + kvh * group + tid];
  __syncthreads();
  const float* lg = logits + (size_t)(b * hq + kvh * group) * ld;
  auto pooled_at = [&](int j) __attribute__((always_inline)) {
    float acc = 0.f;
    for (int g = 0; g < group; ++g) acc += fast_exp2(lg[(size_t)g * ld + j] - l2[g]);
    return acc;  // the sum over heads ranks keys exactly as the mean does
  };
  if (n <= kRegs * kThreads) {
    __shared__ unsigned staged[kStage];
    unsigned u[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int j = i * kThreads + tid;
      u[i] = j < n ? __float_as_uint(pooled_at(j)) : 0u;
      if (j < n) staged[stage_index(j)] = u[i];
    }
    __syncthreads();
    select_registers(u, staged, n, k, k, idx + (size_t)seg * k);
  } else {
    float* dst = spill + (size_t)seg * n;
    for (int j = tid; j < n; j += kThreads) dst[j] = pooled_at(j);
    __threadfence_block();
    __syncthreads();
    select_segment(reinterpret_cast<const unsigned*>(dst), n, k, k, idx + (size_t)seg * k);
  }
}

__global__ __launch_bounds__(kThreads) void topk_prefill_kernel(const float* pooled, int hkv,
                                                                  int n, int tile, int tiles,
                                                                  size_t ragged, int k,
                                                                  int32_t* idx) {
  const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int prefix = min((t + 1) * tile, n);
  const size_t base = (size_t)(b * hkv + kvh) * ragged + (size_t)tile * t * (t + 1) / 2;
  int32_t* out = idx + ((size_t)(b * hkv + kvh) * tiles + t) * k;
  const float* src = pooled + base;
  if (prefix <= kRegs * kThreads) {
    __shared__ unsigned staged[kStage];
    unsigned u[kRegs];
#pragma unroll
    for (int i = 0; i < kRegs; ++i) {
      const int j = i * kThreads + threadIdx.x;
      u[i] = j < prefix ? __float_as_uint(src[j]) : 0u;
      if (j < prefix) staged[stage_index(j)] = u[i];
    }
    __syncthreads();
    select_registers(u, staged, prefix, min(k, prefix), k, out);
  } else {
    select_segment(reinterpret_cast<const unsigned*>(src), prefix, min(k, prefix), k, out);
  }
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

hipError_t launch_topk_rows(const float* scores, int rows, int n, int k, int32_t* idx,
                            hipStream_t s) {
  // A row is a single prefill segment whose tile spans all n keys.
  hipLaunchKernelGGL(topk_prefill_kernel, dim3(1, 1, rows), dim3(kThreads), 0, s, scores, 1, n, n, 1,
                     (size_t)n, k, idx);
  return hipGetLastError();
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

hipError_t launch_topk_decode(const float* logits, int ld, const float* lse2, int batch, int hq,
                              int hkv, int group, int n, int k, float* spill, int32_t* idx,
                              hipStream_t s) {
  hipLaunchKernelGGL(topk_decode_kernel, dim3(batch * hkv), dim3(kThreads), 0, s, logits, ld, lse2,
                     hq, hkv, group, n, k, spill, idx);
  return hipGetLastError();
}

hipError_t launch_topk_prefill(const float* scores, int batch, int hkv, int n, int tile, int k,
                               int32_t* idx, hipStream_t s) {
  const int tiles = (n + tile - 1) / tile;
  hipLaunchKernelGGL(topk_prefill_kernel, dim3(tiles, hkv, batch), dim3(kThreads), 0, s, scores,
                     hkv, n, tile, tiles, prefill_ragged_len(n, tile), k, idx);
  return hipGetLastError();
}

}  // namespace kascade
