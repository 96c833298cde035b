// Exact top-k selection for the anchor layer ("exact Top-k indices", Kascade
// abstract on the opentrain.ai page, "Abstract").
//
// Input: non-negative float32 scores (pooled post-softmax probabilities). For
// non-negative IEEE floats the 32-bit pattern orders like the value, so the
// k-th largest score is found by an MSB-first radix select over the bit
// patterns: four passes of an 8-bit digit histogram in LDS, each narrowing to
// the digit bucket that holds the k-th element. That gives the exact threshold
// pattern and how many keys equal to it are still needed. A final ordered
// pass then writes, in ascending key order, every key above the threshold and
// the lowest-indexed keys equal to it (block-wide ballot scans keep the order),
// then pads with -1. No sort is needed, and the result is deterministic.
//
// One 1024-thread workgroup per segment. Histogram atomics are aggregated per
// wavefront for the most common digit, since the leading digits of
// probabilities cluster around a few exponents.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kascade {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ void hist_add(unsigned* hist, unsigned digit, bool active) {
  const uint64_t act = __ballot(active);
  if (act == 0) return;
  const int leader = __ffsll((unsigned long long)act) - 1;
  const unsigned d0 = __shfl(digit, leader);
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
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += kThreads) {
      const int j = j0 + tid;
      const unsigned u = j < n ? keys[j] : 0u;
      const bool match = j < n && (u & mask) == prefix;
      hist_add(hist, (u >> shift) & 255u, match);
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
    mask |= 255u << shift;
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

__global__ __launch_bounds__(kThreads) void topk_decode_kernel(const float* scores, int n, int k,
                                                                 int32_t* idx) {
  const size_t seg = blockIdx.x;
  select_segment(reinterpret_cast<const unsigned*>(scores) + seg * n, n, k, k, idx + seg * k);
}

__global__ __launch_bounds__(kThreads) void topk_prefill_kernel(const float* scores, int hkv,
                                                                  int n, int tile, int tiles,
                                                                  size_t ragged, int k,
                                                                  int32_t* idx) {
  const int t = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int prefix = min((t + 1) * tile, n);
  const size_t base = (size_t)(b * hkv + kvh) * ragged + (size_t)tile * t * (t + 1) / 2;
  int32_t* out = idx + ((size_t)(b * hkv + kvh) * tiles + t) * k;
  select_segment(reinterpret_cast<const unsigned*>(scores) + base, prefix, min(k, prefix), k, out);
}

}  // namespace

hipError_t launch_topk_decode(const float* scores, int segments, int n, int k, int32_t* idx,
                              hipStream_t s) {
  hipLaunchKernelGGL(topk_decode_kernel, dim3(segments), dim3(kThreads), 0, s, scores, n, k, idx);
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
