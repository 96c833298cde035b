// Decode attention kernels for gfx950.
//
// One decode query per (batch, query head); the G query heads that share a KV
// head are handled together, so every K/V row is read once for the group.
// Anchor layers run the dense mode over all N cached keys (scores for the
// top-k, optionally the dense output); reuse layers run the gather mode over
// the saved index list (Kascade, euno.news summary, "Methodology" steps 2-3).
//
// Work split: each wavefront owns a share of one (b, KV head)'s keys and
// leaves an unnormalised partial (running max, sum, output) that a small
// combine kernel merges (split-K decoding); the bf16 reuse gather merges them
// at the end of the same kernel instead (merge_group).
//
// bf16 path (matrix cores). For a chunk of 32 keys:
//   S^T[key, head] = K_chunk[32 x d] . Q_group^T[d x 16]   (heads padded to 16)
// K rows are loaded straight from HBM as the A operand (16 bytes per lane,
// four lanes per 64-byte segment of a row), so the operands need no LDS (the
// anchor's LDS holds only its score buffers). The output
// O^T[d, head] += V^T[d x 32] . P^T[32 x 16] needs V transposed; each 16x16
// block of V is transposed exactly by one matrix-core step against a 0/1
// selector matrix (a bf16 value times 1.0 plus zeros is exact in fp32), which
// lands the values in the A-operand lanes of the P.V step. Softmax state is
// per head column: four lanes hold four keys each of one column, so the
// chunk maximum needs two cross-lane steps and everything else is lane-local.
//
// fp32 path (vector ALU): one key per lane, dot products against the group's
// query rows kept in LDS, lane-parallel over d for the P.V accumulation.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kascade {

namespace {

constexpr int kWavesPerBlock = 4;

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

// Registers of one 32-key chunk in flight: K and V rows as A operands and the
// validity of the chunk's 32 list entries (bit e = entry e usable). With
// VLATE the V rows are requested after the chunk's scores are computed, into
// the registers K used.
template <int C, bool VLATE>
struct DecodeStage {
  bf16x8 k[2][C];
  bf16x8 v[2][VLATE ? 1 : C];
  int row[2];
  uint32_t valid;
};

#ifndef KASCADE_DECODE_V_LATE
#define KASCADE_DECODE_V_LATE 1
#endif
#ifndef KASCADE_GATHER_V_LATE
#define KASCADE_GATHER_V_LATE 0
#endif

// Fused split merge of the reuse gather (Kascade reuse layer: the softmax of
// each query row restricted to the saved set, merged over the splits that
// share that set). Every wavefront of the workgroup holds, per head column
// n < G of the group, its running maximum m (log2 units), its sum l and its
// unnormalised output acc (element r of acc[i] is d = 16i + 4qg + r).
//   1. The wavefronts' (m, l, acc) go to LDS and the workgroup merges them
//      (one output element per thread and step): M = max m_w,
//      L = sum l_w 2^(m_w - M), O = sum acc_w 2^(m_w - M).
//   2. One workgroup per (b, KV head): out = O / L (0 if L = 0).
//      Otherwise (M, L, O) go to the partial arrays, and the workgroup takes a
//      ticket on counters[unit]; the workgroup holding the last ticket
//      (gridDim.x - 1) merges the workgroups' partials the same way, writes
//      out and sets the counter back to 0 for the next call.
// Publishing the partials: they are written and read with device-coherent
// (agent-scope) accesses, which bypass the per-XCD L2 caches, and every
// thread waits for its partial stores to complete before the workgroup's
// ticket is taken. A device-scope fence would do the same by writing back
// and invalidating its XCD's whole L2, once per workgroup: measured three
// times slower than the gather itself.
// Device-coherent (agent-scope) float store and load.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int WPB>
__device__ __forceinline__ void merge_group(const DecodeArgs& a, int b, int kvh, float m, float l,
                                            const f32x4 (&acc)[D / 16]) {
  extern __shared__ __attribute__((aligned(16))) float merge_lds[];
  __shared__ int is_last;
  const int G = a.group;
  const int lane = threadIdx.x & 63, n = lane & 15, qg = lane >> 4;
  const int w = wave_id();
  float* red_ml = merge_lds;                      // [WPB][G][2]
  float* red_o = merge_lds + WPB * G * 2;         // [WPB][G][D], 16-byte aligned (G*2*4*WPB % 16 == 0)
  if (n < G) {
    if (qg == 0) {
      red_ml[(w * G + n) * 2] = m;
      red_ml[(w * G + n) * 2 + 1] = l;
    }
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      *reinterpret_cast<f32x4*>(&red_o[(w * G + n) * D + 16 * i + 4 * qg]) = acc[i];
  }
  __syncthreads();
  const int unit = b * a.hkv + kvh;
  const int wgs = gridDim.x, wg = blockIdx.x;
  const int nout = G * D;
  u16* out = static_cast<u16*>(a.out) + (size_t)(b * a.hq + kvh * G) * D;
  for (int o = threadIdx.x; o < nout; o += 64 * WPB) {
    const int g = o / D, c = o - g * D;
    float M = kNegBig;
#pragma unroll
    for (int v = 0; v < WPB; ++v) M = fmaxf(M, red_ml[(v * G + g) * 2]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int v = 0; v < WPB; ++v) {
      const float wt = fast_exp2(red_ml[(v * G + g) * 2] - M);
      L += red_ml[(v * G + g) * 2 + 1] * wt;
      O += red_o[(v * G + g) * D + c] * wt;
    }
    if (wgs == 1) {
      out[o] = float_to_bf16_bits(L > 0.f ? O / L : 0.f);
    } else {
      const size_t slot = ((size_t)unit * wgs + wg) * G + g;
      coherent_store(&a.part_o[slot * D + c], O);
      if (c == 0) {
        coherent_store(&a.part_ml[2 * slot], M);
        coherent_store(&a.part_ml[2 * slot + 1], L);
      }
    }
  }
  if (wgs == 1) return;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = __hip_atomic_fetch_add(&a.counters[unit], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == wgs - 1;
  __syncthreads();
  if (!is_last) return;
  const float* pml = a.part_ml + (size_t)unit * wgs * G * 2;
  const float* po = a.part_o + (size_t)unit * wgs * G * D;
  for (int o = threadIdx.x; o < nout; o += 64 * WPB) {
    const int g = o / D, c = o - g * D;
    float M = kNegBig;
    for (int v = 0; v < wgs; ++v) M = fmaxf(M, coherent_load(&pml[(v * G + g) * 2]));
    float L = 0.f, O = 0.f;
    for (int v = 0; v < wgs; ++v) {
      const float wt = fast_exp2(coherent_load(&pml[(v * G + g) * 2]) - M);
      L += coherent_load(&pml[(v * G + g) * 2 + 1]) * wt;
      O += coherent_load(&po[(size_t)(v * G + g) * D + c]) * wt;
    }
    out[o] = float_to_bf16_bits(L > 0.f ? O / L : 0.f);
  }
  if (threadIdx.x == 0) __hip_atomic_store(&a.counters[unit], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// MERGE (gather only): WPB wavefronts per workgroup, splits = gridDim.x * WPB;
// the split merge runs at the end of the kernel instead of in decode_combine.
template <int D, bool GATHER, bool WITH_PV, bool LOGITS, int WPB = kWavesPerBlock, bool MERGE = false>
__global__ __launch_bounds__(64 * WPB) void decode_attn_bf16(DecodeArgs a) {
  static_assert(!MERGE || (GATHER && WITH_PV && !LOGITS), "the fused merge is for the reuse gather");
  constexpr int C = D / 32;  // contraction chunks of 32 along d
  // The anchor's sweep requests V late (measured faster: its loads then
  // trail the K stream); the short gathered lists request K and V together.
  constexpr bool kVLate = GATHER ? KASCADE_GATHER_V_LATE != 0 : KASCADE_DECODE_V_LATE != 0;
  using Stage = DecodeStage<C, kVLate>;
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x * WPB + wave_id();
  if (!MERGE && split >= a.splits) return;  // merged launches have no partial workgroups
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int n = lane & 15;   // head column (B operand / C column) and A-operand row
  const int qg = lane >> 4;  // lane group: contraction slots 8*qg..8*qg+7
  const int G = a.group;
  const int h0 = kvh * G;

  const u16* q = static_cast<const u16*>(a.q);
  const u16* kb = static_cast<const u16*>(a.k) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const u16* vb = static_cast<const u16*>(a.v) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int32_t* list =
      GATHER ? a.idx + (size_t)(b * a.idx_sets + (a.idx_sets == 1 ? 0 : kvh)) * a.list_len : nullptr;

  // B operand: query head n of the group, d = 32c + 8qg + s; padded heads are 0.
  bf16x8 bq[C];
  const u16* qrow = q + (size_t)(b * a.hq + h0 + (n < G ? n : 0)) * D;
#pragma unroll
  for (int c = 0; c < C; ++c) bq[c] = n < G ? load_bf16x8(qrow + 32 * c + 8 * qg) : zero_bf16x8();

  // Selector operands: column j of selector `half` picks d = 32c + 16*half + j.
  bf16x8 sel[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      sel[half][s] = static_cast<__bf16>((8 * qg + s == 16 * half + n) ? 1.0f : 0.0f);

#ifndef KASCADE_DENSE_INTERLEAVE
#define KASCADE_DENSE_INTERLEAVE 1
#endif
  // Gather mode: split s walks list entries [s*kps, min((s+1)*kps, len)).
  // Dense mode: the splits of a (b, KV head) take its 32-key chunks in turn
  // (split s: chunks s, s + splits, ...), so together they sweep the cache
  // front to back in step rather than each streaming a region of its own.
  constexpr bool kInterleave = !GATHER && KASCADE_DENSE_INTERLEAVE;
  const int begin = kInterleave ? 32 * split : split * a.keys_per_split;
  const int end = kInterleave ? a.list_len : max(begin, min(begin + a.keys_per_split, a.list_len));
  const int stride = kInterleave ? 32 * a.splits : 32;  // keys between a split's chunks
  const int nchunk = kInterleave ? (begin < end ? (end - begin + stride - 1) / stride : 0)
                                 : (end - begin + 31) / 32;

  // Gather mode: lane l reads list entry j0 + (l & 31); rows and validity of
  // the chunk follow by lane exchange, so each entry is read once.
  auto entry_key = [&](int j0) __attribute__((always_inline)) {
    const int pos = j0 + (lane & 31);
    int key = (GATHER && pos < end) ? list[pos] : -1;
    return (unsigned)key < (unsigned)a.n ? key : -1;
  };
  auto load_stage = [&](Stage& st, int key_lane, int j0) __attribute__((always_inline)) {
    int row[2];
    if (GATHER) {
      st.valid = (uint32_t)__ballot(key_lane >= 0);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = __shfl(key_lane, 16 * t + n);
        row[t] = r < 0 ? 0 : r;  // unusable entries read row 0, masked below
      }
    } else {
      const int left = end - j0;
      st.valid = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
#pragma unroll
      for (int t = 0; t < 2; ++t) row[t] = j0 + 16 * t + n < end ? j0 + 16 * t + n : 0;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st.row[t] = row[t];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        st.k[t][c] = load_bf16x8(kb + (size_t)row[t] * D + 32 * c + 8 * qg);
        if (WITH_PV && !kVLate) st.v[t][c] = load_bf16x8(vb + (size_t)row[t] * D + 32 * c + 8 * qg);
      }
    }
  };

  float m = kNegBig, l = 0.0f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Dense mode keeps the scores of up to `cap` chunks in LDS and writes them
  // out together after the last of them: logit stores interleaved with the
  // sweep's loads cost more than the same stores issued in one burst per
  // wavefront.
  constexpr bool kBuffered = LOGITS && !GATHER;
  // Per wavefront 16 KB (8 KB without P.V, 4 KB at d = 64), sized so that
  // the buffers never limit how many wavefronts a compute unit holds.
  constexpr int kLogitFloats = D == 128 ? (WITH_PV ? 4096 : 2048) : 1024;
  __shared__ __attribute__((aligned(16))) float logit_buf[kBuffered ? kWavesPerBlock : 1][kBuffered ? kLogitFloats : 4];
  float* lbuf = &logit_buf[kBuffered ? wave_id() : 0][0];
  const int cap = kBuffered ? kLogitFloats / (32 * G) : 1;  // >= 2 chunks for G <= 16
  int filled = 0;
  auto store_logits = [&](float* dst, const f32x4& v, uint32_t valid, int e0) __attribute__((always_inline)) {
    if ((valid >> (e0 + 3)) & 1u) {
      // Streaming store: the scores are read once, by the selection kernel.
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst));
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if ((valid >> (e0 + r)) & 1u) dst[r] = v[r];
    }
  };
  // After chunk ci: write the buffered chunks out once the buffer is full or
  // the sweep is done.
  auto after_chunk = [&](int ci) __attribute__((always_inline)) {
    if (!kBuffered) return;
    if (++filled < cap && ci + 1 < nchunk) return;
    // Every lane writes: lane l takes the 16-byte piece l % 8 of (chunk, head)
    // row l / 8 of the next eight, so each store instruction writes whole
    // 128-byte lines of eight score rows. Lanes read scores that other lanes
    // of the wavefront wrote to LDS; a wavefront's LDS operations complete in
    // order, and the wavefront-scope fences keep the compiler from moving
    // these reads above those writes.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int pairs = filled * G;  // (chunk, head) rows of 32 scores in the buffer
    const int piece = lane & 7;
    for (int p0 = 0; p0 < pairs; p0 += 8) {
      const int P = p0 + (lane >> 3);
      if (P < pairs) {
        const int f = P / G, hn = P - f * G;
        const int j0 = begin + stride * (ci - filled + 1 + f);
        const int left = end - j0;
        const uint32_t valid = left >= 32 ? 0xffffffffu : ((1u << left) - 1u);
        float* dst = a.logits + (size_t)(b * a.hq + h0 + hn) * a.logits_ld + j0 + 4 * piece;
        store_logits(dst, *reinterpret_cast<const f32x4*>(lbuf + P * 32 + 4 * piece), valid, 4 * piece);
      }
    }
    // The next chunk's scores overwrite the buffer.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    filled = 0;
  };

  auto compute = [&](Stage& st, int j0) __attribute__((always_inline)) {
    float x[2][4];
    float cmax = kNegBig;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) s = mfma16x16x32(st.k[t][c], bq[c], s);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = (st.valid >> (16 * t + 4 * qg + r)) & 1u;
        x[t][r] = ok ? s[r] * a.scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, x[t][r]);
      }
      if (LOGITS && n < G) {
        const f32x4 v = {x[t][0], x[t][1], x[t][2], x[t][3]};
        if (kBuffered)
          *reinterpret_cast<f32x4*>(lbuf + (filled * G + n) * 32 + 16 * t + 4 * qg) = v;
        else
          store_logits(a.logits + (size_t)(b * a.hq + h0 + n) * a.logits_ld + j0 + 16 * t + 4 * qg, v,
                       st.valid, 16 * t + 4 * qg);
      }
    }
    cmax = group4_max(cmax);
    // Lazy rescaling: the reference maximum moves only when a head's maximum
    // grows by more than 2^8, so probabilities stay below 256.
    float alpha = 1.0f;
    const bool rescale = __any(cmax > m + kRescaleLog2);
    if (rescale) {
      const float mnew = fmaxf(m, cmax);
      alpha = fast_exp2(m - mnew);
      m = mnew;
    }
    f32x4 p[2];
    float lsum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[t][r] = fast_exp2(x[t][r] - m);
        lsum += p[t][r];
      }
    l = l * alpha + lsum;
    if (WITH_PV) {
      const bf16x8 pb = pack_bf16x8(p[0], p[1]);
      if (rescale) {
#pragma unroll
        for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
      }
      if (kVLate) {  // K's registers are free now
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int c = 0; c < C; ++c) st.k[t][c] = load_bf16x8(vb + (size_t)st.row[t] * D + 32 * c + 8 * qg);
      }
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          const bf16x8 v0 = kVLate ? st.k[0][c] : st.v[0][kVLate ? 0 : c];
          const bf16x8 v1 = kVLate ? st.k[1][c] : st.v[1][kVLate ? 0 : c];
          const f32x4 t0 = mfma16x16x32(v0, sel[half], z);
          const f32x4 t1 = mfma16x16x32(v1, sel[half], z);
          acc[2 * c + half] = mfma16x16x32(pack_bf16x8(t0, t1), pb, acc[2 * c + half]);
        }
    }
  };

  Stage s0, s1;
#ifndef KASCADE_DECODE_PREFETCH
#define KASCADE_DECODE_PREFETCH 1
#endif
  // Streaming the whole cache (dense) keeps the next chunk in flight; the
  // short gathered lists run more wavefronts per SIMD instead.
#ifndef KASCADE_GATHER_PREFETCH
#define KASCADE_GATHER_PREFETCH 0
#endif
  if (GATHER ? !KASCADE_GATHER_PREFETCH : !KASCADE_DECODE_PREFETCH) {
    for (int i = 0; i < nchunk; ++i) {
      const int j0 = begin + stride * i;
      load_stage(s0, entry_key(j0), j0);
      compute(s0, j0);
      after_chunk(i);
    }
  } else {
  // Two chunks in flight: chunk i+1's rows are requested (and chunk i+2's
  // list entries) before chunk i is computed.
  int kn = entry_key(begin);
  load_stage(s0, kn, begin);
  kn = entry_key(begin + stride);
  for (int i = 0; i < nchunk; i += 2) {
    const int j0 = begin + stride * i;
    if (i + 1 < nchunk) {
      load_stage(s1, kn, j0 + stride);
      kn = entry_key(j0 + 2 * stride);
    }
    compute(s0, j0);
    after_chunk(i);
    if (i + 1 >= nchunk) break;
    if (i + 2 < nchunk) {
      load_stage(s0, kn, j0 + 2 * stride);
      kn = entry_key(j0 + 3 * stride);
    }
    compute(s1, j0 + stride);
    after_chunk(i + 1);
  }
  }

  l = group4_sum(l);
  if constexpr (MERGE) {
    merge_group<D, WPB>(a, b, kvh, m, l, acc);
    return;
  }
  if (n < G) {
    const size_t slot = (size_t)(b * a.hq + h0 + n) * a.splits + split;
    if (qg == 0) {
      a.part_ml[2 * slot] = m;
      a.part_ml[2 * slot + 1] = l;
    }
    if (WITH_PV) {
#pragma unroll
      for (int i = 0; i < D / 16; ++i)
        *reinterpret_cast<f32x4*>(a.part_o + slot * D + 16 * i + 4 * qg) = acc[i];
    }
  }
}

constexpr int kMaxGroup = 16;

template <int D, bool GATHER, bool WITH_PV, bool LOGITS>
__global__ __launch_bounds__(256) void decode_attn_f32(DecodeArgs a) {
  constexpr int E = D / 64;  // output columns per lane
  __shared__ float qs[kMaxGroup][D];
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int h0 = kvh * G;
  const float* q = static_cast<const float*>(a.q);
  for (int i = threadIdx.x; i < G * D; i += blockDim.x)
    qs[i / D][i % D] = q[(size_t)(b * a.hq + h0) * D + i];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x * kWavesPerBlock + wave_id();
  if (split >= a.splits) return;
  const float* kb = static_cast<const float*>(a.k) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const float* vb = static_cast<const float*>(a.v) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int32_t* list =
      GATHER ? a.idx + (size_t)(b * a.idx_sets + (a.idx_sets == 1 ? 0 : kvh)) * a.list_len : nullptr;
  const int begin = split * a.keys_per_split;
  const int end = min(begin + a.keys_per_split, a.list_len);

  float m[kMaxGroup], l[kMaxGroup], acc[kMaxGroup][E];
#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc[g][e] = 0.f;
  }

  for (int j0 = begin; j0 < end; j0 += 64) {
    const int pos = j0 + lane;
    int key = pos < end ? (GATHER ? list[pos] : pos) : -1;
    if (key >= a.n) key = -1;  // outside the cache: skipped like padding
    const bool valid = key >= 0;
    const float* krow = kb + (size_t)(valid ? key : 0) * D;
    float x[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) x[g] = 0.f;
    for (int c = 0; c < D; c += 4) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(krow + c);
#pragma unroll
      for (int g = 0; g < kMaxGroup; ++g)
        if (g < G) x[g] += qs[g][c] * kv[0] + qs[g][c + 1] * kv[1] + qs[g][c + 2] * kv[2] + qs[g][c + 3] * kv[3];
    }
    float p[kMaxGroup];
#pragma unroll
    for (int g = 0; g < kMaxGroup; ++g) {
      if (g >= G) break;
      const float xs = valid ? x[g] * a.scale_log2 : -INFINITY;
      if (LOGITS && valid) a.logits[(size_t)(b * a.hq + h0 + g) * a.logits_ld + key] = xs;
      const float mnew = fmaxf(m[g], wave_max(xs));
      const float alpha = fast_exp2(m[g] - mnew);
      m[g] = mnew;
      p[g] = fast_exp2(xs - mnew);
      l[g] = l[g] * alpha + p[g];
#pragma unroll
      for (int e = 0; e < E; ++e) acc[g][e] *= alpha;
    }
    if (WITH_PV) {
      for (int kk = 0; kk < 64; ++kk) {
        const int key_kk = __shfl(key, kk);
        if (key_kk < 0) continue;  // uniform across the wave
        const float* vrow = vb + (size_t)key_kk * D;
        float vv[E];
#pragma unroll
        for (int e = 0; e < E; ++e) vv[e] = vrow[lane + 64 * e];
#pragma unroll
        for (int g = 0; g < kMaxGroup; ++g) {
          if (g >= G) break;
          const float pk = __shfl(p[g], kk);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[g][e] += pk * vv[e];
        }
      }
    }
  }

#pragma unroll
  for (int g = 0; g < kMaxGroup; ++g) {
    if (g >= G) break;
    const float lt = wave_sum(l[g]);
    const size_t slot = (size_t)(b * a.hq + h0 + g) * a.splits + split;
    if (lane == 0) {
      a.part_ml[2 * slot] = m[g];
      a.part_ml[2 * slot + 1] = lt;
    }
    if (WITH_PV) {
#pragma unroll
      for (int e = 0; e < E; ++e) a.part_o[slot * D + lane + 64 * e] = acc[g][e];
    }
  }
}

// Merge per-split (max, sum, partial output) of query rows; one wave per row.
// Every load is issued before any result is needed (one memory round trip):
// lane c holds output columns 2c, 2c+1 (d = 128) or c (d = 64) of each split.
template <bool BF16, int D>
__global__ __launch_bounds__(256) void decode_combine(const float* part_ml, const float* part_o,
                                                     int rows, int splits, void* out,
                                                     float* lse, float* lse2) {
  constexpr int E = D / 64;  // columns per lane
  constexpr int kBatch = 16; // splits loaded per round
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave_id();
  if (row >= rows) return;
  const float* ml = part_ml + (size_t)row * splits * 2;
  const float* po = part_o + (size_t)row * splits * D + E * lane;
  const bool want_o = out != nullptr;  // partial outputs exist only when the output is requested
  float M = kNegBig, L = 0.f;
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < splits; s0 += kBatch) {
    float mv[kBatch], lv[kBatch], ov[kBatch][E];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int s = min(s0 + i, splits - 1);
      mv[i] = ml[2 * s];
      lv[i] = ml[2 * s + 1];
      if (!want_o) {
#pragma unroll
        for (int e = 0; e < E; ++e) ov[i][e] = 0.f;
      } else if (E == 2) {
        const float2 v = *reinterpret_cast<const float2*>(po + (size_t)s * D);
        ov[i][0] = v.x;
        ov[i][E - 1] = v.y;
      } else {
        ov[i][0] = po[(size_t)s * D];
      }
    }
    float mb = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (s0 + i < splits) mb = fmaxf(mb, mv[i]);
    const float alpha = fast_exp2(M - mb);
    L *= alpha;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= alpha;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const float w = s0 + i < splits ? fast_exp2(mv[i] - mb) : 0.f;
      L += lv[i] * w;
#pragma unroll
      for (int e = 0; e < E; ++e) o[e] += ov[i][e] * w;
    }
    M = mb;
  }
  if (lane == 0) {
    if (lse) lse[row] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
    if (lse2) lse2[row] = M + log2f(L);
  }
  if (!out) return;
  const float inv = L > 0.f ? 1.0f / L : 0.f;
  if (BF16) {
    u16* dst = static_cast<u16*>(out) + (size_t)row * D + E * lane;
    if (E == 2)
      *reinterpret_cast<uint32_t*>(dst) =
          float_to_bf16_bits(o[0] * inv) | ((uint32_t)float_to_bf16_bits(o[E - 1] * inv) << 16);
    else
      dst[0] = float_to_bf16_bits(o[0] * inv);
  } else {
    float* dst = static_cast<float*>(out) + (size_t)row * D + E * lane;
#pragma unroll
    for (int e = 0; e < E; ++e) dst[e] = o[e] * inv;
  }
}

template <int D>
hipError_t launch_attn_d(const DecodeArgs& a, bool bf16, bool gather, bool with_pv,
                         hipStream_t s) {
  dim3 grid((a.splits + kWavesPerBlock - 1) / kWavesPerBlock, a.hkv, a.batch);
  dim3 block(64 * kWavesPerBlock);
  const bool logits = a.logits != nullptr;
#define KASCADE_DECODE_CASE(G_, P_, L_)                                                      \
  if (gather == G_ && with_pv == P_ && logits == L_) {                                       \
    if (bf16)                                                                                \
      hipLaunchKernelGGL((decode_attn_bf16<D, G_, P_, L_>), grid, block, 0, s, a);           \
    else                                                                                     \
      hipLaunchKernelGGL((decode_attn_f32<D, G_, P_, L_>), grid, block, 0, s, a);            \
    return hipGetLastError();                                                                \
  }
  KASCADE_DECODE_CASE(true, true, false)
  KASCADE_DECODE_CASE(false, true, true)
  KASCADE_DECODE_CASE(false, false, true)
  KASCADE_DECODE_CASE(false, true, false)
  KASCADE_DECODE_CASE(false, false, false)
#undef KASCADE_DECODE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_attn(const DecodeArgs& a, bool bf16, bool gather, bool with_pv,
                              hipStream_t s) {
  if (a.d == 64) return launch_attn_d<64>(a, bf16, gather, with_pv, s);
  if (a.d == 128) return launch_attn_d<128>(a, bf16, gather, with_pv, s);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_gather_merged(const DecodeArgs& a, hipStream_t s) {
  if (a.splits % kGatherWaves != 0 || a.group > 16) return hipErrorInvalidValue;
  const dim3 grid(a.splits / kGatherWaves, a.hkv, a.batch), block(64 * kGatherWaves);
  const size_t lds = gather_merge_lds_bytes(a.group, a.d);
  if (a.d == 128)
    hipLaunchKernelGGL((decode_attn_bf16<128, true, true, false, kGatherWaves, true>), grid, block, lds, s, a);
  else if (a.d == 64)
    hipLaunchKernelGGL((decode_attn_bf16<64, true, true, false, kGatherWaves, true>), grid, block, lds, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_combine(const float* part_ml, const float* part_o, int rows, int splits,
                                 int d, bool bf16, void* out, float* lse, float* lse2,
                                 hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
#define KASCADE_COMBINE(B_, D_) \
  hipLaunchKernelGGL((decode_combine<B_, D_>), grid, block, 0, s, part_ml, part_o, rows, splits, out, lse, lse2)
  if (d == 128) {
    if (bf16) KASCADE_COMBINE(true, 128); else KASCADE_COMBINE(false, 128);
  } else if (d == 64) {
    if (bf16) KASCADE_COMBINE(true, 64); else KASCADE_COMBINE(false, 64);
  } else {
    return hipErrorInvalidValue;
  }
#undef KASCADE_COMBINE
  return hipGetLastError();
}

}  // namespace kascade
