// Decode attention kernels for gfx950.
//
// One decode query per (batch, query head); the G query heads that share a KV
// head are handled together, so every K/V row is read once for the group.
// Anchor layers run the dense mode over all N cached keys (scores for the
// top-k, optionally the dense output); reuse layers run the gather mode over
// the saved index list (Kascade, euno.news summary, "Methodology" steps 2-3).
//
// Work split: each wavefront owns `keys_per_split` consecutive list entries of
// one (b, KV head) and leaves an unnormalised partial (running max, sum,
// output) that a small combine kernel merges (split-K decoding).
//
// bf16 path (matrix cores). For a chunk of 32 keys:
//   S^T[key, head] = K_chunk[32 x d] . Q_group^T[d x 16]   (heads padded to 16)
// K rows are loaded straight from HBM as the A operand (16 bytes per lane,
// four lanes per 64-byte segment of a row), so no LDS is needed. The output
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

template <int D, bool GATHER, bool WITH_PV, bool LOGITS>
__global__ __launch_bounds__(256) void decode_attn_bf16(DecodeArgs a) {
  constexpr int C = D / 32;  // contraction chunks of 32 along d
  const int lane = threadIdx.x & 63;
  const int split = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (split >= a.splits) return;
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int n = lane & 15;   // head column (B operand / C column) and A-operand row
  const int qg = lane >> 4;  // lane group: contraction slots 8*qg..8*qg+7
  const int G = a.group;
  const int h0 = kvh * G;

  const u16* q = static_cast<const u16*>(a.q);
  const u16* kb = static_cast<const u16*>(a.k) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const u16* vb = static_cast<const u16*>(a.v) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int32_t* list = GATHER ? a.idx + (size_t)(b * a.hkv + kvh) * a.list_len : nullptr;

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

  const int begin = split * a.keys_per_split;
  const int end = min(begin + a.keys_per_split, a.list_len);

  float m = kNegBig, l = 0.0f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int j0 = begin; j0 < end; j0 += 32) {
    // Row loaded by this lane for tiles t = 0, 1 (keys j0 + 16t + n).
    int row[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int pos = j0 + 16 * t + n;
      int key = pos < end ? (GATHER ? list[pos] : pos) : -1;
      row[t] = (key < 0 || key >= a.n) ? 0 : key;  // masked keys read row 0, discarded
    }
    // Keys held in this lane's accumulator slots: j0 + 16t + 4qg + r.
    bool valid[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = j0 + 16 * t + 4 * qg + r;
        valid[t][r] = pos < end && (!GATHER || (unsigned)list[pos] < (unsigned)a.n);
      }

    bf16x8 ka[2][C];
    bf16x8 va[2][C];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        ka[t][c] = load_bf16x8(kb + (size_t)row[t] * D + 32 * c + 8 * qg);
        if (WITH_PV) va[t][c] = load_bf16x8(vb + (size_t)row[t] * D + 32 * c + 8 * qg);
      }

    float x[2][4];
    float cmax = kNegBig;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < C; ++c) s = mfma16x16x32(ka[t][c], bq[c], s);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[t][r] = valid[t][r] ? s[r] * a.scale_log2 : -INFINITY;
        cmax = fmaxf(cmax, x[t][r]);
      }
      if (LOGITS && n < G) {
        float* dst = a.logits + (size_t)(b * a.hq + h0 + n) * a.logits_ld + j0 + 16 * t + 4 * qg;
        if (valid[t][3]) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{x[t][0], x[t][1], x[t][2], x[t][3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (valid[t][r]) dst[r] = x[t][r];
        }
      }
    }
    cmax = group4_max(cmax);
    const float mnew = fmaxf(m, cmax);
    const float alpha = fast_exp2(m - mnew);
    m = mnew;
    l *= alpha;
    f32x4 p[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[t][r] = fast_exp2(x[t][r] - m);
        l += p[t][r];
      }
    if (WITH_PV) {
      const bf16x8 pb = pack_bf16x8(p[0], p[1]);
#pragma unroll
      for (int i = 0; i < D / 16; ++i) acc[i] *= alpha;
#pragma unroll
      for (int c = 0; c < C; ++c)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          f32x4 t0 = mfma16x16x32(va[0][c], sel[half], z);
          f32x4 t1 = mfma16x16x32(va[1][c], sel[half], z);
          acc[2 * c + half] = mfma16x16x32(pack_bf16x8(t0, t1), pb, acc[2 * c + half]);
        }
    }
  }

  l = group4_sum(l);
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
  const int split = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (split >= a.splits) return;
  const float* kb = static_cast<const float*>(a.k) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const float* vb = static_cast<const float*>(a.v) + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int32_t* list = GATHER ? a.idx + (size_t)(b * a.hkv + kvh) * a.list_len : nullptr;
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

// Merge per-split (max, sum, partial output) of one query row.
template <bool BF16>
__global__ __launch_bounds__(128) void decode_combine(const float* part_ml, const float* part_o,
                                                     int splits, int d, void* out, float* lse) {
  const int row = blockIdx.x;
  const float* ml = part_ml + (size_t)row * splits * 2;
  float M = kNegBig;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
  float L = 0.f;
  for (int s = 0; s < splits; ++s) L += ml[2 * s + 1] * fast_exp2(ml[2 * s] - M);
  if (out) {
    for (int c = threadIdx.x; c < d; c += blockDim.x) {
      float o = 0.f;
      for (int s = 0; s < splits; ++s)
        o += part_o[((size_t)row * splits + s) * d + c] * fast_exp2(ml[2 * s] - M);
      o = L > 0.f ? o / L : 0.f;
      if (BF16)
        static_cast<u16*>(out)[(size_t)row * d + c] = float_to_bf16_bits(o);
      else
        static_cast<float*>(out)[(size_t)row * d + c] = o;
    }
  }
  if (lse && threadIdx.x == 0) lse[row] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

__global__ __launch_bounds__(256) void decode_pool(const float* logits, const float* part_ml,
                                                   int hq, int hkv, int group, int n, int splits,
                                                   float* pooled) {
  const size_t ld = decode_logits_ld(n);
  __shared__ float lse2[kMaxGroup];
  const int kvh = blockIdx.y, b = blockIdx.z;
  if (threadIdx.x < group) {
    const float* ml = part_ml + (size_t)(b * hq + kvh * group + threadIdx.x) * splits * 2;
    float M = kNegBig;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f;
    for (int s = 0; s < splits; ++s) L += ml[2 * s + 1] * fast_exp2(ml[2 * s] - M);
    lse2[threadIdx.x] = M + log2f(L);
  }
  __syncthreads();
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= n) return;
  float acc = 0.f;
  for (int g = 0; g < group; ++g)
    acc += fast_exp2(logits[(size_t)(b * hq + kvh * group + g) * ld + j] - lse2[g]);
  // The sum over heads ranks keys exactly as the mean does.
  pooled[(size_t)(b * hkv + kvh) * n + j] = acc;
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

hipError_t launch_decode_combine(const float* part_ml, const float* part_o, int rows, int splits,
                                 int d, bool bf16, void* out, float* lse, hipStream_t s) {
  if (bf16)
    hipLaunchKernelGGL(decode_combine<true>, dim3(rows), dim3(128), 0, s, part_ml, part_o, splits,
                       d, out, lse);
  else
    hipLaunchKernelGGL(decode_combine<false>, dim3(rows), dim3(128), 0, s, part_ml, part_o, splits,
                       d, out, lse);
  return hipGetLastError();
}

hipError_t launch_decode_pool(const float* logits, const float* part_ml, int batch, int hq,
                              int hkv, int group, int n, int splits, float* pooled,
                              hipStream_t s) {
  dim3 grid((n + 255) / 256, hkv, batch);
  hipLaunchKernelGGL(decode_pool, grid, dim3(256), 0, s, logits, part_ml, hq, hkv, group, n,
                     splits, pooled);
  return hipGetLastError();
}

}  // namespace kascade
