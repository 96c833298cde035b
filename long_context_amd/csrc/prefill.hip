// Causal prefill kernels for gfx950 (bf16 inputs, fp32 accumulation).
//
// prefill_attn: flash-style causal attention of one query tile of one head
// over a key list. Dense mode (anchor pass 1) walks keys 0..prefix_t-1 and
// writes the per-row log-sum-exp (and, on request, the dense output); gather
// mode (reuse layer) walks the tile's saved index list, softmax restricted to
// the saved keys j <= i (Kascade, euno.news summary, "Methodology" steps 3
// and 6: one index set per query tile, values recomputed with the layer's own
// tensors).
//   Per 64-key chunk the workgroup stages K and V rows in LDS (gathered rows
//   are fetched 16 bytes per lane, 16 lanes per 256-byte row). Each wave owns
//   32 query rows and computes S^T = K . Q^T on the matrix cores, so the
//   softmax of a row lives in one lane column (four lanes, two cross-lane
//   steps per chunk), and O^T += V^T . P^T with P^T taken straight from the
//   S^T accumulators. V^T operands are read from LDS transposed.
//
// prefill_pool: anchor pass 2. For tile t and key j < prefix_t:
//   pooled[t, j] = sum over the group's heads and the tile's rows i >= j of
//                  exp2(x_ij - lse2_i)
// i.e. the post-softmax probabilities summed over the tile (the sum ranks
// keys as the mean does). The row log-sum-exp must be final before any term
// is added, so the scores are recomputed rather than stored. Each wave keeps
// 64 keys of K resident as matrix-core operands and streams the tile's query
// rows through LDS; column sums are lane-local until one final cross-lane step.
#include "device_common.hpp"
#include "kernels.hpp"

namespace kascade {

namespace {

constexpr int kKeyChunk = 64;
constexpr int kRowsPerWave = 32;
constexpr int kTile = 128;            // query tile; four waves of 32 rows
constexpr int kLdsPad = 8;            // bf16 elements of padding per LDS row

__device__ __forceinline__ int pv_key(int qg, int s) {
  // Contraction slot s of lane group qg in the P.V step, as laid out by the
  // S^T accumulators of two consecutive 16-key tiles.
  return s < 4 ? 4 * qg + s : 16 + 4 * qg + (s - 4);
}

template <int D, bool GATHER, bool WITH_O>
__global__ __launch_bounds__(256) void prefill_attn(PrefillArgs a) {
  constexpr int C = D / 32;
  constexpr int LD = D + kLdsPad;
  __shared__ __attribute__((aligned(16))) __bf16 ks[kKeyChunk * LD];
  __shared__ __attribute__((aligned(16))) __bf16 vs[kKeyChunk * LD];
  __shared__ int keys_s[kKeyChunk];

  const int t = a.tiles - 1 - blockIdx.x;  // longest tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = h / a.group;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, qg = lane >> 4;
  const int prefix = min((t + 1) * kTile, a.n);
  const int wrow0 = t * kTile + wave * kRowsPerWave;  // first row of this wave

  const u16* kb = a.k + (size_t)(b * a.hkv + kvh) * a.n * D;
  const u16* vb = a.v + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int32_t* list = GATHER ? a.idx + ((size_t)(b * a.hkv + kvh) * a.tiles + t) * a.topk : nullptr;
  const int list_len = GATHER ? min(a.topk, prefix) : prefix;

  // Q^T operands for the wave's two 16-row blocks (rows past N read row N-1).
  bf16x8 bq[2][C];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = min(wrow0 + 16 * rb + n16, a.n - 1);
    const u16* qrow = a.q + ((size_t)(b * a.hq + h) * a.n + row) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) bq[rb][c] = load_bf16x8(qrow + 32 * c + 8 * qg);
  }

  float m[2] = {kNegBig, kNegBig}, l[2] = {0.f, 0.f};
  f32x4 acc[2][D / 16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < D / 16; ++i) acc[rb][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int kThreadsPerRow = D / 8;
  constexpr int kRowsPerPass = 256 / kThreadsPerRow;

  for (int j0 = 0; j0 < list_len; j0 += kKeyChunk) {
    __syncthreads();  // previous chunk fully consumed
    if (tid < kKeyChunk) {
      const int pos = j0 + tid;
      int key = pos < list_len ? (GATHER ? list[pos] : pos) : -1;
      keys_s[tid] = key < a.n ? key : -1;  // entries outside the sequence are skipped
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kKeyChunk / kRowsPerPass; ++p) {
      const int rr = p * kRowsPerPass + tid / kThreadsPerRow;
      const int cc = (tid % kThreadsPerRow) * 8;
      const int key = keys_s[rr];
      const int src = key < 0 ? 0 : key;
      *reinterpret_cast<bf16x8*>(&ks[rr * LD + cc]) = load_bf16x8(kb + (size_t)src * D + cc);
      if (WITH_O)
        *reinterpret_cast<bf16x8*>(&vs[rr * LD + cc]) = load_bf16x8(vb + (size_t)src * D + cc);
    }
    __syncthreads();

    // Smallest key of the chunk above every row of this wave: nothing to do.
    int kmin = 0x7fffffff;
    {
      const int key = keys_s[lane];
      if (key >= 0) kmin = key;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) kmin = min(kmin, __shfl_xor(kmin, o));
    }
    if (kmin > wrow0 + kRowsPerWave - 1) continue;

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {  // two 32-key halves of the chunk
      int kkey[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) kkey[kt][r] = keys_s[32 * sub + 16 * kt + 4 * qg + r];

      f32x4 p[2][2];  // [row block][key tile]
      float alpha[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int row = wrow0 + 16 * rb + n16;
        float x[2][4], cmax = kNegBig;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          f32x4 s = {0.f, 0.f, 0.f, 0.f};
          const __bf16* krow = &ks[(32 * sub + 16 * kt + n16) * LD];
#pragma unroll
          for (int c = 0; c < C; ++c)
            s = mfma16x16x32(*reinterpret_cast<const bf16x8*>(krow + 32 * c + 8 * qg), bq[rb][c], s);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = kkey[kt][r];
            x[kt][r] = (key >= 0 && key <= row) ? s[r] * a.scale_log2 : -INFINITY;
            cmax = fmaxf(cmax, x[kt][r]);
          }
        }
        cmax = group4_max(cmax);
        const float mnew = fmaxf(m[rb], cmax);
        alpha[rb] = fast_exp2(m[rb] - mnew);
        m[rb] = mnew;
        l[rb] *= alpha[rb];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[rb][kt][r] = fast_exp2(x[kt][r] - mnew);
            l[rb] += p[rb][kt][r];
          }
      }
      if (WITH_O) {
        bf16x8 pb[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          pb[rb] = pack_bf16x8(p[rb][0], p[rb][1]);
#pragma unroll
          for (int i = 0; i < D / 16; ++i) acc[rb][i] *= alpha[rb];
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          bf16x8 av;
#pragma unroll
          for (int s = 0; s < 8; ++s) av[s] = vs[(32 * sub + pv_key(qg, s)) * LD + 16 * db + n16];
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[rb][db] = mfma16x16x32(av, pb[rb], acc[rb][db]);
        }
      }
    }
  }

#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float lt = group4_sum(l[rb]);
    const int row = wrow0 + 16 * rb + n16;
    if (row >= a.n) continue;
    const size_t orow = (size_t)(b * a.hq + h) * a.n + row;
    if (!GATHER && qg == 0) a.lse2[orow] = m[rb] + log2f(lt);
    if (WITH_O) {
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        u16 o4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) o4[r] = float_to_bf16_bits(acc[rb][db][r] * inv);
        *reinterpret_cast<uint2*>(a.out + orow * D + 16 * db + 4 * qg) =
            make_uint2(o4[0] | (uint32_t(o4[1]) << 16), o4[2] | (uint32_t(o4[3]) << 16));
      }
    }
  }
}

constexpr int kPoolKeysPerWave = 64;
constexpr int kPoolKeysPerBlock = 4 * kPoolKeysPerWave;

template <int D>
__global__ __launch_bounds__(256) void prefill_pool(PrefillArgs a) {
  constexpr int C = D / 32;
  constexpr int LD = D + kLdsPad;
  __shared__ __attribute__((aligned(16))) __bf16 qs[16 * LD];
  __shared__ float lse_s[16];

  const int chunk = blockIdx.x, t = blockIdx.y;
  const int kvh = blockIdx.z % a.hkv, b = blockIdx.z / a.hkv;
  const int prefix = min((t + 1) * kTile, a.n);
  const int kbase = chunk * kPoolKeysPerBlock;
  if (kbase >= prefix) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, qg = lane >> 4;
  const int row0 = t * kTile, rows = prefix - row0;
  const int wkey0 = kbase + wave * kPoolKeysPerWave;

  // K^T operands of this wave's 64 keys (keys past prefix read key 0, masked).
  const u16* kb = a.k + (size_t)(b * a.hkv + kvh) * a.n * D;
  bf16x8 bk[4][C];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = wkey0 + 16 * kt + n16;
    const u16* krow = kb + (size_t)(key < prefix ? key : 0) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) bk[kt][c] = load_bf16x8(krow + 32 * c + 8 * qg);
  }
  float colsum[4] = {0.f, 0.f, 0.f, 0.f};

  const int blocks_per_head = (rows + 15) / 16;
  for (int g = 0; g < a.group; ++g) {
    const int h = kvh * a.group + g;
    for (int rbk = 0; rbk < blocks_per_head; ++rbk) {
      const int r0 = row0 + 16 * rbk;
      if (r0 + 15 < kbase) continue;  // every key of the block is above every row
      __syncthreads();
      {
        const int rr = tid / (D / 8), cc = (tid % (D / 8)) * 8;
        if (rr < 16) {
          const int row = min(r0 + rr, a.n - 1);
          *reinterpret_cast<bf16x8*>(&qs[rr * LD + cc]) =
              load_bf16x8(a.q + ((size_t)(b * a.hq + h) * a.n + row) * D + cc);
        }
        if (tid < 16) {
          const int row = r0 + tid;
          lse_s[tid] = row < a.n ? a.lse2[(size_t)(b * a.hq + h) * a.n + row] : INFINITY;
        }
      }
      __syncthreads();
      if (r0 + 15 < wkey0) continue;
      bf16x8 aq[C];
#pragma unroll
      for (int c = 0; c < C; ++c)
        aq[c] = *reinterpret_cast<const bf16x8*>(&qs[n16 * LD + 32 * c + 8 * qg]);
      float lse_r[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) lse_r[r] = lse_s[4 * qg + r];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < C; ++c) s = mfma16x16x32(aq[c], bk[kt][c], s);
        const int key = wkey0 + 16 * kt + n16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 4 * qg + r;
          const float pr = fast_exp2(s[r] * a.scale_log2 - lse_r[r]);
          colsum[kt] += (key <= row && row < a.n) ? pr : 0.f;
        }
      }
    }
  }

  const size_t ragged = prefill_ragged_len(a.n, kTile);
  float* dst = a.pooled + (size_t)(b * a.hkv + kvh) * ragged + (size_t)kTile * t * (t + 1) / 2;
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const float v = group4_sum(colsum[kt]);
    const int key = wkey0 + 16 * kt + n16;
    if (qg == 0 && key < prefix) dst[key] = v;
  }
}

__global__ void lse2_to_lse_kernel(const float* lse2, float* lse, size_t count) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) lse[i] = lse2[i] * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_prefill_dense(const PrefillArgs& a, hipStream_t s) {
  dim3 grid(a.tiles, a.hq, a.batch), block(256);
  const bool with_o = a.out != nullptr;
  if (a.d == 128) {
    if (with_o) hipLaunchKernelGGL((prefill_attn<128, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((prefill_attn<128, false, false>), grid, block, 0, s, a);
  } else if (a.d == 64) {
    if (with_o) hipLaunchKernelGGL((prefill_attn<64, false, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((prefill_attn<64, false, false>), grid, block, 0, s, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_reuse(const PrefillArgs& a, hipStream_t s) {
  dim3 grid(a.tiles, a.hq, a.batch), block(256);
  if (a.d == 128) hipLaunchKernelGGL((prefill_attn<128, true, true>), grid, block, 0, s, a);
  else if (a.d == 64) hipLaunchKernelGGL((prefill_attn<64, true, true>), grid, block, 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s) {
  dim3 grid((a.n + kPoolKeysPerBlock - 1) / kPoolKeysPerBlock, a.tiles, a.hkv * a.batch);
  if (a.d == 128) hipLaunchKernelGGL(prefill_pool<128>, grid, dim3(256), 0, s, a);
  else if (a.d == 64) hipLaunchKernelGGL(prefill_pool<64>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lse2_to_lse(const float* lse2, float* lse, size_t count, hipStream_t s) {
  hipLaunchKernelGGL(lse2_to_lse_kernel, dim3((count + 255) / 256), dim3(256), 0, s, lse2, lse,
                     count);
  return hipGetLastError();
}

}  // namespace kascade
