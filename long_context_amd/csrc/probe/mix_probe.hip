// Measurement probe (not part of the attention path): how much of the vector
// work of the prefill kernels hides behind their matrix-core work on gfx950,
// against wavefronts per SIMD and against workgroup synchronisation. Register-
// and LDS-only loops with the instruction mix of the kernels' inner steps:
//
//   pool: the pooled pass's 16-row block -- 4C v_mfma_f32_16x16x32_bf16 on
//     resident K operands (C = d / 32 slices of 32), then an fma, an exp2 and
//     an add on each of the 16 scores of the lane, which depend on the MFMAs.
//   attn: a 32-row x 32-key attention step on v_mfma_f32_32x32x16_bf16 --
//     S^T = K . Q^T (d / 16 MFMAs, K slices read from LDS), the online softmax
//     of the lane's 16 scores (max, exchange with lane l^32, fma, exp2, sum,
//     bf16 packing) and O^T += V^T . P^T (d / 16 MFMAs, V^T read transposed
//     from LDS), on a static K / V tile in LDS.
//     mode 0: each step's operands read one step ahead, no synchronisation;
//     mode 1: as 0, plus a workgroup barrier per step;
//     mode 2: each MFMA's operands read just before it, barrier per step;
//     mode 3: as 0, but instead of a barrier each wavefront waits (bounded
//             spin on an LDS counter) until every wavefront of the workgroup
//             has finished the step before the previous one;
//     mode 4: as 0, but K stays in registers (read from LDS once), so that
//             the step's LDS traffic is the V^T reads alone.
// Results are folded into `out` so that nothing is optimised away. Used by
// bench.py --probe mix.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "lds_stage.hpp"

namespace {

using namespace kascade;

template <int C>
__global__ __launch_bounds__(256) void pool_mix(float* out, int iters, float sl2) {
  const int tid = threadIdx.x;
  bf16x8 a[C], bk[4][C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) a[c][i] = static_cast<__bf16>(0.01f * ((tid + i + c) & 7));
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) bk[k][c][i] = static_cast<__bf16>(0.01f * ((tid * 3 + i + k + c) & 7));
  const f32x4 lse = {1.f, 2.f, 3.f, 4.f};
  float colsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
    f32x4 s[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) s[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) s[k] = mfma16x16x32(a[c], bk[k][c], s[k]);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) colsum[k] += fast_exp2(fmaf(s[k][r], sl2, -lse[r]));
    __builtin_amdgcn_sched_barrier(0);
  }
  out[blockIdx.x * 256 + tid] = colsum[0] + colsum[1] + colsum[2] + colsum[3];
}

template <int MODE, int D, int WAVES>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(WAVES)))
void attn_mix(float* out, int iters, float sl2) {
  constexpr int C = D / 16, DB = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char ks[32 * 256];
  __shared__ __attribute__((aligned(16))) unsigned char vs[32 * 256];
  __shared__ int done;
  const int tid = threadIdx.x, lane = tid & 63, col = lane & 31, hf = lane >> 5;
  for (int i = tid; i < 32 * 256 / 4; i += 256) {
    reinterpret_cast<unsigned*>(ks)[i] = 0x3c003c00u ^ ((unsigned)i * 2654435761u & 0x00ff00ffu);
    reinterpret_cast<unsigned*>(vs)[i] = 0x3c003c00u ^ ((unsigned)i * 2246822519u & 0x00ff00ffu);
  }
  if (tid == 0) done = 0;
  __syncthreads();
  bf16x8 q[C];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int i = 0; i < 8; ++i) q[c][i] = static_cast<__bf16>(0.01f * ((tid + i + c) & 7));
  const int kswz = col & 15;
  const int vL = lane & 15, vg = lane >> 4;
  const int vrow = 4 * (vg >> 1) + (vL >> 2), vslot = 2 * (vg & 1) + ((vL & 3) >> 1);
  // The tile never changes, so the compiler would hoist every K read out of
  // the loop; an offset it cannot see through (always 0) keeps them in.
  int koff = 0;
  auto kread = [&](int c) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(ks + koff + col * 256 + 16 * ((2 * c + hf) ^ kswz));
  };
  auto vread = [&](int db, int s2) -> bf16x8 {
    const unsigned char* v0 = vs + koff + vrow * 256;
    const int off0 = 16 * ((vslot + 4 * db) ^ (vrow & 15)) + 8 * (vL & 1);
    const int off1 = 16 * ((vslot + 4 * db) ^ ((vrow + 8) & 15)) + 8 * (vL & 1);
    const lds_bf16x4 lo = lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2) * 256 + off0));
    const lds_bf16x4 hi = lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2 + 8) * 256 + off1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  f32x16 o[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) o[d] = zero_f32x16();
  float m = -1e30f, l = 0.f;
  constexpr bool AHEAD = MODE != 2;
  bf16x8 kf[AHEAD ? C : 1], vf[AHEAD ? DB : 1][2], pb[2];
  if constexpr (AHEAD) {
#pragma unroll
    for (int c = 0; c < C; ++c) kf[c] = kread(c);
#pragma unroll
    for (int d = 0; d < DB; ++d) vf[d][0] = vf[d][1] = q[0];
  }
  pb[0] = pb[1] = q[0];
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(koff));
    if constexpr (MODE == 1 || MODE == 2) __syncthreads();
    if constexpr (MODE == 3) {
      const int target = 4 * (it - 1);
      int spins = 0;
      while (__hip_atomic_load(&done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target && ++spins < (1 << 16))
        __builtin_amdgcn_s_sleep(1);
    }
    f32x16 s = zero_f32x16();
    if constexpr (AHEAD) {
      // P.V of the previous step, V^T of this one, scores, next step's K.
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) o[d] = mfma32x32x16(vf[d][s2], pb[s2], o[d]);
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) vf[d][s2] = vread(d, s2);
#pragma unroll
      for (int c = 0; c < C; ++c) s = mfma32x32x16(kf[c], q[c], s);
      if constexpr (MODE != 4) {
#pragma unroll
        for (int c = 0; c < C; ++c) kf[c] = kread(c);
      }
    } else {
#pragma unroll
      for (int c = 0; c < C; ++c) s = mfma32x32x16(kread(c), q[c], s);
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(m, mx * sl2);
    m = mn;
    float p[16];
    float ls = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = fast_exp2(fmaf(s[i], sl2, -mn));
      ls += p[i];
    }
    l += ls;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pb[0][i] = static_cast<__bf16>(p[i]);
      pb[1][i] = static_cast<__bf16>(p[8 + i]);
    }
    if constexpr (MODE == 3) {
      if (lane == 0) __hip_atomic_fetch_add(&done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if constexpr (!AHEAD) {
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) o[d] = mfma32x32x16(vread(d, s2), pb[s2], o[d]);
    }
  }
  float r = m + l;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) r += o[d][i];
  out[blockIdx.x * 256 + tid] = r;
}

template <int MODE, int D>
hipError_t launch_attn_mix(int wps, int blocks, float* out, int iters, hipStream_t s) {
  // The register budget follows the wavefronts per SIMD asked for.
  if (wps <= 2) hipLaunchKernelGGL((attn_mix<MODE, D, 2>), dim3(blocks), dim3(256), 0, s, out, iters, 0.1f);
  else hipLaunchKernelGGL((attn_mix<MODE, D, 3>), dim3(blocks), dim3(256), 0, s, out, iters, 0.1f);
  return hipGetLastError();
}

}  // namespace

// kind 0: pooled-pass mix, kind 1: attention step (mode 0..4, see above).
// d: 64 or 128. waves_per_simd: 1..6 (pool), 1..3 (attention; at most 2 at
// d = 128 except for mode 2); the grid is
// 256 * waves_per_simd workgroups of four wavefronts, so that each of the
// 1024 SIMDs holds that many. out: at least 256 * 256 * waves_per_simd floats.
// Returns 0, 1 for an invalid argument, 4 for a launch error.
extern "C" int kascade_probe_mix(int kind, int mode, int d, int waves_per_simd, int iters, float* out,
                                 void* stream) {
  if (!out || iters < 1 || (d != 64 && d != 128) || waves_per_simd < 1 || waves_per_simd > 6) return 1;
  if (kind == 1 && (mode < 0 || mode > 4 || waves_per_simd > 3)) return 1;
  // At d = 128 the modes that hold a step of operands ahead need 170-200
  // VGPRs: at most two wavefronts per SIMD.
  if (kind == 1 && d == 128 && mode != 2 && waves_per_simd > 2) return 1;
  const int blocks = 256 * waves_per_simd;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (kind == 0) {
    if (d == 128) hipLaunchKernelGGL((pool_mix<4>), dim3(blocks), dim3(256), 0, s, out, iters, 0.1f);
    else hipLaunchKernelGGL((pool_mix<2>), dim3(blocks), dim3(256), 0, s, out, iters, 0.1f);
    e = hipGetLastError();
  } else if (kind == 1) {
#define MIX(M)                                                                                 \
  e = d == 128 ? launch_attn_mix<M, 128>(waves_per_simd, blocks, out, iters, s)              \
               : launch_attn_mix<M, 64>(waves_per_simd, blocks, out, iters, s)
    if (mode == 0) MIX(0); else if (mode == 1) MIX(1); else if (mode == 2) MIX(2); else if (mode == 3) MIX(3);
    else MIX(4);
#undef MIX
  } else {
    return 1;
  }
  return e == hipSuccess ? 0 : 4;
}
