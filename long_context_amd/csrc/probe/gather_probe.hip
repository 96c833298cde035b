// Measurement probe (not part of the attention path): the memory ceiling of
// the decode reuse layer's access pattern. A load-only kernel reads the K and V
// rows named by an index list -- the reuse gather's bytes, without its
// arithmetic -- or the same number of rows read contiguously, so the achieved
// rate can be set against the reuse kernel's. Used by bench.py --probe.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Unit u = blockIdx.y (a (batch, KV head) segment of n rows of ROWB bytes);
// wavefront w of the unit's `splits` reads list entries
// [w * per, (w + 1) * per) of the unit's list (or rows w*per .. when
// contiguous), 16 bytes per lane, ROWB / 16 lanes per row, INF row groups of
// K and V in flight. The loaded words are folded into one value per lane and
// written to `sink` only when it equals one arbitrary constant (rare, and in
// bounds either way), so the compiler has to keep every load.
template <int ROWB, int INF, bool CONTIG>
__global__ __launch_bounds__(256) void gather_load(const unsigned char* k, const unsigned char* v,
                                                   const int32_t* idx, int n, int len, int splits, int per,
                                                   unsigned* sink) {
  constexpr int LPR = ROWB / 16;       // lanes per row
  constexpr int RPI = 64 / LPR;        // rows per instruction
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= splits) return;
  const int unit = blockIdx.y;
  const int begin = w * per, end = min(begin + per, len);
  const size_t base = (size_t)unit * n * ROWB;
  const int32_t* list = idx + (size_t)unit * len;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int e0 = begin; e0 < end; e0 += RPI * INF) {
    u32x4 kr[INF], vr[INF];
#pragma unroll
    for (int i = 0; i < INF; ++i) {
      const int e = e0 + i * RPI + lane / LPR;
      int row = 0;
      if (e < end) row = CONTIG ? e : list[e];
      if (row < 0 || row >= n) row = 0;  // padding or out-of-range entries read row 0
      const size_t off = base + (size_t)row * ROWB + (lane % LPR) * 16;
      kr[i] = *reinterpret_cast<const u32x4*>(k + off);
      vr[i] = *reinterpret_cast<const u32x4*>(v + off);
    }
#pragma unroll
    for (int i = 0; i < INF; ++i) acc ^= kr[i] ^ vr[i];
  }
  const unsigned x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (x == 0x7fc00001u) sink[w] = x;
}

}  // namespace

// bytes of one row: 256 (d = 128 bf16). inflight: row groups in flight per
// wavefront (1, 2, 4 or 8). contiguous != 0 reads rows 0 .. len-1 of each unit.
// sink: at least `splits` words. Returns 0, 1 for an invalid argument, 4 for
// a launch error.
extern "C" int kascade_probe_gather(const void* k, const void* v, const int32_t* idx, int units, int n,
                                    int len, int splits, int inflight, int contiguous, unsigned* sink,
                                    void* stream) {
  if (units < 1 || n < 1 || len < 1 || len > n || splits < 1 || !k || !v || !sink || (!contiguous && !idx))
    return 1;
  const int per = (len + splits - 1) / splits;
  const dim3 grid((splits + 3) / 4, units), block(256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned char* kb = static_cast<const unsigned char*>(k);
  const unsigned char* vb = static_cast<const unsigned char*>(v);
#define PROBE(I, C) hipLaunchKernelGGL((gather_load<256, I, C>), grid, block, 0, s, kb, vb, idx, n, len, splits, per, sink)
  if (contiguous) {
    if (inflight == 1) PROBE(1, true); else if (inflight == 2) PROBE(2, true);
    else if (inflight == 4) PROBE(4, true); else if (inflight == 8) PROBE(8, true); else return 1;
  } else {
    if (inflight == 1) PROBE(1, false); else if (inflight == 2) PROBE(2, false);
    else if (inflight == 4) PROBE(4, false); else if (inflight == 8) PROBE(8, false); else return 1;
  }
#undef PROBE
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
