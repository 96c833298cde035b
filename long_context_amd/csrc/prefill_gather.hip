// Reuse-layer causal prefill attention on gfx950, gathered rows staged
// straight into LDS (bf16 inputs, fp32 accumulation).
//
// A reuse layer attends, for each query row i of tile t, only to the keys j of
// the tile's saved index list with j <= i: softmax restricted to those keys,
// values from the layer's own K and V (Kascade, euno.news summary,
// "Methodology" steps 3 and 6: one index set per query tile, reused by the
// following layers).
//
// Work: one workgroup per (query tile, NH heads of one KV group), WAVES
// wavefronts of 32 query rows sharing every staged chunk of the list's K and V
// rows.
//
// Staging: the list is consumed in chunks of KC entries. Each wavefront copies
// every chunk's entries into LDS slots of its own (direct 4-byte loads), six
// chunks ahead, and three chunks ahead gathers its KC / WAVES rows of the
// chunk's K and V straight into a ring of four LDS buffers (direct 16-byte
// loads, unpadded rows, swizzled 16-byte slots). The loads are issued
// from inline assembly and awaited with explicit vmcnt counts; they complete in
// issue order, so the wait for a chunk's rows also covers the entries the next
// rows need. No gathered byte passes through registers.
//
// Masking: only chunks that hold a key some row of the wavefront must not see,
// or that run past the list, compare keys per score.
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16): lane l serves query row
// (l % 32), lane half hf = l / 32.
//   S^T[key, row] = K[key, :] . Q^T[:, row]: A operand key (l % 32) with d
//   slice 16c + 8hf, B operand (resident Q) row l % 32, same slice; element i of
//   the result is key 8(i/4) + 4hf + (i%4) of the step for the lane's row.
//   O^T[d, row] += V^T[d, keys] . P^T[keys, row]: the B operand of 16-key half
//   s2 is the lane's own probabilities 8s2 .. 8s2+7; the A operand supplies V
//   at the matching keys, read from LDS transposed.
#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_stage.hpp"

namespace kascade {

namespace {

constexpr float kGatherRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

// WAVES wavefronts of 32 rows per workgroup, KC list entries per chunk.
template <int D, int TR, int WAVES, int KC>
__global__ __launch_bounds__(64 * WAVES) void prefill_reuse_ring(PrefillArgs a) {
  constexpr int C = D / 16;           // 16-element contraction chunks of S^T
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int ROWB = 2 * D;         // bytes per row
  constexpr int SLOTS = ROWB / 16;    // 16-byte slots per row
  constexpr int SPC = KC / 32;        // 32-key steps per chunk
  constexpr int NB = 4;               // K/V chunk buffers
  constexpr int KS = 8;               // list-entry slots per wavefront
  constexpr int CB = KC * ROWB;       // bytes of one chunk of K (or of V)
  constexpr int RPI = 1024 / ROWB;    // rows per 1-KB direct load
  constexpr int NI = KC / RPI / WAVES;  // 1-KB loads per wavefront, tensor and chunk
  constexpr int RB = TR / 32;         // wavefronts per head
  constexpr int NH = WAVES / RB;      // heads per workgroup
  constexpr int QB = NH * TR * ROWB;  // bytes of the workgroup's query rows
  constexpr int QI = QB / 1024 / WAVES;  // 1-KB query loads per wavefront
  static_assert((NB & (NB - 1)) == 0 && (KS & (KS - 1)) == 0, "ring sizes are powers of two");
  static_assert(QB == 4 * CB && NI >= 1 && QI >= 1 && QI < 64 && 4 * NI + 2 < 64 && KC % 32 == 0 && KC <= 64,
                "staging shape");
  __shared__ __attribute__((aligned(1024))) unsigned char ks[NB][CB];
  __shared__ __attribute__((aligned(1024))) unsigned char vs[NB][CB];
  // Entry slots hold 64 entries (one per lane of a copy), of which the chunk's
  // KC are used; a spare slot takes the padding loads.
  __shared__ __attribute__((aligned(16))) int keys_w[WAVES][KS + 1][64];

  // Longest tiles first across all heads and batches; consecutive workgroups
  // (dealt to the XCDs in turn) keep a KV group's head blocks on one XCD.
  const int units = a.batch * (a.hq / NH);
  const int wtiles = (a.n + TR - 1) / TR;
  const int t = wtiles - 1 - (int)blockIdx.x / units;
  const int u = (int)blockIdx.x % units;
  const int kvg = u % (a.batch * a.hkv), member = u / (a.batch * a.hkv);
  const int b = kvg / a.hkv;
  const int h0 = ((kvg % a.hkv) * (a.group / NH) + member) * NH;  // first head of the workgroup
  const int kvh = h0 / a.group;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int col = lane & 31, hf = lane >> 5;
  const int rb = w % RB, hh_w = w / RB;  // row block, head of the workgroup
  const int row0 = t * TR;
  const int wrow0 = row0 + 32 * rb;
  const int my_row = wrow0 + col;
  const int prefix = min(row0 + TR, a.n);
  const float sl2 = a.scale_log2;

  const u16* kb = a.k + (size_t)(b * a.hkv + kvh) * a.n * D;
  const u16* vb = a.v + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int set = a.idx_sets == 1 ? 0 : kvh;
  const int32_t* list = a.idx + ((size_t)(b * a.idx_sets + set) * a.tiles + t) * a.topk;
  const int list_len = min(a.topk, prefix);  // >= 1
  const int nchunks = (list_len + KC - 1) / KC;
  const int nsteps = (list_len + 31) / 32;

  // The workgroup's query rows (and at the end its output rows) are staged in
  // buffers 2 and 3 of K and of V: head hh, row r at byte (hh * TR + r) * ROWB,
  // slot s at s ^ swz(r).
  auto stage_at = [&](int off) __attribute__((always_inline)) -> unsigned char* {
    return off < 2 * CB ? &ks[2][0] + off : &vs[2][0] + (off - 2 * CB);
  };

  // ---- loads ------------------------------------------------------------------
  // Entries of chunk x: lane l copies position x * KC + l (positions past the
  // list repeat its last entry; the masks know the list length).
  auto issue_keys = [&](int x) __attribute__((always_inline)) {
    const int pos = min(x * KC + lane, list_len - 1);
    lds_dma4_at(list, (unsigned)pos * 4u, lds_address(&keys_w[w][x & (KS - 1)][0]));
  };
  auto issue_pad = [&]() __attribute__((always_inline)) {
    lds_dma4_at(list, 0u, lds_address(&keys_w[w][KS][0]));
  };
  // Rows of chunk x: load j of this wavefront fills chunk rows
  // (w * NI + j) * RPI + lane / SLOTS, stored slot lane % SLOTS, which holds
  // slot (lane % SLOTS) ^ swz(row) of the row's key. Entries outside the list
  // or the sequence load row 0 (masked).
  unsigned slot_off[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int r16 = ((w * NI + j) * RPI + lane / SLOTS) & 15;
    slot_off[j] = 16u * (unsigned)((lane % SLOTS) ^ swz<D>(r16));
  }
  auto row_offsets = [&](int x, unsigned (&off)[NI]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int rho = (w * NI + j) * RPI + lane / SLOTS;
      const int key = keys_w[w][x & (KS - 1)][rho];
      const bool ok = x * KC + rho < list_len && (unsigned)key < (unsigned)a.n;
      off[j] = (ok ? (unsigned)key * (unsigned)ROWB : 0u) + slot_off[j];
    }
  };
  auto issue_rows = [&](int x, const unsigned (&off)[NI]) __attribute__((always_inline)) {
    const int buf = x & (NB - 1);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      lds_dma16_at(kb, off[j], lds_address(&ks[buf][(w * NI + j) * 1024]));
      lds_dma16_at(vb, off[j], lds_address(&vs[buf][(w * NI + j) * 1024]));
    }
  };
  // A chunk needs masks when it runs past the list or holds a key that some
  // row of this wavefront must not see (above its first row, or outside the
  // sequence: unsigned compare).
  auto chunk_masked = [&](int x) __attribute__((always_inline)) -> bool {
    const int key = keys_w[w][x & (KS - 1)][lane];
    return (x + 1) * KC > list_len || __any(lane < KC && (unsigned)key > (unsigned)wrow0);
  };

  // Each wait is a count of loads issued after the ones awaited. Every advance
  // issues one chunk's entries and one chunk's rows (past the list: the last
  // entry again and row 0, cache hits into released slots), and the prologue
  // pads with one-load copies into a spare slot, so every count is a
  // compile-time constant:
  //   keys(0..5), Q, rows(0), pad, rows(1) | pad, rows(2) | advance(0):
  //   keys(6), rows(3) | advance(1): keys(7), rows(4) | ...
  // advance(y) waits for rows(y) with 2 + 4 NI loads issued after it.
  constexpr int kAfterRows = 2 + 4 * NI;
#pragma unroll
  for (int x = 0; x < 6; ++x) issue_keys(x);
  {
    // Query rows into the stage; rows past the sequence repeat its last row.
    const u16* qb = a.q + ((size_t)(b * a.hq + h0) * a.n + row0) * D;
    const int last = a.n - 1 - row0;
#pragma unroll
    for (int jq = 0; jq < QI; ++jq) {
      const unsigned o = (unsigned)(w * QI + jq) * 1024u + 16u * (unsigned)lane;
      const unsigned hh = o / (TR * ROWB), r = (o % (TR * ROWB)) / ROWB, p = (o % ROWB) / 16;
      const unsigned off = (hh * (unsigned)a.n + (unsigned)min((int)r, last)) * (unsigned)ROWB +
                           16u * (p ^ (unsigned)swz<D>((int)r));
      lds_dma16_at_nt(qb, off, lds_address(stage_at((int)(o & ~1023u))));
    }
  }
  wait_vm(QI);  // the entries of chunks 0..5 are in place
  unsigned off[NI];
  row_offsets(0, off);
  issue_rows(0, off);
  issue_pad();
  row_offsets(1, off);
  issue_rows(1, off);
  wait_vm(4 * NI + 1);  // the query rows
  __syncthreads();      // ... are in place for every wavefront

  bf16x8 bq[C];
  {
    const int r = 32 * rb + col;
    const int sw = swz<D>(r);
    const unsigned char* qrow = stage_at((hh_w * TR + r) * ROWB);
#pragma unroll
    for (int c = 0; c < C; ++c) bq[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ((2 * c + hf) ^ sw));
  }
  __syncthreads();  // the stage is free: buffers 2 and 3 take chunks 2 and 3
  issue_pad();
  row_offsets(2, off);
  issue_rows(2, off);

  // Chunk y's rows are in place for every wavefront and chunk y - 1 is
  // released; chunk y + 3 goes into chunk y - 1's buffer. Returns chunk y's
  // mask flag.
  auto advance = [&](int y) __attribute__((always_inline)) -> bool {
    wait_vm(kAfterRows);
    unsigned offn[NI];
    row_offsets(y + 3, offn);
    const bool masked = chunk_masked(y);
    __syncthreads();
    issue_keys(y + 6);
    issue_rows(y + 3, offn);
    return masked;
  };

  // ---- operands and the step ------------------------------------------------------
  const int kswz = swz<D>(col & 15);
  auto read_k = [&](int buf, int sub, bf16x8 (&kf)[C]) __attribute__((always_inline)) {
    const unsigned char* krow = &ks[buf][(32 * sub + col) * ROWB];
#pragma unroll
    for (int c = 0; c < C; ++c) kf[c] = *reinterpret_cast<const bf16x8*>(krow + 16 * ((2 * c + hf) ^ kswz));
  };
  // V^T operand of d block db and 16-key half s2: lane group g = l/16 reads,
  // for d = 32db + 16(g%2) + (l%16), keys 16s2 + 4hf + 0..3 and 16s2 + 8 + 4hf
  // + 0..3 of the step (two transposed reads, each swizzle a lane constant).
  const int vL = lane & 15, vg = lane >> 4;
  const int vrow = 4 * (vg >> 1) + (vL >> 2);
  const int vslot = 2 * (vg & 1) + ((vL & 3) >> 1);
  const int vswz0 = swz<D>(vrow), vswz1 = swz<D>(vrow + 8);
  auto read_v = [&](int buf, int sub, bf16x8 (&vf)[DB][2]) __attribute__((always_inline)) {
    const unsigned char* v0 = &vs[buf][(32 * sub + vrow) * ROWB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int off0 = 16 * ((vslot + 4 * db) ^ vswz0) + 8 * (vL & 1);
      const int off1 = 16 * ((vslot + 4 * db) ^ vswz1) + 8 * (vL & 1);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const lds_bf16x4 lo = lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2) * ROWB + off0));
        const lds_bf16x4 hi = lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2 + 8) * ROWB + off1));
        vf[db][s2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  // Masked steps: scores of keys the lane's row must not see (above the row,
  // outside the sequence, or past the list) become -inf. Element i of the
  // scores is key 8(i/4) + 4hf + (i%4) of the step.
  auto apply_mask = [&](int j, f32x16& s) __attribute__((always_inline)) {
    const int c = j / SPC, sub = j % SPC;
    const int lim = list_len - c * KC;
    const int* kr = &keys_w[w][c & (KS - 1)][32 * sub + 4 * hf];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int4 k4 = *reinterpret_cast<const int4*>(kr + 8 * q);
      const int kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 32 * sub + 8 * q + 4 * hf + r < lim ? kv[r] : -1;
        if ((unsigned)key > (unsigned)my_row) s[4 * q + r] = -INFINITY;
      }
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = zero_f32x16();
  float m = kNegBig, l = 0.f;
  bf16x8 kf[C], vf[DB][2], pb[2];
#pragma unroll
  for (int i = 0; i < DB; ++i) vf[i][0] = vf[i][1] = zero_bf16x8();
  pb[0] = pb[1] = zero_bf16x8();
  auto pv = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) acc[db] = mfma32x32x16(vf[db][s2], pb[s2], acc[db]);
  };

  bool masked = advance(0);  // chunk 0
  read_k(0, 0, kf);
  for (int j = 0; j < nsteps; ++j) {
    const int c = j / SPC, sub = j % SPC, buf = c & (NB - 1);
    pv();  // step j - 1 (nothing at j = 0)
    read_v(buf, sub, vf);
    f32x16 s = zero_f32x16();
#pragma unroll
    for (int cc = 0; cc < C; ++cc) s = mfma32x32x16(kf[cc], bq[cc], s);
    if (masked) apply_mask(j, s);
    // Step j + 1: its chunk and K operands, during this step's softmax (past
    // the last step, K of ring rows that are not used).
    const int jn = j + 1;
    if (sub == SPC - 1 && c + 1 < nchunks) masked = advance(c + 1);
    read_k((jn / SPC) & (NB - 1), jn % SPC, kf);

    float cmax = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, s[i]);
    {
      float lo_, hi_;
      pair32(cmax, lo_, hi_);
      cmax = fmaxf(lo_, hi_) * sl2;
    }
    // Lazy rescaling: the reference maximum moves only when some row's maximum
    // grew by more than 2^8, so probabilities stay below 256.
    float alpha = 1.0f;
    const bool rescale = __any(cmax > m + kGatherRescaleLog2);
    if (rescale) {
      const float mnew = fmaxf(m, cmax);
      alpha = fast_exp2(m - mnew);
      m = mnew;
      // The accumulators are scaled here rather than after the probabilities:
      // a second branch on the same condition makes the register allocator
      // give them two homes and copy them between the two every step.
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
    }
    const float neg_m = -m;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(fmaf(s[i], sl2, neg_m));
      lsum += s[i];
    }
    l = l * alpha + lsum;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f32x4 p0 = {s[8 * s2 + 0], s[8 * s2 + 1], s[8 * s2 + 2], s[8 * s2 + 3]};
      const f32x4 p1 = {s[8 * s2 + 4], s[8 * s2 + 5], s[8 * s2 + 6], s[8 * s2 + 7]};
      pb[s2] = pack_bf16x8(p0, p1);
    }
  }
  pv();  // the last step

  // ---- output: normalised rows through the stage, out in 1-KB pieces ------------
  float lo_, hi_;
  pair32(l, lo_, hi_);
  const float inv = lo_ + hi_ > 0.f ? 1.0f / (lo_ + hi_) : 0.f;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load left in flight
  __syncthreads();                     // every wavefront is done with the ring
  {
    const int r = 32 * rb + col;
    const int sw = swz<D>(r);
    unsigned char* orow = stage_at((hh_w * TR + r) * ROWB);
    // acc[db] element i is d = 32db + 8(i/4) + 4hf + (i%4) of this row.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u16 o4[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o4[rr] = float_to_bf16_bits(acc[db][4 * q + rr] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * ((4 * db + q) ^ sw) + 8 * hf) =
            make_uint2(o4[0] | (uint32_t(o4[1]) << 16), o4[2] | (uint32_t(o4[3]) << 16));
      }
  }
  __syncthreads();
  // Head hh's rows are contiguous from the workgroup's first: one uniform base,
  // 32-bit lane offsets.
  unsigned char* ob = reinterpret_cast<unsigned char*>(a.out + ((size_t)(b * a.hq + h0) * a.n + row0) * D);
#pragma unroll
  for (int jq = 0; jq < QI; ++jq) {
    const unsigned o = (unsigned)(w * QI + jq) * 1024u + 16u * (unsigned)lane;
    const unsigned hh = o / (TR * ROWB), r = (o % (TR * ROWB)) / ROWB, p = (o % ROWB) / 16;
    if (row0 + (int)r < a.n) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(stage_at((int)o));  // eight bf16, moved as bits
      const unsigned off = (hh * (unsigned)a.n + r) * (unsigned)ROWB + 16u * (p ^ (unsigned)swz<D>((int)r));
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(ob + off));
    }
  }
}

}  // namespace

// Four wavefronts and 32-entry chunks: 73 KB of LDS (d = 128), so two
// workgroups share a compute unit and overlap each other's prologue, barriers
// and softmax phases. Measured at the 8K / 32K workloads (d 128 / 64): 157-158
// / 1493 us, against 157 / 1740 us with eight wavefronts and 64-entry chunks
// (one workgroup per unit) and 170 / 1733 us for the register-staged gather.
constexpr int kRingWaves = 4;
constexpr int kRingChunk = 32;

// Heads per workgroup of the ring kernel for a selection tile.
static int ring_heads(int tile) { return kRingWaves / (tile / 32); }

bool prefill_reuse_ring_supported(const PrefillArgs& a) {
  if ((a.d != 128 && a.d != 64) || (a.tile != 128 && a.tile != 64)) return false;
  const int nh = ring_heads(a.tile);
  if (a.group % nh != 0) return false;
  // Row offsets are 32-bit: the workgroup's query rows and a KV head's rows.
  const size_t rowb = (size_t)a.d * 2;
  return (size_t)nh * a.n * rowb < (1ull << 31) && (size_t)a.n * rowb < (1ull << 31);
}

hipError_t launch_prefill_reuse_ring(const PrefillArgs& a, hipStream_t s) {
  if (!prefill_reuse_ring_supported(a)) return hipErrorInvalidValue;
  const int nh = ring_heads(a.tile);
  const int wtiles = (a.n + a.tile - 1) / a.tile;
  constexpr int W = kRingWaves, KC = kRingChunk;
  dim3 grid(wtiles * a.batch * (a.hq / nh)), block(64 * W);
  if (a.tile == 128 && a.d == 128) hipLaunchKernelGGL((prefill_reuse_ring<128, 128, W, KC>), grid, block, 0, s, a);
  else if (a.tile == 128 && a.d == 64) hipLaunchKernelGGL((prefill_reuse_ring<64, 128, W, KC>), grid, block, 0, s, a);
  else if (a.tile == 64 && a.d == 128) hipLaunchKernelGGL((prefill_reuse_ring<128, 64, W, KC>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((prefill_reuse_ring<64, 64, W, KC>), grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace kascade
