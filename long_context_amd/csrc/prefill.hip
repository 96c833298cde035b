// Causal prefill kernels for gfx950 (bf16 inputs, fp32 accumulation).
//
// prefill_attn: flash-style causal attention of one query tile of one head
// over a key list. Dense mode (anchor pass 1) walks keys 0..prefix_t-1 and
// writes the per-row log-sum-exp (and, on request, the dense output); gather
// mode (reuse layer; the fallback of prefill_reuse_ring for the shapes that
// kernel does not take) walks the tile's saved index list, softmax restricted
// to the saved keys j <= i (Kascade, euno.news summary, "Methodology" steps 3
// and 6: one index set per query tile, values recomputed with the layer's own
// tensors).
//   Per chunk the workgroup stages K and V rows in LDS (gathered rows are
//   fetched 16 bytes per lane, 16 lanes per 256-byte row). Each wave owns 32
//   query rows and computes S^T = K . Q^T on the matrix cores, so a row's
//   scores live in two lanes (l and l ^ 32: one cross-lane exchange per
//   32-key step), and O^T += V^T . P^T with P^T taken straight from the S^T
//   accumulators. V^T operands are read from LDS transposed.
//
// prefill_pool: anchor pass 2. For tile t and key j < prefix_t:
//   pooled[t, j] = sum over the group's heads and the tile's rows i >= j of
//                  exp2(x_ij - lse2_i)
// i.e. the post-softmax probabilities summed over the tile (the sum ranks
// keys as the mean does). The row log-sum-exp must be final before any term
// is added, so the scores are recomputed rather than stored. Each wave keeps
// 64 keys of K resident as matrix-core operands and streams the group's query
// rows of the tile through a two-slot LDS ring of 64-row units; column sums
// are lane-local until one final cross-lane step.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"
#include "lds_stage.hpp"

namespace kascade {

namespace {

constexpr int kRowsPerWave = 32;   // query rows per wavefront in prefill_attn
constexpr int kTile = 128;         // dense-pass work tile: four wavefronts of 32 rows
constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)

// KC keys are staged per pipeline step (64 or 128).
//
// Matrix-core layout (v_mfma_f32_32x32x16_bf16). A wavefront owns 32 query
// rows; lane l serves row wrow0 + (l % 32) and lane half hf = l / 32.
//   S^T[key, row] += K[key, d-chunk] . Q^T[d-chunk, row]: the A operand is
//   key (kb0 + l%32) with d slice 16c + 8hf; the B operand (Q, resident) is
//   row l%32 with the same slice. Lane l receives its row's scores for keys
//   kb0 + 8(i/4) + 4hf + (i%4), i = 0..15, so a row's maximum is lane-local
//   plus one exchange with lane l^32.
//   O^T[d, row] += V^T[d, keys] . P^T[keys, row], 16 keys per step ks: the
//   B operand takes the lane's own probabilities i = 8ks .. 8ks+7, so slot j of
//   half hf stands for key 16ks + 8(j/4) + 4hf + (j%4); the A operand supplies
//   V at those keys for d = 32db + l%32, two transposed LDS reads of four
//   consecutive keys each.

// TR query rows per workgroup and head (the selection tile in gather mode;
// kTile in the dense pass), TR / 32 wavefronts per head, NH heads, key chunks
// of KC keys.
//   Dense pass: the chunk's rows go straight from HBM into a ring of NB LDS
//   buffers (unpadded rows, 16-byte slots swizzled), chunk c + NB - 1 loading
//   while chunk c is used.
//   Gather (reuse layers whose shape the LDS-ring kernel of prefill_gather.hip
//   does not take): rows go through registers into two LDS buffers, the list
//   entries one chunk ahead of the rows. These rows are padded instead of swizzled,
//   which keeps every operand offset a compile-time constant: K rows by 8
//   elements (an odd number of 16-byte slots per row), V rows by 32 (four
//   consecutive rows start 64 bytes apart modulo a bank sweep).
#ifndef KASCADE_REUSE_STAGE
#define KASCADE_REUSE_STAGE 1
#endif

// d = 64 dense pass: four wavefronts per SIMD (at most 128 VGPRs). Its step is
// bound by vector work, so the extra wavefronts pay; the next step's K
// operands are then read after the P.V (kLateK), where the other wavefronts
// hide their latency, so that the softmax fits in the register budget.
template <int D, bool GATHER>
constexpr int attn_waves_per_simd() { return D == 64 && !GATHER ? 4 : 1; }

template <int D, bool GATHER, bool WITH_O, int NH, int KC, int TR, int NB>
__global__ __launch_bounds__(64 * (TR / kRowsPerWave) * NH)
    __attribute__((amdgpu_waves_per_eu(attn_waves_per_simd<D, GATHER>()))) void prefill_attn(PrefillArgs a) {
  constexpr bool DMA = !GATHER;
  constexpr bool kLateK = attn_waves_per_simd<D, GATHER>() > 1;
  constexpr int kKeyChunk = KC;
  constexpr int kKeyWaves = KC / 64;  // wavefronts that hold the chunk's list entries (gather)
  constexpr int C = D / 16;           // 16-element contraction chunks of S^T
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int ROWB = D * 2;         // bytes per unpadded row
  constexpr int WPH = TR / kRowsPerWave;                 // wavefronts per head
  constexpr int THREADS = 64 * WPH * NH;
  constexpr int WAVES = THREADS / 64;
  constexpr int VPR = D / 8;                             // 16-byte vectors per row
  constexpr int LPT = kKeyChunk * VPR / THREADS;         // vectors per thread per tensor (registers)
  static_assert(LPT >= 1 && kKeyChunk * VPR % THREADS == 0, "chunk must split evenly");
  constexpr int NBUF = DMA ? NB : 2;
  constexpr int KROW_BYTES = DMA ? ROWB : (D + 8) * 2;
  constexpr int VROW_BYTES = DMA ? ROWB : (D + 32) * 2;
  constexpr int NI = KC * ROWB / 1024 / WAVES;           // 1-KB direct loads per wavefront and tensor
  static_assert(!DMA || (NI >= 1 && KC * ROWB % (1024 * WAVES) == 0), "direct loads must split evenly");
  static_assert(KC % 32 == 0 && (!GATHER || KC % 64 == 0) && NB >= 2, "staging shape");
  constexpr int R = NI * (WITH_O ? 2 : 1);               // direct loads per wavefront and chunk
  __shared__ __attribute__((aligned(1024))) unsigned char ks[NBUF][KC * KROW_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vs[WITH_O ? NBUF : 1][WITH_O ? KC * VROW_BYTES : 16];
  __shared__ int keys_s[GATHER ? 2 : 1][GATHER ? kKeyChunk : 1];
  // gather mode, per key-holding wavefront: smallest valid key, largest key, any padding
  __shared__ int info_s[GATHER ? 2 : 1][GATHER ? kKeyWaves : 1][4];

  // Longest tiles first across all heads and batches: workgroup i takes tile
  // tiles-1 - i / (B * Hq/NH) of TR rows, so the dispatcher hands out the work in
  // decreasing length and the last workgroups to start are the shortest.
  // Within a tile, u % (B*Hkv) is the (b, KV head) and u / (B*Hkv) the head
  // block of its group: consecutive workgroups, which the dispatcher deals to
  // the 8 XCDs in turn, keep a KV group's head blocks on one XCD and its L2.
  const int units = a.batch * (a.hq / NH);
  const int wtiles = (a.n + TR - 1) / TR;
  const int t = wtiles - 1 - (int)blockIdx.x / units;
  const int u = (int)blockIdx.x % units;
  const int kvg = u % (a.batch * a.hkv), member = u / (a.batch * a.hkv);
  const int b = kvg / a.hkv;
  const int hb = (kvg % a.hkv) * (a.group / NH) + member;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int h = hb * NH + wave / WPH;
  const int kvh = h / a.group;             // the NH heads of a block share one KV head
  const int col = lane & 31, hf = lane >> 5;
  const int prefix = min((t + 1) * TR, a.n);
  const int wrow0 = t * TR + (wave % WPH) * kRowsPerWave;
  const int wrow_last = min(wrow0 + kRowsPerWave, a.n) - 1;
  const int my_row = wrow0 + col;
  const float sl2 = a.scale_log2;

  const u16* kb = a.k + (size_t)(b * a.hkv + kvh) * a.n * D;
  const u16* vb = a.v + (size_t)(b * a.hkv + kvh) * a.n * D;
  const int set = a.idx_sets == 1 ? 0 : kvh;
  const int32_t* list = GATHER ? a.idx + ((size_t)(b * a.idx_sets + set) * a.tiles + t) * a.topk : nullptr;
  const int list_len = GATHER ? min(a.topk, prefix) : prefix;
  const int nchunks = (list_len + kKeyChunk - 1) / kKeyChunk;

  // Gather mode with an even head count: the block's query rows come in, and
  // its output rows go out, through the second K/V buffer in whole 1-KB
  // pieces (each head's TR rows are contiguous in Q and O), instead of every
  // lane touching 32 rows in 8- or 16-byte pieces per instruction. Heads
  // 0 .. NH/2-1 use the K half of that buffer, the others the V half; 16-byte
  // slot s of row r sits at slot s ^ swz<D>(r). Both streams carry the
  // non-temporal hint: each workgroup's XCD serves one KV head, whose K and V
  // rows fill about its whole L2 and are gathered again by the next tiles.
  // Measured at the 8K workload: 187-188 us unstaged, 179-181 staged,
  // 172-174 staged and non-temporal.
  constexpr int QH = TR * ROWB;  // bytes of one head's tile rows
  constexpr bool STAGE = GATHER && KASCADE_REUSE_STAGE && NH % 2 == 0 && QH % 1024 == 0 &&
                         (NH / 2) * QH <= KC * KROW_BYTES && (NH / 2) * QH <= KC * VROW_BYTES &&
                         (NH * QH) % (1024 * WAVES) == 0;
  constexpr int SQI = STAGE ? NH * QH / 1024 / WAVES : 1;  // 1-KB pieces per wavefront
  auto stage_at = [&](int hh) __attribute__((always_inline)) {
    return (hh < NH / 2 ? &ks[NBUF - 1][0] : &vs[WITH_O ? NBUF - 1 : 0][0]) + (hh % (NH / 2 > 0 ? NH / 2 : 1)) * QH;
  };
  bf16x8 bq[C];
  if constexpr (!STAGE) {
    const u16* qrow = a.q + ((size_t)(b * a.hq + h) * a.n + min(my_row, a.n - 1)) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) bq[c] = load_bf16x8(qrow + 16 * c + 8 * hf);
  }

  float m = kNegBig, l = 0.f;
  f32x16 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = zero_f32x16();

  // ---- register staging (gather): global -> registers -> padded LDS ---------
  bf16x8 kr[DMA ? 1 : LPT], vr[DMA ? 1 : LPT];
  int key_reg = -1;
  auto key_at = [&](int pos) __attribute__((always_inline)) {
    int key = pos < list_len ? (GATHER ? list[pos] : pos) : -1;
    return key < a.n ? key : -1;  // entries outside the sequence are skipped
  };
  // The chunk's list entries are read one fetch ahead (next_keys), so the row
  // loads of a fetch never wait on the list.
  int next_keys[DMA ? 1 : LPT];
  int next_key_reg = -1;
  auto load_keys = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) next_keys[i] = key_at(c * kKeyChunk + (tid + i * THREADS) / VPR);
    if (tid < kKeyChunk) next_key_reg = key_at(c * kKeyChunk + tid);
  };
  auto fetch = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int slot = tid + i * THREADS;
      const int colv = (slot % VPR) * 8;
      const size_t src = (size_t)(next_keys[i] < 0 ? 0 : next_keys[i]) * D + colv;
      kr[i] = load_bf16x8(kb + src);
      if (WITH_O) vr[i] = load_bf16x8(vb + src);
    }
    if (tid < kKeyChunk) key_reg = next_key_reg;
    if ((c + 1) * kKeyChunk < list_len) load_keys(c + 1);
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int slot = tid + i * THREADS;
      const int row = slot / VPR, vec = slot % VPR;
      *reinterpret_cast<bf16x8*>(&ks[buf][row * KROW_BYTES + 16 * vec]) = kr[i];
      if (WITH_O) *reinterpret_cast<bf16x8*>(&vs[buf][row * VROW_BYTES + 16 * vec]) = vr[i];
    }
    if (wave < kKeyWaves) {  // these waves hold the chunk's keys, one per lane
      keys_s[buf][tid] = key_reg;
      int lo = key_reg >= 0 ? key_reg : 0x7fffffff, hi = key_reg;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, __shfl_xor(lo, o));
        hi = max(hi, __shfl_xor(hi, o));
      }
      const bool pad = __any(key_reg < 0);
      if (lane == 0) {
        info_s[buf][wave][0] = lo;
        info_s[buf][wave][1] = hi;
        info_s[buf][wave][2] = pad;
      }
    }
  };

  // ---- direct staging (dense): chunk c into ring buffer c % NB ----------------
  // This wavefront's NI 1-KB loads per tensor: lane l of load j fills row r,
  // stored slot p, which holds slot p ^ swz<D>(r) of key c * KC + r.
  // A chunk whose rows all exist in the sequence loads from the chunk's first
  // row (a scalar base) at lane-constant offsets; only a chunk running past
  // the last row computes per-lane addresses, with those rows replaced by row 0.
  unsigned dma_off[DMA ? NI : 1];
#pragma unroll
  for (int j = 0; j < (DMA ? NI : 1); ++j) {
    const int o = (wave * NI + j) * 1024 + 16 * lane;
    const int r = o / ROWB, p = (o % ROWB) / 16;
    dma_off[j] = (unsigned)(r * D + 8 * (p ^ swz<D>(r))) * 2u;
  }
  auto issue_rows = [&](int c) __attribute__((always_inline)) {
    const int buf = c % NB;
    if ((c + 1) * kKeyChunk <= a.n) {
      const u16* kc = kb + (size_t)c * kKeyChunk * D;
      const u16* vc = vb + (size_t)c * kKeyChunk * D;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        lds_dma16_at(kc, dma_off[j], lds_address(&ks[buf][(wave * NI + j) * 1024]));
        if constexpr (WITH_O) lds_dma16_at(vc, dma_off[j], lds_address(&vs[buf][(wave * NI + j) * 1024]));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int o = (wave * NI + j) * 1024 + 16 * lane;
        const int r = o / ROWB, p = (o % ROWB) / 16;
        const int key = c * kKeyChunk + r;
        const size_t src = (size_t)(key < a.n ? key : 0) * D + 8 * (p ^ swz<D>(r));
        lds_dma16(kb + src, lds_address(&ks[buf][(wave * NI + j) * 1024]));
        if constexpr (WITH_O) lds_dma16(vb + src, lds_address(&vs[buf][(wave * NI + j) * 1024]));
      }
    }
  };

  // ---- one 32-key step of a staged chunk -------------------------------------
  // Operands come from LDS ahead of use: the K fragments of a step are read
  // before the previous step's P.V, and the V^T fragments of a step before its
  // softmax, so LDS latency hides behind matrix-core and ALU work.
  // K operand: row 32sub + col, elements 16c + 8hf (slot 2c + hf; the swizzle
  // of the direct-load layout depends on row % 16 = col % 16).
  const int kswz = swz<D>(col & 15);
  auto read_k = [&](int buf, int sub, bf16x8 (&kf)[C]) __attribute__((always_inline)) {
    const unsigned char* krow = &ks[buf][(32 * sub + col) * KROW_BYTES];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const int off = DMA ? 16 * ((2 * c + hf) ^ kswz) : 32 * c + 16 * hf;
      kf[c] = *reinterpret_cast<const bf16x8*>(krow + off);
    }
  };
  // V^T operand of d block db and key step s2: lane group g = l/16 reads, for
  // d = 32db + 16(g%2) + (l%16), keys 16s2 + 4hf + 0..3 and 16s2 + 8 + 4hf + 0..3
  // (row base + L/4, columns 4(L%4) of the lane's transposed read). Those rows
  // have row % 16 = 4(g/2) + L/4 for the first read and 8 more for the second,
  // so each read's swizzle is a lane constant.
  const int vL = lane & 15, vg = lane >> 4;
  const int vrow = 4 * (vg >> 1) + (vL >> 2);
  const int vslot = 2 * (vg & 1) + ((vL & 3) >> 1);
  const int vswz0 = swz<D>(vrow), vswz1 = swz<D>(vrow + 8);
  auto read_v = [&](int buf, int sub, bf16x8 (&vf)[DB][2]) __attribute__((always_inline)) {
    const unsigned char* v0 = &vs[WITH_O ? buf : 0][(32 * sub + vrow) * VROW_BYTES];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int off0 = DMA ? 16 * ((vslot + 4 * db) ^ vswz0) + 8 * (vL & 1) : 16 * (vslot + 4 * db) + 8 * (vL & 1);
      const int off1 = DMA ? 16 * ((vslot + 4 * db) ^ vswz1) + 8 * (vL & 1) : off0;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const lds_bf16x4 lo =
            lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2) * VROW_BYTES + off0));
        const lds_bf16x4 hi =
            lds_read_transposed(reinterpret_cast<const __bf16*>(v0 + (16 * s2 + 8) * VROW_BYTES + off1));
        vf[db][s2] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
  };
  auto step = [&](int buf, int c, int sub, bool masked, bf16x8 (&kf)[C]) __attribute__((always_inline)) {
    bf16x8 vf[DB][2];
    if constexpr (WITH_O) read_v(buf, sub, vf);
    f32x16 s = zero_f32x16();
#pragma unroll
    for (int cc = 0; cc < C; ++cc) s = mfma32x32x16(kf[cc], bq[cc], s);
    // Next step's K operands: during this softmax, or (kLateK) after this
    // step's P.V, which keeps them out of the softmax's live registers.
    if (!kLateK && sub + 1 < KC / 32) read_k(buf, sub + 1, kf);
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 32 * sub + 8 * (i >> 2) + 4 * hf + (i & 3);  // key slot in the chunk
        const int key = GATHER ? keys_s[buf][kk] : (c * kKeyChunk + kk < list_len ? c * kKeyChunk + kk : -1);
        if (key < 0 || key > my_row) s[i] = -INFINITY;
      }
    }
    float cmax = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) cmax = fmaxf(cmax, s[i]);
    {
      float lo_, hi_;
      pair32(cmax, lo_, hi_);
      cmax = fmaxf(lo_, hi_) * sl2;
    }
    // Lazy rescaling: keep the reference maximum unless some row's maximum
    // grew by more than 2^8; probabilities then stay below 256 in fp32.
    float alpha = 1.0f;
    const bool rescale = __any(cmax > m + kRescaleLog2);
    if (rescale) {
      const float mnew = fmaxf(m, cmax);
      alpha = fast_exp2(m - mnew);
      m = mnew;
      // The accumulators are scaled here rather than after the probabilities:
      // a second branch on the same condition can make the register allocator
      // give them two homes and copy them between the two every step.
      if constexpr (WITH_O) {
#pragma unroll
        for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      }
    }
    const float neg_m = -m;
    float lsum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s[i] = fast_exp2(fmaf(s[i], sl2, neg_m));
      lsum += s[i];
    }
    l = l * alpha + lsum;
    if constexpr (WITH_O) {
      bf16x8 pb[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        f32x4 p0 = {s[8 * s2 + 0], s[8 * s2 + 1], s[8 * s2 + 2], s[8 * s2 + 3]};
        f32x4 p1 = {s[8 * s2 + 4], s[8 * s2 + 5], s[8 * s2 + 6], s[8 * s2 + 7]};
        pb[s2] = pack_bf16x8(p0, p1);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) acc[db] = mfma32x32x16(vf[db][s2], pb[s2], acc[db]);
    }
    if (kLateK && sub + 1 < KC / 32) read_k(buf, sub + 1, kf);
  };
  auto chunk_step = [&](int buf, int c, bool masked) __attribute__((always_inline)) {
    bf16x8 kf[C];
    read_k(buf, 0, kf);
#pragma unroll 1
    for (int sub = 0; sub < KC / 32; ++sub) step(buf, c, sub, masked, kf);
  };

  if constexpr (DMA) {
    // Per wavefront the direct loads are counted as issued; before chunk c is
    // used, s_waitcnt vmcnt(issued - rows_q[0]) leaves only later chunks' loads
    // in flight. rows_q[i] is the count right after chunk c + i's loads.
    // Chunks past the end issue no loads, so the count is tracked rather than
    // assumed. The Q operand loads complete at the first vmcnt(0).
    __builtin_amdgcn_s_waitcnt(0x0F70);
    int issued = 0;
    int rows_q[NB - 1];
#pragma unroll
    for (int c = 0; c < NB - 1; ++c) {
      if (c < nchunks) {
        issue_rows(c);
        issued += R;
      }
      rows_q[c] = issued;
    }
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c % NB;
      wait_vm(issued - rows_q[0]);
      __syncthreads();  // chunk c is in place; chunk c - 1's buffer is released
      const int nc = c + NB - 1;
      if (nc < nchunks) {
        issue_rows(nc);
        issued += R;
      }
#pragma unroll
      for (int i = 0; i + 1 < NB - 1; ++i) rows_q[i] = rows_q[i + 1];
      rows_q[NB - 2] = issued;
      if (wrow0 < a.n) {
        const int vmin = c * kKeyChunk;
        const int vmax = min(vmin + kKeyChunk, list_len) - 1;
        const bool pad = vmin + kKeyChunk > list_len;
        if (vmin <= wrow_last)  // otherwise every key is above every row of the wave
          chunk_step(buf, c, pad || vmax > wrow0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no load left in flight at exit
  } else {
    if constexpr (STAGE) {
      // The block's query rows into the stage: piece B of the block holds
      // head B / (QH / 1024); rows past the sequence repeat its last row.
      const int row0 = t * TR;
      const int last = a.n - 1 - row0;
      const u16* qb = a.q + ((size_t)(b * a.hq + hb * NH) * a.n + row0) * D;
#pragma unroll
      for (int j = 0; j < SQI; ++j) {
        const int B = wave * SQI + j;
        const int hh = B / (QH / 1024), o = (B % (QH / 1024)) * 1024 + 16 * lane;
        const int r = o / ROWB, p = (o % ROWB) / 16;
        const unsigned off = (unsigned)(((size_t)hh * a.n + min(r, last)) * ROWB) + 16u * (unsigned)(p ^ swz<D>(r));
        lds_dma16_at_nt(qb, off, lds_address(stage_at(hh) + (B % (QH / 1024)) * 1024));
      }
    }
    // list_len >= 1 (k >= 1 and prefix_t >= 1), so chunk 0 always exists.
    load_keys(0);
    fetch(0);
    stash(0);
    // Complete the Q operand loads here: a wait for them inside the loop would
    // also wait for the prefetch of the next chunk (vector-memory counts retire
    // in order). s_waitcnt vmcnt(0), other counters unconstrained.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    if constexpr (STAGE) {
      const int r = (wave % WPH) * kRowsPerWave + col;
      const unsigned char* qrow = stage_at(wave / WPH) + r * ROWB;
      const int sw = swz<D>(r);
#pragma unroll
      for (int c = 0; c < C; ++c) bq[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ((2 * c + hf) ^ sw));
      __syncthreads();  // the stage is chunk 1's buffer from here on
    }
    if (nchunks > 1) fetch(1);
    for (int c = 0; c < nchunks; ++c) {
      const int buf = c & 1;
      if (wrow0 < a.n) {
        int vmin = info_s[buf][0][0], vmax = info_s[buf][0][1];
        bool pad = info_s[buf][0][2] != 0;
#pragma unroll
        for (int w = 1; w < kKeyWaves; ++w) {
          vmin = min(vmin, info_s[buf][w][0]);
          vmax = max(vmax, info_s[buf][w][1]);
          pad = pad || info_s[buf][w][2] != 0;
        }
        if (vmin <= wrow_last)  // otherwise every key is above every row of the wave
          chunk_step(buf, c, pad || vmax > wrow0);
      }
      if (c + 1 < nchunks) stash(buf ^ 1);  // that buffer was released at the last barrier
      __syncthreads();
      if (c + 2 < nchunks) fetch(c + 2);
    }
  }

  // Row totals: each lane half summed its own keys.
  float lo_, hi_;
  pair32(l, lo_, hi_);
  const float lt = lo_ + hi_;
  if constexpr (STAGE) {
    // Every buffer is free after the loop's last barrier: the normalised rows
    // go to the stage, then out in whole 1-KB pieces.
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    {
      const int r = (wave % WPH) * kRowsPerWave + col;
      unsigned char* orow_s = stage_at(wave / WPH) + r * ROWB;
      const int sw = swz<D>(r);
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u16 o4[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) o4[rr] = float_to_bf16_bits(acc[db][4 * q + rr] * inv);
          *reinterpret_cast<uint2*>(orow_s + 16 * ((4 * db + q) ^ sw) + 8 * hf) =
              make_uint2(o4[0] | (uint32_t(o4[1]) << 16), o4[2] | (uint32_t(o4[3]) << 16));
        }
    }
    __syncthreads();
    const int row0 = t * TR;
#pragma unroll
    for (int j = 0; j < SQI; ++j) {
      const int B = wave * SQI + j;
      const int hh = B / (QH / 1024), o = (B % (QH / 1024)) * 1024 + 16 * lane;
      const int r = o / ROWB, p = (o % ROWB) / 16;
      if (row0 + r < a.n) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(stage_at(hh) + o);  // eight bf16, moved as bits
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(a.out + ((size_t)(b * a.hq + hb * NH + hh) * a.n + row0 + r) * D +
                                                                8 * (p ^ swz<D>(r))));
      }
    }
    return;
  }
  if (my_row < a.n) {
    const size_t orow = (size_t)(b * a.hq + h) * a.n + my_row;
    if (!GATHER && hf == 0) a.lse2[orow] = m + log2f(lt);
    if constexpr (WITH_O) {
      // acc[db] element i is d = 32db + 8(i/4) + 4hf + (i%4) of this row.
      const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u16 o4[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) o4[r] = float_to_bf16_bits(acc[db][4 * q + r] * inv);
          *reinterpret_cast<uint2*>(a.out + orow * D + 32 * db + 8 * q + 4 * hf) =
              make_uint2(o4[0] | (uint32_t(o4[1]) << 16), o4[2] | (uint32_t(o4[3]) << 16));
        }
    }
  }
}

// ---- anchor pass 2: pooled post-softmax probabilities per query tile ---------

constexpr int kPoolWaves = 4;
constexpr int kPoolKeysPerWave = 64;
constexpr int kPoolKeys = kPoolWaves * kPoolKeysPerWave;  // keys per workgroup

// Work items of one (b, KV head) are (tile t, chunk of kPoolKeys candidate keys).
// With T-row tiles, tile t is given ceil((t+1) T / 256) chunks (its prefix_t
// candidates need at most that many; a chunk past a ragged last tile's prefix
// does nothing), so the items before tile t number
// sum_{u=1..t} ceil(u / p), p = 256 / T, which is p Q(Q+1)/2 + R(Q+1) for
// t = Qp + R, 0 <= R < p.
__host__ __device__ inline int pool_items_before(int t, int tile) {
  const int p = kPoolKeys / tile;
  const int q = t / p, r = t % p;
  return p * q * (q + 1) / 2 + r * (q + 1);
}

// The pooled pass is built for occupancy: the matrix and vector work of one
// wavefront hides behind the other wavefronts of its SIMD. A workgroup (four
// wavefronts, 256 keys) walks the units of the group's heads for its tile: 64
// query rows (a head's tile, or half of it), staged by direct global -> LDS
// loads into a ring of two slots (unpadded rows, 16-byte slots swizzled by
// swz<D>), unit u + 1 landing while unit u is used. Per 16-row block a
// wavefront computes its 16 x 64 scores and their exp2/sum work with few
// operands live, and the LDS footprint stays near 32 KiB at d = 128. A unit
// whose rows lie wholly before the wavefront's keys costs nothing but its
// share of the loads.
constexpr int kPoolUnit = 64;  // query rows per staged unit

// Wavefronts per SIMD: four at d = 128 (128 VGPRs), five at d = 64 (85).
template <int D>
constexpr int pool_waves_per_simd() { return D == 128 ? 4 : 5; }

template <int D, int TP>
__global__ __launch_bounds__(64 * kPoolWaves) __attribute__((amdgpu_waves_per_eu(pool_waves_per_simd<D>())))
void prefill_pool(PrefillArgs a, int items, int per_xcd) {
  constexpr int C = D / 32;
  constexpr int SLOTS = D / 8;                                   // 16-byte slots per row
  constexpr int DPW = kPoolUnit * D * 2 / (kPoolWaves * 1024);   // 1 KiB direct loads per wave and unit
  static_assert(DPW >= 1 && kPoolUnit * D * 2 == DPW * kPoolWaves * 1024, "unit must split evenly");
  static_assert(TP % kPoolUnit == 0, "tile must hold whole units");
  __shared__ __attribute__((aligned(16))) __bf16 qs[2][kPoolUnit * D];
  __shared__ __attribute__((aligned(16))) float ls[2][kPoolUnit];

  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= items) return;
  int t = max(0, (int)sqrtf(512.0f / TP * (float)item) - 1);
  while (pool_items_before(t + 1, TP) <= item) ++t;
  while (t > 0 && pool_items_before(t, TP) > item) --t;
  const int kbase = (item - pool_items_before(t, TP)) * kPoolKeys;
  const int kvh = blockIdx.z % a.hkv, b = blockIdx.z / a.hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int n16 = lane & 15, qg = lane >> 4;
  const int wkey0 = kbase + wave * kPoolKeysPerWave;
  const int row0 = t * TP;
  const int prefix = min(row0 + TP, a.n);
  const float sl2 = a.scale_log2;
  // Units of the tile that hold rows below N (one or two per head); unit u
  // is head u / 2 and rows row0 + 64 (u % 2) onward when there are two.
  const bool two = prefix - row0 > kPoolUnit;
  const int units = two ? 2 * a.group : a.group;

  const u16* kb = a.k + (size_t)(b * a.hkv + kvh) * a.n * D;
  bf16x8 bk[4][C];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = wkey0 + 16 * kt + n16;
    const u16* krow = kb + (size_t)(key < a.n ? key : 0) * D;
#pragma unroll
    for (int c = 0; c < C; ++c) bk[kt][c] = load_bf16x8(krow + 32 * c + 8 * qg);
  }
  float colsum[4] = {0.f, 0.f, 0.f, 0.f};

  // Direct load i of this wave fills LDS slot position q % SLOTS of unit row
  // q / SLOTS, q = 64 (DPW wave + i) + lane, with source slot pos ^ swz(row).
  int last_u = 0;  // last row of the unit issued last, from its first row
  auto issue = [&](int u) __attribute__((always_inline)) {
    const int h = kvh * a.group + (two ? u >> 1 : u);
    const int ur0 = row0 + (two ? kPoolUnit * (u & 1) : 0);
    const int last = a.n - 1 - ur0;  // >= 0: the unit starts below N
    const u16* src = a.q + ((size_t)(b * a.hq + h) * a.n + ur0) * D;
    const unsigned lds = lds_address(&qs[u & 1][0]) + (unsigned)(wave * DPW) * 1024u;
    // The rows' log2-sum-exp straight into LDS as well (rows past N read row
    // N - 1 and are set to +inf once the load has landed, so that they add 0).
    if (wave == 0)
      lds_dma4_at(a.lse2 + (size_t)(b * a.hq + h) * a.n + ur0, (unsigned)min(lane, last) * 4u,
                  lds_address(&ls[u & 1][0]));
    last_u = last;
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
      const int r = (64 / SLOTS) * (DPW * wave + i) + lane / SLOTS, pos = lane % SLOTS;
      const unsigned off = (unsigned)(min(r, last) * D + 8 * (pos ^ swz<D>(r))) * 2u;
      lds_dma16_at(src, off, lds + 1024u * i);
    }
  };
  auto land = [&](int u) __attribute__((always_inline)) {
    wait_vm(0);
    if (wave == 0 && last_u < kPoolUnit - 1) {
      const int ml = __lane_id();  // not kept live through the loop
      if (ml > last_u) ls[u & 1][ml] = INFINITY;
    }
  };
  auto read_q = [&](int buf, int rb, bf16x8 (&aq)[C], f32x4& lse) __attribute__((always_inline)) {
    const int row = 16 * rb + n16;
#pragma unroll
    for (int c = 0; c < C; ++c)
      aq[c] = *reinterpret_cast<const bf16x8*>(&qs[buf][row * D + 8 * ((4 * c + qg) ^ swz<D>(row))]);
    lse = *reinterpret_cast<const f32x4*>(&ls[buf][16 * rb + 4 * qg]);
  };
  auto scores = [&](const bf16x8 (&aq)[C], f32x4 (&s)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[kt] = mfma16x16x32(aq[c], bk[kt][c], s[kt]);
  };

  issue(0);
  land(0);
  __syncthreads();
  for (int u = 0; u < units; ++u) {
    const int buf = u & 1;
    if (u + 1 < units) issue(u + 1);
    const int ur0 = row0 + (two ? kPoolUnit * (u & 1) : 0);
    if (wkey0 + kPoolKeysPerWave - 1 <= ur0) {
      // Every key of the wave is visible to every row of the unit.
#pragma unroll
      for (int rb = 0; rb < kPoolUnit / 16; ++rb) {
        bf16x8 aq[C];
        f32x4 lse, s[4];
        read_q(buf, rb, aq, lse);
        scores(aq, s);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) colsum[kt] += fast_exp2(fmaf(s[kt][r], sl2, -lse[r]));
        // One block's operands live at a time: the other wavefronts of the
        // SIMD fill the gaps.
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (wkey0 < prefix && wkey0 <= ur0 + kPoolUnit - 1) {
      // Diagonal: key j counts for row i only when j <= i.
#pragma unroll 1
      for (int rb = 0; rb < kPoolUnit / 16; ++rb) {
        const int rr0 = ur0 + 16 * rb;
        if (rr0 + 15 < wkey0 || rr0 >= prefix) continue;  // no key of the wave is visible
        bf16x8 aq[C];
        f32x4 lse, s[4];
        read_q(buf, rb, aq, lse);
        scores(aq, s);
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int key = wkey0 + 16 * kt + n16;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(fmaf(s[kt][r], sl2, -lse[r]));
            colsum[kt] += key <= rr0 + 4 * qg + r ? pr : 0.f;
          }
        }
      }
    }
    if (u + 1 < units) land(u + 1);
    __syncthreads();
  }

  const size_t ragged = prefill_ragged_len(a.n, TP);
  float* dst = a.pooled + (size_t)(b * a.hkv + kvh) * ragged + (size_t)TP * t * (t + 1) / 2;
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

template <int D, bool GATHER, bool WITH_O, int TR>
hipError_t launch_attn(const PrefillArgs& a, hipStream_t s) {
  // Reuse layers: the heads of a GQA group that fill eight wavefronts (two
  // heads of 128 rows, or four of 64) share every gathered K/V chunk, staged
  // 128 keys at a time so each gather has a long step of work to land behind.
  // Dense pass: one head per workgroup, 64-key chunks in a ring of two
  // buffers, two workgroups per compute unit.
  constexpr int WPH = TR / kRowsPerWave;
  constexpr int NHG = 8 / WPH;
  const int wtiles = (a.n + TR - 1) / TR;
  if (GATHER && a.group % NHG == 0) {
    dim3 grid(wtiles * a.batch * (a.hq / NHG));
    hipLaunchKernelGGL((prefill_attn<D, GATHER, WITH_O, NHG, 128, TR, 2>), grid, dim3(64 * WPH * NHG), 0, s, a);
  } else if (GATHER && NHG > 2 && a.group % 2 == 0) {
    dim3 grid(wtiles * a.batch * (a.hq / 2));
    hipLaunchKernelGGL((prefill_attn<D, GATHER, WITH_O, 2, 64, TR, 2>), grid, dim3(64 * WPH * 2), 0, s, a);
  } else {
    dim3 grid(wtiles * a.batch * a.hq);
    hipLaunchKernelGGL((prefill_attn<D, GATHER, WITH_O, 1, 64, TR, 2>), grid, dim3(64 * WPH), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill_dense(const PrefillArgs& a, hipStream_t s) {
  const bool with_o = a.out != nullptr;
  // The row log-sum-exp and the dense output do not depend on the selection
  // tile, so the dense pass always works in kTile-row tiles.
  if (a.d == 128)
    return with_o ? launch_attn<128, false, true, kTile>(a, s) : launch_attn<128, false, false, kTile>(a, s);
  if (a.d == 64)
    return with_o ? launch_attn<64, false, true, kTile>(a, s) : launch_attn<64, false, false, kTile>(a, s);
  return hipErrorInvalidValue;
}

// 1: reuse layers use the LDS-ring kernel where it applies (prefill_gather.hip);
// 0: always the register-staged gather mode of prefill_attn.
#ifndef KASCADE_REUSE_RING
#define KASCADE_REUSE_RING 1
#endif

hipError_t launch_prefill_reuse(const PrefillArgs& a, hipStream_t s) {
  if (KASCADE_REUSE_RING && prefill_reuse_ring_supported(a)) return launch_prefill_reuse_ring(a, s);
  if (a.tile == 128) {
    if (a.d == 128) return launch_attn<128, true, true, 128>(a, s);
    if (a.d == 64) return launch_attn<64, true, true, 128>(a, s);
  } else if (a.tile == 64) {
    if (a.d == 128) return launch_attn<128, true, true, 64>(a, s);
    if (a.d == 64) return launch_attn<64, true, true, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_pool(const PrefillArgs& a, hipStream_t s) {
  const int items = pool_items_before(a.tiles, a.tile);
  const int per_xcd = (items + 7) / 8;
  dim3 grid(8 * per_xcd, 1, a.hkv * a.batch);
  dim3 block(64 * kPoolWaves);
  if (a.tile == 128 && a.d == 128) hipLaunchKernelGGL((prefill_pool<128, 128>), grid, block, 0, s, a, items, per_xcd);
  else if (a.tile == 128 && a.d == 64) hipLaunchKernelGGL((prefill_pool<64, 128>), grid, block, 0, s, a, items, per_xcd);
  else if (a.tile == 64 && a.d == 128) hipLaunchKernelGGL((prefill_pool<128, 64>), grid, block, 0, s, a, items, per_xcd);
  else if (a.tile == 64 && a.d == 64) hipLaunchKernelGGL((prefill_pool<64, 64>), grid, block, 0, s, a, items, per_xcd);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_lse2_to_lse(const float* lse2, float* lse, size_t count, hipStream_t s) {
  hipLaunchKernelGGL(lse2_to_lse_kernel, dim3((count + 255) / 256), dim3(256), 0, s, lse2, lse,
                     count);
  return hipGetLastError();
}

}  // namespace kascade
