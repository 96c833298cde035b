// LDS staging building blocks of the prefill kernels (gfx950): direct
// global -> LDS loads, the transposed LDS read, explicit vector-memory waits
// and the 16-byte slot swizzle of unpadded LDS rows.
#pragma once

#include <hip/hip_runtime.h>

namespace kascade {

typedef __bf16 lds_bf16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each 16-lane group, lane L receives element
// (L mod 4) of the 4-element vectors addressed by lanes 4s + L/4, s = 0..3.
// Pointing lane L' at row (base + L'/4), columns (col + 4*(L' mod 4)) of a
// row-major [row][col] tile therefore hands lane L the four values
// tile[base + s][col + L], s = 0..3: a column of four rows, as the A operand
// of a contraction over rows needs.
__device__ __forceinline__ lds_bf16x4 lds_read_transposed(const __bf16* p) {
  typedef __attribute__((address_space(3))) lds_bf16x4 lds_vec;
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_vec*)(p));
}

// Direct global -> LDS loads (16 bytes per lane; lane l of the wavefront
// writes LDS bytes [lds + 16 l, +16)). They are issued from inline assembly so
// that the compiler does not wait for them before every LDS read (it cannot
// tell the buffers apart); completion is awaited explicitly with s_waitcnt
// vmcnt, see wait_vm. lds_dma16 takes a per-lane address; lds_dma16_at a
// wave-uniform base in scalar registers plus a per-lane 32-bit byte offset,
// which costs no vector ALU work per load. The lds argument (M0) must be
// wave-uniform.
__device__ __forceinline__ void lds_dma16(const void* src, unsigned lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void lds_dma16_at(const void* base, unsigned offset, unsigned lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"(base), "{m0}"(lds) : "memory");
}
// The same with the non-temporal hint: for rows read once, so that they do
// not displace rows that are read again from the L2.
__device__ __forceinline__ void lds_dma16_at_nt(const void* base, unsigned offset, unsigned lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(offset), "s"(base), "{m0}"(lds) : "memory");
}
// Four bytes per lane: lane l writes LDS bytes [lds + 4 l, +4).
__device__ __forceinline__ void lds_dma4_at(const void* base, unsigned offset, unsigned lds) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(offset), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ unsigned lds_address(const void* p) { return (unsigned)(size_t)p; }

// s_waitcnt vmcnt(n) for a run-time n (expcnt and lgkmcnt left unconstrained),
// followed by a compiler barrier, so that no LDS read of data those loads
// deliver is moved above the wait.
__device__ __forceinline__ void wait_vm(int n) {
#define KASCADE_VM(N) \
  case N: __builtin_amdgcn_s_waitcnt(0x0F70 | ((N) & 15) | (((N) >> 4) << 14)); break;
  switch (n) {
    KASCADE_VM(0) KASCADE_VM(1) KASCADE_VM(2) KASCADE_VM(3) KASCADE_VM(4) KASCADE_VM(5) KASCADE_VM(6)
    KASCADE_VM(7) KASCADE_VM(8) KASCADE_VM(9) KASCADE_VM(10) KASCADE_VM(11) KASCADE_VM(12) KASCADE_VM(13)
    KASCADE_VM(14) KASCADE_VM(15) KASCADE_VM(16) KASCADE_VM(17) KASCADE_VM(18) KASCADE_VM(19)
    KASCADE_VM(20) KASCADE_VM(21) KASCADE_VM(22) KASCADE_VM(23) KASCADE_VM(24) KASCADE_VM(25)
    KASCADE_VM(26) KASCADE_VM(27) KASCADE_VM(28) KASCADE_VM(29) KASCADE_VM(30) KASCADE_VM(31)
    KASCADE_VM(32) KASCADE_VM(33) KASCADE_VM(34) KASCADE_VM(35) KASCADE_VM(36) KASCADE_VM(37)
    KASCADE_VM(38) KASCADE_VM(39) KASCADE_VM(40) KASCADE_VM(41) KASCADE_VM(42) KASCADE_VM(43)
    KASCADE_VM(44) KASCADE_VM(45) KASCADE_VM(46) KASCADE_VM(47) KASCADE_VM(48) KASCADE_VM(49)
    KASCADE_VM(50) KASCADE_VM(51) KASCADE_VM(52) KASCADE_VM(53) KASCADE_VM(54) KASCADE_VM(55)
    KASCADE_VM(56) KASCADE_VM(57) KASCADE_VM(58) KASCADE_VM(59) KASCADE_VM(60) KASCADE_VM(61)
    KASCADE_VM(62) KASCADE_VM(63)
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
#undef KASCADE_VM
  asm volatile("" ::: "memory");
}

// LDS banks: 64 of four bytes, so 256 bytes are one bank sweep. A 16-byte read
// is served sixteen lanes at a time (lanes 16j..16j+15), an 8-byte transposed
// read thirty-two lanes at a time; a read runs at full rate when each such
// group covers distinct banks. The attention operand reads are
//   K (16 bytes, lane l: row 32 sub + l % 32, slot 2c + l / 32): sixteen
//   consecutive rows at one slot;
//   V^T (8 bytes transposed, per lane half): four consecutive rows, aligned
//   to four, each at the four consecutive slots 4db + 0..3.
// Direct loads fill unpadded rows, so there the 16-byte slot s of row r sits
// at slot s ^ swz<D>(r). D = 128: the row bits (r1, r0, r2, r3), high to low,
// whose top two bits tell four consecutive rows apart. D = 64 (rows r and
// r ^ 1 share a bank sweep): the bit reversal of (r >> 1) & 7, whose top bit
// tells rows two apart.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1))
                  : ((((r >> 1) & 1) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1));
}

}  // namespace kascade
