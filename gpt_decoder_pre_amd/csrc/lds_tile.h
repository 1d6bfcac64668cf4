// LDS tiles for the MFMA kernels: direct global->LDS loads, bank swizzles and
// fragment reads, shared by the GEMM and attention kernels.
//
// Tiles are filled with global_load_lds_dwordx4 (each lane moves 16 bytes; a
// wave instruction fills 1 KB of LDS at m0 + 16 * lane), so a tile's layout is
// chosen by which global chunk each lane fetches:
//   * k-contiguous tile (rows of BK elements, fragments read row-wise with
//     ds_read_b128): the 16-byte chunks of a row are XOR-swizzled by kswz(row)
//     so that the fragment reads of 16 consecutive rows hit distinct banks;
//   * transposed tile (rows are k, R elements each, fragments read with
//     ds_read_b64_tr_b16, which hands each lane four consecutive k of one
//     column): chunks are XOR-swizzled by tswz<R>(k) (below).
#pragma once

#include "common.h"

namespace gpt2k {

typedef short i16x4g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4g lds_i16x4g;
typedef __attribute__((address_space(3))) void lds_void;

template <int BK>
DEVI int kswz(int r) {
  if constexpr (BK == 32) return ((r >> 1) ^ (r >> 3)) & 3;
  else return (r ^ (r >> 3)) & 7;
}
// A transposed fragment read takes, per 256-byte slice, 4 consecutive k rows
// x 4 consecutive chunks.  For rows of 128 or 256 elements (a whole number of
// bank cycles) the 4 rows must land in 4 different chunk quads: XOR by
// 4 (k mod 4).  For 192-element rows consecutive rows are already half a
// bank cycle apart and XOR by 2 (k mod 4) suffices (a 12-wide XOR would also
// leave the row's 24 chunks).
template <int R>
DEVI int tswz(int k) {
  if constexpr (R % 128 == 0) return 4 * (k & 3);
  else return 2 * (k & 3);
}


// Workgroup barrier without the release fence of __syncthreads (which would
// drain every outstanding global->LDS load): ordering of LDS data across waves
// comes from each wave's own vmcnt wait before the barrier, and the memory
// clobber keeps the compiler from moving LDS accesses across it.
DEVI void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One global_load_lds_dwordx4: each lane moves 16 bytes from gptr to LDS
// address m0 + 16 * lane (m0 = lds_base, wave-uniform).  Written as inline asm
// so that the compiler does not treat it as an LDS store it must wait for
// before every LDS read (it cannot tell the pipeline stages apart); the
// kernel orders it with explicit vmcnt waits.  The instruction has no output
// registers; its address registers are read at issue.  m0 is set in the same
// asm block as its one use; nothing else in these kernels reads m0 (the
// compiler needs it on gfx950 only for LDS DMA builtins, message sends and
// indexed register moves, none of which they use), so clobbering the
// reserved register here is safe.
DEVI void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}

// The same with a wave-uniform 64-bit base (SGPRs) and a per-lane 32-bit
// byte offset (the SADDR form): no per-lane 64-bit address arithmetic.
DEVI void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// One global_load_lds_dword: each lane moves 4 bytes from gptr to LDS address
// m0 + 4 * lane (dma16 with 4-byte elements).
DEVI void dma4(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds_base), "v"(gptr) : "memory", "m0");
}

// A pointer the compiler can keep in SGPRs (the value must be wave-uniform).
template <typename T>
DEVI const T* uniform_ptr(const T* q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// vmcnt(n) with expcnt and lgkmcnt left alone (gfx9 encoding).
template <int N>
DEVI void wait_vmcnt() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Fragment (eight consecutive k of one row, rows = lane % 32) for the 16-k step kk.
template <bool KMAJ, int R, int BK>
DEVI h16x8 frag(const h16* tile, int row0, int kk, int lane) {
  if constexpr (KMAJ) {
    const int r = row0 + (lane & 31);
    const int c = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const h16x8*>(tile + r * BK + 8 * (c ^ kswz<BK>(r)));
  } else {
    const int g = lane >> 4, s = lane & 15;
    const int k = 16 * kk + 8 * (g >> 1) + (s >> 2);
    const int m = row0 + 16 * (g & 1) + 4 * (s & 3);
    const int c = m >> 3, o = m & 7;
    const h16* p1 = tile + k * R + 8 * (c ^ tswz<R>(k)) + o;
    const h16* p2 = tile + (k + 4) * R + 8 * (c ^ tswz<R>(k + 4)) + o;
    const i16x4g a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4g*)p1);
    const i16x4g b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4g*)p2);
    const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
    u32x4 v = {ua[0], ua[1], ub[0], ub[1]};
    return __builtin_bit_cast(h16x8, v);
  }
}

}  // namespace gpt2k
