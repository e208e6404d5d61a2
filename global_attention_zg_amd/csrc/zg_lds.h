// LDS tile helpers shared by the gfx950 attention kernels of libzgattn:
// untracked global -> LDS copies, explicit waits and barriers, and the LDS
// operand reads of the MFMA tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zg_common.h"

namespace zg {

typedef short i16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) unsigned char lds_u8;

// Global -> LDS copies are issued as inline asm, so that the compiler does not
// track them: it would otherwise place a vmcnt(0) wait in front of every LDS
// read that it cannot prove disjoint from an in-flight copy, which serialises
// the tile ring.  Every wait for copied data is explicit below (in-order
// completion of vector loads makes "at most N outstanding" exact), and M0 is
// written only here.
__device__ __forceinline__ uint32_t lds_addr(const lds_u8* p) { return (uint32_t)(uintptr_t)p; }

// 16 bytes per lane from a per-lane 64-bit address to LDS base + 16 * lane.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory");
}

// Same, from a wave-uniform base plus a per-lane 32-bit byte offset.
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "s"(lds)
               : "memory");
}

// At most N of this wave's vector loads still in flight.
template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// At most N vector loads in flight and this wave's LDS accesses done, then
// the workgroup barrier.
template <int N> __device__ __forceinline__ void sync_tiles() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Phase boundaries of a ping-pong loop: the barrier (after at most N vector
// loads in flight, and with LGKM also drained) fenced on both sides against
// the instruction scheduler, so that no ALU or MFMA work moves across.
template <int N, bool LGKM> __device__ __forceinline__ void phase_sync() {
  __builtin_amdgcn_sched_barrier(0);
  if (LGKM) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
  __builtin_amdgcn_sched_barrier(0);
}
// An empty asm that consumes x: x is computed before this point (keeps the
// compiler from sinking a phase's results into the next phase).
template <typename T> __device__ __forceinline__ void pin(const T& x) { asm volatile("" ::"v"(x)); }
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const lds_u8* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(p);
}

// Two transposing 8-byte LDS loads -> one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 lds_read_tr2(const lds_u8* p0, const lds_u8* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_u8*>(p0)));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_u8*>(p1)));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

}  // namespace zg
