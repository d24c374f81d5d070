// LDS and direct global->LDS load primitives shared by the MFMA kernels
// (step / training attention, fused LM head).
#pragma once

#include <stdint.h>

#include "common.h"

namespace tidar {

// LDS pointers stay in address space 3 end to end (no generic casts)
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0]+[15:14], expcnt[6:4], lgkmcnt[11:8])
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
// Workgroup barrier that is also a compiler memory barrier: LDS reads and
// writes stay on their side of it.  Waiting for this wave's own memory
// operations is left to the caller (the ring waits for some direct loads
// only).
__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global->LDS load of 16 B per lane: lane t's bytes land at
// lds_dst + 16*t.  Issued as inline asm with a scalar base and a 32-bit
// per-lane offset, so the compiler neither rebuilds 64-bit addresses every
// tile nor treats the load as an LDS store it must order against unrelated
// LDS reads (its LDS-DMA alias tracking would serialise the pipeline); the
// kernel orders these loads itself with s_waitcnt vmcnt and barriers.  The
// load takes its LDS address from m0, which the block sets and then restores
// (the load reads m0 when it issues, not when its data arrives), so whatever
// the compiler keeps in m0 survives; no vector register is written.
// NT: the nontemporal form, for data read once (a streaming hint to the
// caches; measured on plain streaming reads to raise the delivered rate).
template <bool NT = false>
__device__ __forceinline__ void dma_b128(const char* base, unsigned off, lds_char* lds_dst) {
  const unsigned long long b = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)b);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(b >> 32));
  const unsigned long long sb = ((unsigned long long)hi << 32) | lo;
  const unsigned dst = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_dst);
  unsigned saved;
  if constexpr (NT)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(off), "s"(sb), "s"(dst)
                 : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "v"(off), "s"(sb), "s"(dst)
                 : "memory");
}

}  // namespace tidar
