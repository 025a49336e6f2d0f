// Global-memory-to-LDS DMA staging helpers for the gfx950 GEMM kernels.
//
// A DMA instruction (global_load_lds, 16 or 4 bytes per lane) writes lane l's
// bytes at lds_base + l * bytes.  It is issued as inline assembly so that the
// compiler's wait-count pass, which cannot tell LDS stages apart, does not
// add a wait for every DMA in flight before each LDS read; the kernels wait
// explicitly with wait_vm<P>() (this wave's loads older than its newest P are
// complete) and synchronize with barrier_no_fence().  M0 holds the wave's LDS
// base (wave-uniform); one wait state separates its write from the load.  M0
// is not otherwise used by these kernels, so clobbering it is safe.  The
// instructions have no register results, so nothing is left in flight in a
// register the compiler could reuse.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quads {

typedef __attribute__((address_space(3))) void lds_t;

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma(const void *g, void *lds_base, int bytes) {
  const uint32_t m0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_t *)lds_base));
  if (bytes == 16)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
#pragma clang diagnostic pop

// Wait until at most the newest P vector-memory operations of this wave are
// outstanding (gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
// lgkmcnt 11:8 left at their maxima).
template <int P>
__device__ __forceinline__ void wait_vm() {
  static_assert(P >= 0 && P < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (P & 15) | ((P >> 4) << 14));
}

// Workgroup barrier without a memory fence: __syncthreads() would also wait
// for every DMA in flight (vmcnt(0)), including the stages being prefetched.
// LDS visibility comes from the explicit vmcnt wait before the barrier (DMA
// writes) and from every fragment read having been consumed before it; the
// empty asm statements keep the compiler from moving memory accesses across.
// This wave's LDS (and scalar memory) accesses are complete.
__device__ __forceinline__ void wait_lgkm0() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier_no_fence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace quads
