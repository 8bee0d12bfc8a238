// Direct global -> LDS loads (LDS DMA) and the waits of the pipelines built on them, shared
// by the GEMM kernels of the library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8moe {

// global -> LDS without VGPR staging: lane i of the wave copies `size` bytes from
// base + voff (base wave-uniform, voff per lane) to LDS byte address lds + size * i (lds
// wave-uniform, passed in M0). Issued as inline assembly so that the compiler does not
// track these loads: it would otherwise make LDS reads of the stage being computed wait
// for every load in flight (vmcnt(0)), which serialises the pipeline. The kernel waits
// for them itself, by count, and a workgroup barrier then publishes them. Because the
// compiler does not see the load, it cannot insert the wait states the ISA requires
// around a vector memory instruction's operands, so the asm provides them: 5 before it,
// for a VALU write of an SGPR (v_readlane / v_readfirstlane, e.g. a restored spill) that
// the load reads as its base address (this also covers the one after a write of M0), and
// 1 after it, before an instruction may overwrite an SGPR the load reads.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// The base address is wave-uniform by contract; readfirstlane makes that explicit to the
// compiler (a no-op when it already holds the value in SGPRs).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1\n\ts_nop 0"
               :: "v"(voff), "s"(uniform_ptr(base)), "{m0}"(lds_addr(lds)) : "memory");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, const void* lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1\n\ts_nop 0"
               :: "v"(voff), "s"(uniform_ptr(base)), "{m0}"(lds_addr(lds)) : "memory");
}

// Waits and barriers of the pipeline. They are compiler memory barriers ("memory"
// clobber), so no LDS access moves across them. The barrier drains this wave's LDS
// traffic first (the only data other waves read after it); the direct-to-LDS loads are
// waited for with vmcnt.
__device__ __forceinline__ void wait_all_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory loads (LDS DMA included) are still in
// flight; loads complete in issue order for this count.
template <int N>
__device__ __forceinline__ void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace fp8moe
