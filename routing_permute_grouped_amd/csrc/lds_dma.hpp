// Direct global->LDS loads shared by the GEMM kernels: LDS addresses, raw buffer
// descriptors with hardware range checking, and the 16-byte-per-lane buffer load that
// writes LDS without passing through registers.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime.h>

namespace moe {

// LDS byte address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// Raw buffer descriptor over [base, base + bytes): the hardware zero-fills any lane
// whose offset falls outside the range.
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = 0x00020000;   // raw (untyped) buffer, 32-bit data format
  return r;
}

// 16 bytes per lane from a buffer straight into LDS: lane l reads base + voff_l + soff
// and the 64 lanes of the wave fill 1 KiB at LDS address `lds` (wave-uniform), lane l
// at lds + 16*l. Buffer addressing takes a 32-bit offset per lane and the k-step in a
// scalar offset, which issues faster than 64-bit flat addresses. Issued as inline
// assembly so the compiler adds no waits of its own for it (nor counts it among the
// loads it waits for): a caller waits with an explicit s_waitcnt vmcnt and a barrier
// before any wave reads the LDS the loads fill.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(soff)),
                 "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}

}  // namespace moe
