// Direct buffer-to-LDS loads for gfx950 kernels (buffer_load ... lds), used by the backward
// kernels.  Each instruction moves 16 bytes per lane from a per-lane byte offset of a buffer
// resource to 64 consecutive 16-byte LDS slots starting at M0, without passing through
// registers.  They are issued as inline asm so that the compiler does not wait for them before
// every LDS read; the kernel waits for them itself with wait_vmcnt<N> (they count in vmcnt, in
// issue order).  Offsets at or past the resource's range read as zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssw {
namespace lds_dma {

typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kOutOfRange = 0x80000000u;

// Buffer resource over `bytes` bytes at `base` (no stride, no swizzle, 32-bit data format).
__device__ __forceinline__ i32x4 resource(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from rsrc + voff to LDS [lds_base + 16 * lane]; lds_base wave-uniform.
__device__ __forceinline__ void load16(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  i32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds_base)),
               "v"(voff), "s"(u)
               : "memory");
}

// 4 bytes per lane from rsrc + voff to LDS [lds_base + 4 * lane].
__device__ __forceinline__ void load4(i32x4 rsrc, uint32_t lds_base, uint32_t voff) {
  i32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = __builtin_amdgcn_readfirstlane(rsrc[i]);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(
                   __builtin_amdgcn_readfirstlane(lds_base)),
               "v"(voff), "s"(u)
               : "memory");
}

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)p;
}

}  // namespace lds_dma
}  // namespace ssw
