// Helpers shared by the matrix-core GEMM kernels (gfx950, wave64): the XCD
// tile remap, raw buffer resources and buffer loads that write LDS directly.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {
namespace gemm {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ uint32_t xcd_remap(uint32_t id, uint32_t n) {
  const uint32_t q = n / 8, r = n % 8, x = id % 8, local = id / 8;
  return (x < r) ? x * (q + 1) + local : r * (q + 1) + (x - r) * q + local;
}

// Buffer load of 16 bytes per lane straight into LDS: lane l's bytes land at
// M0 + 16 l, M0 being the (wavefront-uniform) LDS address passed here.
__device__ void buffer_load_lds(i32x4 rsrc, lds_u32 *lds, int32_t size, int32_t voffset, int32_t soffset,
                                int32_t offset, int32_t aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Raw buffer resource (stride 0, 32-bit elements) over num_bytes from base.
__device__ __forceinline__ i32x4 make_rsrc(const void *base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = (int32_t)(uint32_t)a;
  r.y = (int32_t)((uint32_t)(a >> 32) & 0xffffu);
  r.z = (int32_t)num_bytes;
  r.w = 0x00020000;
  return r;
}

// The same descriptor, marked wavefront-uniform for the compiler (a buffer
// instruction takes its descriptor from scalar registers; without the mark a
// descriptor the compiler keeps in vector registers costs a loop per load).
__device__ __forceinline__ i32x4 uniform_rsrc(i32x4 r) {
  return i32x4{__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
               __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w)};
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

}  // namespace gemm
}  // namespace kvc
