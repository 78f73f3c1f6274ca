// Global -> LDS direct loads through buffer resources, shared by the NVFP4
// and MXFP4 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pact {

typedef int int4v_t __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): raw (stride 0), so an access at
// offset >= bytes returns zeros instead of touching memory.
__device__ __forceinline__ int4v_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  int4v_t r;
  r[0] = (int)(uint32_t)a;
  r[1] = (int)((a >> 32) & 0xffffu);
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at voff + soff into LDS at lds + 16 * lane.
// Issued through inline asm so that the compiler does not treat every later
// LDS read as a possible alias of the asynchronous write (it would then wait
// for all outstanding loads and serialize the stage pipeline); the kernel
// waits for them explicitly with s_waitcnt vmcnt before the barrier that
// publishes a stage.
__device__ __forceinline__ void lds_dma_buf16(int4v_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory", "m0");
}
// 4 bytes per lane from the buffer at voff + soff into LDS at lds + 4 * lane.
__device__ __forceinline__ void lds_dma_buf4(int4v_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds"
               ::"v"(voff), "s"(rsrc), "s"(lds), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define PACT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))


}  // namespace pact
