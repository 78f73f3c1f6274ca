// Measured MFMA-loop peak: the rate at which the matrix cores of this GPU
// retire back-to-back independent MFMAs, the ceiling the GEMM kernels are
// compared against beside the published dense peaks.  Each of 512 workgroups
// (4 waves: two per SIMD when two workgroups share a CU) runs `iters`
// iterations of 16 independent accumulation chains, with no memory traffic in
// the loop.  Every workgroup also reads the shader clock (s_memtime) and the
// 100 MHz constant clock (s_memrealtime) at its start and end, so the caller
// gets the clock the chip held under the load.
//   kind 0: v_mfma_f32_32x32x16_f16             (32768 FLOP per instruction)
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4, FP4 operands with unit E8M0
//           scales (131072 FLOP per instruction)
#include "pact_internal.h"

namespace pact {

typedef _Float16 ph8_t __attribute__((ext_vector_type(8)));
typedef float pfx16_t __attribute__((ext_vector_type(16)));
typedef int pv8i_t __attribute__((ext_vector_type(8)));

template <int KIND>
__global__ __launch_bounds__(256) void k_mfma_probe(int iters, float* __restrict__ sink,
                                                    unsigned long long* __restrict__ clocks) {
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  pfx16_t acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.0f;
  const int lane = threadIdx.x & 63;
  if constexpr (KIND == 0) {
    ph8_t a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      a[t] = (_Float16)(float)((lane + t) & 7);
      b[t] = (_Float16)(float)((lane * 3 + t) & 3);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
  } else {
    pv8i_t a, b;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      a[t] = t < 4 ? (int)(0x22222222u + (uint32_t)lane) : 0;
      b[t] = t < 4 ? (int)(0x11111111u * (uint32_t)((lane & 3) + 1)) : 0;
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int c = 0; c < 16; ++c)
        acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 4, 4, 0, 127, 0, 127);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

hipError_t launch_mfma_probe(int kind, int iters, float* sink, unsigned long long* clocks, hipStream_t s) {
  if (kind == 0) k_mfma_probe<0><<<kMfmaProbeGroups, 256, 0, s>>>(iters, sink, clocks);
  else k_mfma_probe<1><<<kMfmaProbeGroups, 256, 0, s>>>(iters, sink, clocks);
  return hipGetLastError();
}

}  // namespace pact
