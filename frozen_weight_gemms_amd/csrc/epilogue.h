// Output slabs of the GEMM epilogues (NVFP4, single-layout dgrad, MXFP4).
//
// A wave stages 32 rows of its WN-column part of the tile in LDS as FP32
// (row stride LD floats) and writes them out as BF16.  For a slab that lies
// inside the output with 16-byte aligned rows, lane l owns WN / 16 pieces of
// 8 columns: piece t is row (l + 64 t) / (WN / 8), columns 8 ((l + 64 t) mod
// (WN / 8)) .. + 7.  The LDS reads of a group of pieces are issued before its
// first store and every store is addressed from the slab's base pointer (a
// loop that read, waited and checked bounds per piece cost the 256 x 256
// tile about 2 us per launch round).
#pragma once

#include "nvfp4_device.h"

namespace pact {

// The staged slab, plus the BF16 values already in the output when
// accumulating (each sum in FP32, then one BF16 rounding), stored as BF16.
// The caller waits for the LDS reads (lgkmcnt) before it stages the next slab
// over this one.
template <int WN, int LD>
__device__ __forceinline__ void slab_store(const float* epi, uint16_t* out, int64_t ldo, bool accumulate, int lane) {
  constexpr int CH = WN / 8, IT = WN / 16;
  // pieces in flight per group (bounds the registers held): 4, or 3 for
  // six pieces
  constexpr int G = IT % 4 == 0 ? 4 : (IT % 3 == 0 ? 3 : 1);
  static_assert(WN % 16 == 0 && LD % 4 == 0, "slab pieces");
#pragma unroll
  for (int t0 = 0; t0 < IT; t0 += G) {
    uint4 old[G];
    if (accumulate) {
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int q = lane + 64 * (t0 + u), row = q / CH, ch = q % CH;
        old[u] = *reinterpret_cast<const uint4*>(out + row * ldo + ch * 8);
      }
    }
    float4 v[G][2];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int q = lane + 64 * (t0 + u), row = q / CH, ch = q % CH;
      const float4* src = reinterpret_cast<const float4*>(epi + row * LD + ch * 8);
      v[u][0] = src[0];
      v[u][1] = src[1];
    }
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int q = lane + 64 * (t0 + u), row = q / CH, ch = q % CH;
      float4 a = v[u][0], b = v[u][1];
      if (accumulate) {
        a.x += bf16_lo(old[u].x); a.y += bf16_hi(old[u].x); a.z += bf16_lo(old[u].y); a.w += bf16_hi(old[u].y);
        b.x += bf16_lo(old[u].z); b.y += bf16_hi(old[u].z); b.z += bf16_lo(old[u].w); b.w += bf16_hi(old[u].w);
      }
      uint4 o;
      o.x = pack_bf16x2(a.x, a.y); o.y = pack_bf16x2(a.z, a.w);
      o.z = pack_bf16x2(b.x, b.y); o.w = pack_bf16x2(b.z, b.w);
      *reinterpret_cast<uint4*>(out + row * ldo + ch * 8) = o;
    }
  }
}

}  // namespace pact
