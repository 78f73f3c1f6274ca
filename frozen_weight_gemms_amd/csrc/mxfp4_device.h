// Device-side MXFP4 block encoding (PACT, Appendix Table 6, MXFP4 column:
// 32-element blocks, E2M1 elements, one E8M0 scale per block), shared by the
// MXFP4 quantizer and the fused RMSNorm / SiLU-multiply kernels' MXFP4 mode.
// Block scale (the OCP microscaling rule): shared exponent
// e = floor(log2(blockmax)) - 2 clamped to [-127, 127] (-127 for an all-zero
// block), stored as the byte e + 127; element code = RNE(|x| / 2^e) onto E2M1,
// ties to even, saturating at 6, sign kept.  |x| / 2^e is an exact power-of-
// two scaling (2^-e is a normal FP32 number for every e a finite FP32 block
// maximum can produce), and v_cvt_scalef32_pk_fp4_f32 with scale 1.0 performs
// the RNE, saturation and sign handling.
#pragma once

#include "nvfp4_device.h"

namespace pact {

constexpr int kMxBlock = 32;

// floor(log2(amax)) - 2, clamped to [-127, 127]; -127 for amax == 0 (amax >= 0 finite).
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0u) return -127;
  const int ef = (int)(u >> 23);
  const int fl = ef != 0 ? ef - 127 : (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;   // subnormal amax
  const int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 8 elements times 2^-e -> 8 packed E2M1 codes (element 0 in the low nibble).
__device__ __forceinline__ uint32_t mx_encode8(const float* x, float inv) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * inv, x[1] * inv, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * inv, x[3] * inv, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * inv, x[5] * inv, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * inv, x[7] * inv, 1.0f, 3);
  return w;
}

// Value of an E8M0 scale byte b (0..254): 2^(b - 127), exact in FP32 (b = 0 is
// the subnormal 2^-127).
__device__ __forceinline__ float e8m0_decode(uint32_t b) {
  return b != 0u ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// 2^-e as FP32 for e in [-127, 125] (a normal number)
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// Quantize chunk c (8 elements) of a row to MXFP4.  The four lanes 4p .. 4p + 3
// that hold chunks 4q .. 4q + 3 (one 32-element block) must all call this: the
// block maximum is exchanged with lanes ^ 1 and ^ 2.
__device__ __forceinline__ void mx_quant_chunk(const float* x, bool valid, uint8_t* codes_row, uint8_t* scales_row,
                                               int c) {
  float m = valid ? absmax8(x) : 0.0f;
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  if (!valid) return;
  const int e = mx_shared_exp(m);
  *reinterpret_cast<uint32_t*>(codes_row + 4 * (int64_t)c) = mx_encode8(x, mx_inv_scale(e));
  if ((c & 3) == 0) scales_row[c >> 2] = (uint8_t)(e + 127);
}

// Quantize one 16-element half of a 32-element block held by one lane; the
// other half is on lane ^ 1 (blocks of 16 on consecutive lanes).  bmax16 is
// this half's maximum; both lanes of the pair must call this.
__device__ __forceinline__ void mx_quant_half(const float* x, float bmax16, bool valid, uint8_t* codes_row,
                                              uint8_t* scales_row, int blk16) {
  const float m = fmaxf(bmax16, __shfl_xor(bmax16, 1, 64));
  if (!valid) return;
  const int e = mx_shared_exp(m);
  const float inv = mx_inv_scale(e);
  *reinterpret_cast<uint2*>(codes_row + 8 * (int64_t)blk16) = make_uint2(mx_encode8(x, inv), mx_encode8(x + 8, inv));
  if ((blk16 & 1) == 0) scales_row[blk16 >> 1] = (uint8_t)(e + 127);
}

}  // namespace pact
