// Device-side NVFP4 arithmetic shared by the quantizer, fused and GEMM kernels.
//
// Format: 16-element blocks, E2M1 elements, E4M3 block scales (PACT, Appendix
// Table 6), plus one power-of-two FP32 scale per row.  Every rounding decision
// here reproduces the format's exact-real definition bit for bit:
//   * row exponent e: smallest integer with rowmax <= 6*448*2^e, clamped to
//     [-126, 127], 0 for an all-zero row;
//   * block scale s = RNE_E4M3(blockmax / (6 r)): blockmax/r is exact (r is a
//     power of two), its correctly rounded division by 6 can never sit on the
//     wrong side of an E4M3 midpoint (a midpoint times 6 r has at most 7
//     significant bits, so an FP32 blockmax is either on it or an ulp away), and
//     the E4M3 rounding below is integer arithmetic on the FP32 bit pattern;
//   * element code = RNE(|x| / (s r)) onto E2M1, ties to even, saturating at 6:
//     the quotient is computed correctly rounded (reciprocal correctly rounded
//     once per block, then one Markstein correction), and a correctly rounded
//     quotient equals an E2M1 midpoint exactly when the real quotient does;
//     v_cvt_scalef32_pk_fp4_f32 with scale 1.0 then performs exactly the RNE,
//     saturation and sign handling of the format (its scale operand contributes
//     only its exponent, so the block scale is divided out beforehand).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pact {

constexpr int kBlock = 16;

// *p where ok, else zero, without a branch: the load always reads a valid
// address (p, or `safe` where !ok) and the value is selected afterwards.  A
// conditional load compiles to a branch around it, and the compiler then waits
// for each such load before the next one: the loads of a step would be
// serialized instead of in flight together.
template <typename T>
__device__ __forceinline__ T load_or_zero(const T* p, const T* safe, bool ok) {
  const T v = *(ok ? p : safe);
  return ok ? v : T{};
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float -> bf16 bits, round to nearest even: the hardware conversion
// (v_cvt_pk_bf16_f32), which equals integer RNE on the bit pattern,
// u + 0x7FFF + ((u >> 16) & 1) >> 16, for every non-NaN input (the device
// self-test checks all 2^32 patterns).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Correctly rounded 1/d for d in [2^-126, 2^126) (normal d with a normal
// reciprocal): the hardware estimate y, the exact residual e = 1 - d*y (one
// FMA), then y + e*y rounded once.  Equal to IEEE division for every such d
// (the device self-test checks them all).
__device__ __forceinline__ float recip_rn(float d) {
  const float y = __builtin_amdgcn_rcpf(d);
  const float e = __builtin_fmaf(-d, y, 1.0f);
  return __builtin_fmaf(e, y, y);
}

// Correctly rounded x / 6: q = x * RN(1/6), then one correction with the
// exact remainder x - 6q (Markstein's division step).  Equal to IEEE division
// for every x >= 6 * 2^-126 (a normal quotient; the device self-test checks
// them all).  Below that both quotients are under 2^-126, far beneath the
// smallest E4M3 step 2^-9, so the block-scale code is 0 either way (and the
// round-up recipe decides with exact comparisons on x, not on the quotient).
__device__ __forceinline__ float div6_rn(float x) {
  const float c = __uint_as_float(0x3E2AAAABu);        // RN(1/6)
  const float q = __fmul_rn(x, c);
  const float r = __builtin_fmaf(-q, 6.0f, x);
  return __builtin_fmaf(r, c, q);
}

// Smallest e with amax <= 2688 * 2^e (2688 = 1.3125 * 2^11), clamped; 0 for amax == 0.
__device__ __forceinline__ int row_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0u) return 0;
  const int ef = (int)((u >> 23) & 0xFFu);
  if (ef == 0) return -126;                       // subnormal rowmax: e would be < -126
  const int e = ef - 127 - 11 + ((u & 0x7FFFFFu) > 0x280000u ? 1 : 0);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float pow2f(int e) {   // e in [-126, 127]
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// Conventional FP32 tensor scale for a tensor maximum amax (finite, >= 0):
// stored scale S = RN32(amax / 2688), at least 2^-126 (1 for amax == 0), and
// encoding multiplier R = RN32(1 / S).  Both quotients are taken in FP64 and
// rounded once more to FP32; FP64 carries more than twice FP32's precision
// plus two bits, so that second rounding of a correctly rounded quotient
// equals the correctly rounded FP32 quotient.  A subnormal S (flushed or not)
// is raised to 2^-126 either way.
__device__ __forceinline__ void tensor_scale_fp32(float amax, float& S, float& R) {
  if (amax == 0.0f) {
    S = 1.0f;
    R = 1.0f;
    return;
  }
  const float s = fmaxf((float)((double)amax / 2688.0), 1.17549435e-38f);
  S = s;
  R = (float)(1.0 / (double)s);
}

// Scale pair (r, inv_r) of a row from its (or the tensor's) maximum: the
// power of two of the row rule, or with kQuantFp32Tensor the FP32 tensor
// scale S and multiplier R (then |x| * inv_r is the rounded product u).
constexpr int kQuantRoundUp = 1;
constexpr int kQuantFp32Tensor = 2;
__device__ __forceinline__ void row_scale_pair(float amax, int qmode, float& r, float& inv_r) {
  if (qmode & kQuantFp32Tensor) {
    tensor_scale_fp32(amax, r, inv_r);
  } else {
    const int e = row_exponent(amax);
    r = pow2f(e);
    inv_r = pow2f(-e);
  }
}

// RNE of t >= 0 onto the E4M3FN grid, saturating at 448 (code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  if (t >= 448.0f) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);   // subnormal grid m * 2^-9 (m = 8 is 2^-6)
  uint32_t u = __float_as_uint(t);
  u += 0x7FFFFu + ((u >> 20) & 1u);                         // keep 3 mantissa bits, ties to even
  const uint32_t c = (u >> 20) - (120u << 3);                // exponent bias 127 -> 7
  return c > 0x7Eu ? 0x7Eu : c;
}
__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  return c >= 8u ? __uint_as_float((c + (120u << 3)) << 20) : (float)c * 0.001953125f;
}

// Per-block constants for quantizing one block.  The quotient |x| / (s r) is
// formed as (|x| 2^-e) / s: the power-of-two scaling is exact, and s is a
// normal FP32 number, so the division stays out of the FP32 subnormal range
// (where the remainder of the correction step would not be exact).  With the
// FP32 tensor scale, inv_r = R and |x| * inv_r is the recipe's rounded product
// u itself; u / s is again correctly rounded, and since u has 24 significant
// bits and every threshold (midpoint times s) at most 7, an exact quotient off
// a threshold lies more than half an ulp from it, so the rounded quotient
// takes the same side (a quotient below 2^-126 is far below the first one).
struct BlockQ {
  float s;      // block scale (0 if it rounds to 0)
  float rcp;    // correctly rounded 1/s
  float inv_r;  // 2^-e
  uint32_t sc;  // E4M3 code of s
};

// Smallest E4M3FN code whose value is >= X / 6 (X = blockmax / r <= 2688, so
// no saturation): round t = RN32(X / 6) up on the grid, then correct by one
// step with exact comparisons (6 * value has at most 6 significant bits).
__device__ __forceinline__ uint32_t e4m3_encode_up(float X) {
  const float t = div6_rn(X);
  uint32_t c = e4m3_encode(t);                         // nearest, then step to the ceiling
  if (c < 0x7Eu && 6.0f * e4m3_decode(c) < X) ++c;
  if (c > 0u && 6.0f * e4m3_decode(c - 1u) >= X) --c;
  return c;
}

__device__ __forceinline__ BlockQ block_setup(float bmax, float r, float inv_r, bool round_up = false) {
  (void)r;
  BlockQ q;
  const float X = bmax * inv_r;                        // |x| / r exactly, or the largest u of the block
  q.sc = round_up ? e4m3_encode_up(X) : e4m3_encode(div6_rn(X));
  q.s = e4m3_decode(q.sc);
  q.rcp = q.s != 0.0f ? recip_rn(q.s) : 0.0f;          // s >= 2^-9: normal, with a normal reciprocal
  q.inv_r = inv_r;
  return q;
}

// Correctly rounded |x| / (s r) with the sign of x (0 with x's sign if s == 0:
// then rcp == 0, so q0 == 0, rem == ax and the correction adds ax * 0).
__device__ __forceinline__ float block_quot(float x, const BlockQ& q) {
  const float ax = fabsf(x) * q.inv_r;
  const float q0 = __fmul_rn(ax, q.rcp);
  const float rem = __builtin_fmaf(-q0, q.s, ax);
  const float v = __builtin_fmaf(rem, q.rcp, q0);
  return __builtin_copysignf(v, x);
}

// 8 consecutive elements -> 8 packed E2M1 codes (element 0 in the low nibble).
__device__ __forceinline__ uint32_t encode8(const float* x, const BlockQ& q) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, block_quot(x[0], q), block_quot(x[1], q), 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, block_quot(x[2], q), block_quot(x[3], q), 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, block_quot(x[4], q), block_quot(x[5], q), 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, block_quot(x[6], q), block_quot(x[7], q), 1.0f, 3);
  return w;
}

__device__ __forceinline__ float absmax8(const float* x) {
  float m = fabsf(x[0]);
#pragma unroll
  for (int i = 1; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Wave and workgroup reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Dequantize 8 packed E2M1 codes (one 32-bit word) times a block multiplier m
// (= s * r, exactly representable in FP32) into 8 floats.
__device__ __forceinline__ void decode8_f32(uint32_t w, float m, float* out) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  float2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  float2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  out[0] = a.x * m; out[1] = a.y * m; out[2] = b.x * m; out[3] = b.y * m;
  out[4] = c.x * m; out[5] = c.y * m; out[6] = d.x * m; out[7] = d.y * m;
}

}  // namespace pact
