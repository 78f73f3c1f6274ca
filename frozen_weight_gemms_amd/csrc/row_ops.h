// Device helpers for the row-per-workgroup kernels (quantizers, fused forward
// and backward kernels): workgroup reductions, the per-chunk NVFP4 encoder,
// an error-free float64 sum and the pinned FP32 exponential.
#pragma once

#include "nvfp4_device.h"

namespace pact {

constexpr int kThreads = 256;

__device__ __forceinline__ float block_max_256(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// E4M3FN code and value by the hardware FP8 conversions (v_cvt_pk_fp8_f32,
// round to nearest even; v_cvt_f32_fp8).  For t in [0, 448] the code equals
// e4m3_encode(t), and for every code 0 .. 0x7E the value equals
// e4m3_decode(c) (the device self-test checks every such t and c).  The
// encoder's argument is clamped to 448 first: e4m3_encode saturates there,
// and so the two agree for every t >= 0 and NaN (which e4m3_encode maps to
// 0x7E as well).
__device__ __forceinline__ uint32_t e4m3_encode_hw(float t) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(t, 448.0f), 0.0f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_decode_hw(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// block_setup of the row kernels: the same BlockQ, its E4M3 steps by the
// hardware conversions (the round-up recipe keeps the software ceiling).
__device__ __forceinline__ BlockQ block_setup_row(float bmax, float r, float inv_r, bool round_up) {
  if (round_up) return block_setup(bmax, r, inv_r, true);
  BlockQ q;
  q.sc = e4m3_encode_hw(div6_rn(bmax * inv_r));
  q.s = e4m3_decode_hw(q.sc);
  q.rcp = q.s != 0.0f ? recip_rn(q.s) : 0.0f;
  q.inv_r = inv_r;
  return q;
}

// Quantize one chunk (8 floats) of a row whose exponent is known.  Both lanes
// of the pair must call this (it exchanges the chunk amax with lane ^ 1).
__device__ __forceinline__ void quant_chunk(const float* x, bool valid, float r, float inv_r,
                                            uint8_t* codes_row, uint8_t* scales_row, int c, bool round_up = false) {
  float m = valid ? absmax8(x) : 0.0f;
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  if (!valid) return;
  const BlockQ q = block_setup_row(m, r, inv_r, round_up);
  const uint32_t w = encode8(x, q);
  *reinterpret_cast<uint32_t*>(codes_row + 4 * (int64_t)c) = w;
  if ((c & 1) == 0) scales_row[c >> 1] = (uint8_t)q.sc;
}

// Quantize one whole 16-element block held by one lane (block maximum bmax
// already known): 8 code bytes and the scale byte of block `blk` of the row.
__device__ __forceinline__ void quant_block16(const float* x, float bmax, float r, float inv_r, uint8_t* codes_row,
                                              uint8_t* scales_row, int blk, bool round_up = false) {
  const BlockQ q = block_setup_row(bmax, r, inv_r, round_up);
  const uint32_t w0 = encode8(x, q);
  const uint32_t w1 = encode8(x + 8, q);
  *reinterpret_cast<uint2*>(codes_row + 8 * (int64_t)blk) = make_uint2(w0, w1);
  scales_row[blk] = (uint8_t)q.sc;
}

// Error-free sum of two doubles.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// FP32 exponential: Cody-Waite reduction with ln 2 split in two (the high part
// has 16 significant bits, so n * LN2_HI is exact for |n| <= 128), then the
// degree-7 Taylor polynomial of e^r in Horner form; each reduction and Horner
// step is one fused multiply-add (a single IEEE round to nearest), the other
// operations plain round-to-nearest ones.
//   L2E    = RN32(1 / ln 2)          = 0x3FB8AA3B
//   LN2_HI = ln 2 to 16 significant bits = 0x3F317200
//   LN2_LO = RN32(ln 2 - LN2_HI)     = 0x35BFBE8E
//   C_k    = RN32(1 / k!)            k = 2..7: 0x3F000000 0x3E2AAAAB 0x3D2AAAAB 0x3C088889 0x3AB60B61 0x39500D01
__device__ __forceinline__ float exp_pinned(float x) {
  const float L2E = __uint_as_float(0x3FB8AA3Bu);
  const float LN2_HI = __uint_as_float(0x3F317200u);
  const float LN2_LO = __uint_as_float(0x35BFBE8Eu);
  const float xc = fminf(fmaxf(x, -80.0f), 89.0f);
  const float n = rintf(__fmul_rn(xc, L2E));
  const float rr = __builtin_fmaf(-n, LN2_LO, __builtin_fmaf(-n, LN2_HI, xc));
  float p = __uint_as_float(0x39500D01u);                         // 1/7!
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3AB60B61u));        // 1/6!
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3C088889u));        // 1/5!
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3D2AAAABu));        // 1/4!
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3E2AAAABu));        // 1/3!
  p = __builtin_fmaf(p, rr, 0.5f);
  p = __builtin_fmaf(p, rr, 1.0f);
  p = __builtin_fmaf(p, rr, 1.0f);
  float e = __builtin_ldexpf(p, (int)n);
  e = x < -80.0f ? 0.0f : e;
  e = x > 89.0f ? __builtin_huge_valf() : e;
  return e;
}

// The sigmoid's denominator d = 1 + E(-a).  E's two range selects are left
// out because they cannot change d: below the clamp (-a < -80) E(-80) is about
// 2^-115, and 1 + 2^-115 rounds to 1 = 1 + 0; above it (-a > 89) the clamped
// argument gives n = 128 and a polynomial value above 1, so the ldexp
// overflows to +inf, the value the select would give.  NaN takes neither
// select.  (The device self-test compares the sigmoid below with the full
// E for every non-NaN a.)
__device__ __forceinline__ float sigmoid_den(float a) {
  const float x = -a;
  const float L2E = __uint_as_float(0x3FB8AA3Bu);
  const float LN2_HI = __uint_as_float(0x3F317200u);
  const float LN2_LO = __uint_as_float(0x35BFBE8Eu);
  const float xc = fminf(fmaxf(x, -80.0f), 89.0f);
  const float n = rintf(__fmul_rn(xc, L2E));
  const float rr = __builtin_fmaf(-n, LN2_LO, __builtin_fmaf(-n, LN2_HI, xc));
  float p = __uint_as_float(0x39500D01u);
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3AB60B61u));
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3C088889u));
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3D2AAAABu));
  p = __builtin_fmaf(p, rr, __uint_as_float(0x3E2AAAABu));
  p = __builtin_fmaf(p, rr, 0.5f);
  p = __builtin_fmaf(p, rr, 1.0f);
  p = __builtin_fmaf(p, rr, 1.0f);
  return __fadd_rn(1.0f, __builtin_ldexpf(p, (int)n));
}

// sigma(a) = 1 / (1 + E(-a)) in the pinned FP32 sequence (0 when E overflows),
// the division correctly rounded: recip_rn while 1 + E < 2^126, IEEE division
// beyond (a < -87, where the reciprocal is subnormal or 0).  The forward
// SiLU kernel takes recip_rn(d) for all elements, tracks the largest d (never
// NaN: 1 <= d <= +inf) and redoes a chunk with this function when it reaches
// 2^126, so the per-element division branch is not in its common path.
__device__ __forceinline__ float sigmoid_pinned(float a) {
  const float d = sigmoid_den(a);
  float sig;
  if (d < 0x1p126f) sig = recip_rn(d);
  else sig = __fdiv_rn(1.0f, d);
  return sig;
}

__device__ __forceinline__ float silu_mul(float a, float b) {
  const float sig = sigmoid_pinned(a);
  return __fmul_rn(__fmul_rn(a, sig), b);
}

// silu_mul of 8 elements: recip_rn for every sigmoid, and the chunk redone by
// silu_mul when any denominator reaches 2^126 (the same values either way).
__device__ __forceinline__ void silu_mul8(const float* a, const float* b, float* h) {
  float dmax = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float d = sigmoid_den(a[t]);
    dmax = fmaxf(dmax, d);
    h[t] = __fmul_rn(__fmul_rn(a[t], recip_rn(d)), b[t]);
  }
  if (!(dmax < 0x1p126f)) {
#pragma unroll
    for (int t = 0; t < 8; ++t) h[t] = silu_mul(a[t], b[t]);
  }
}

// Workgroup (256 threads) sum of per-thread double-double partials (sh, sl),
// returned rounded once to float64.  dred: __shared__ double[2][4].
__device__ __forceinline__ double block_sum_dd(double sh, double sl, double (*dred)[4]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double oh = __shfl_xor(sh, o, 64), ol = __shfl_xor(sl, o, 64);
    double s, e;
    two_sum(sh, oh, s, e);
    sh = s;
    sl = sl + ol + e;
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { dred[0][w] = sh; dred[1][w] = sl; }
  __syncthreads();
  sh = dred[0][0];
  sl = dred[1][0];
  for (int k = 1; k < 4; ++k) {
    double s, e;
    two_sum(sh, dred[0][k], s, e);
    sh = s;
    sl = sl + dred[1][k] + e;
  }
  __syncthreads();
  return sh + sl;
}

}  // namespace pact
