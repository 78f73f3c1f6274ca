// SiLU-multiply and RMSNorm backward from the saved NVFP4 state (PACT,
// Appendix Table 7, rows "SiLU-multiply", "RMSNorm" and "Residuals", backward
// column: both operators rebuild their inputs from the NVFP4 copies and work
// in FP32, RMSNorm adding a row reduction; gradients leave as BF16, and the
// residual gradients are summed in BF16).  HBM-bound elementwise /
// row-reduction kernels.
//
//   silu_mul_bwd: a^ = deq(gate_q), b^ = deq(up_q), sigma = 1/(1+E(-a^))
//                 dgate = ((dh b^) sigma) (1 + a^ (1 - sigma)),  dup = (dh a^) sigma
//   rmsnorm_bwd:  y^ = deq(y_q), S = sum_j dy_j y^_j (exact, rounded once to
//                 float64), mean = fp32(S / H)
//                 dx = rstd ((g dy) - ((y^ / g) mean))
// Every FP32 step is one IEEE round-to-nearest operation in the order written
// (no contraction), and E is the pinned exponential of the forward SiLU (whose
// own steps are fused multiply-adds), so the BF16 gradients are reproducible
// bit for bit.
//
// The quantize-on-emit variants also write the NVFP4 copy of what they store
// (the input of the next input-gradient GEMM): silu_mul_bwd_quant emits
// Q(dgate), Q(dup) next to the BF16 gradients the LoRA backward needs, and
// rmsnorm_bwd_residual adds the incoming residual gradient in BF16
// (out = bf16(bf16(dx) + resid)) and can emit Q(out).
#include "mxfp4_device.h"
#include "pact_internal.h"
#include "row_ops.h"

namespace pact {

// The sigmoid per element, its rare IEEE division behind a branch: a chunk
// test on the largest denominator (as in the forward SiLU) measured slower
// here, where keeping the chunk's inputs for the redo costs occupancy.
__device__ __forceinline__ void silu_bwd_elem(float a, float b, float d, float& da, float& db) {
  const float sig = sigmoid_pinned(a);
  const float t = __fmul_rn(__fmul_rn(d, b), sig);
  const float w = __fadd_rn(1.0f, __fmul_rn(a, __fsub_rn(1.0f, sig)));
  da = __fmul_rn(t, w);
  db = __fmul_rn(__fmul_rn(d, a), sig);
}

// Decode one chunk of a and b, load dh, and form the BF16 gradients (packed).
__device__ __forceinline__ void silu_bwd_chunk(uint32_t wa, float ma, uint32_t wb, float mb, const uint4& vd,
                                               uint4& oa, uint4& ob) {
  float a[8], b[8], d[8], da[8], db[8];
  decode8_f32(wa, ma, a);
  decode8_f32(wb, mb, b);
  unpack_bf16x8(vd, d);
#pragma unroll
  for (int t = 0; t < 8; ++t) silu_bwd_elem(a[t], b[t], d[t], da[t], db[t]);
  oa.x = pack_bf16x2(da[0], da[1]); oa.y = pack_bf16x2(da[2], da[3]);
  oa.z = pack_bf16x2(da[4], da[5]); oa.w = pack_bf16x2(da[6], da[7]);
  ob.x = pack_bf16x2(db[0], db[1]); ob.y = pack_bf16x2(db[2], db[3]);
  ob.z = pack_bf16x2(db[4], db[5]); ob.w = pack_bf16x2(db[6], db[7]);
}

__device__ __forceinline__ float absmax_bf16x8(const uint4& v) {
  float f[8];
  unpack_bf16x8(v, f);
  return absmax8(f);
}

// One thread per 8-element chunk (one 32-bit word of codes).
__global__ __launch_bounds__(256) void k_silu_mul_bwd(const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs,
                                                      const float* __restrict__ gr, const uint8_t* __restrict__ uc,
                                                      const uint8_t* __restrict__ us, const float* __restrict__ ur,
                                                      const uint16_t* __restrict__ dh, int64_t M, int64_t I,
                                                      uint16_t* __restrict__ dgate, uint16_t* __restrict__ dup) {
  const int64_t nchunk_row = I >> 3;
  const int64_t total = M * nchunk_row;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total; q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = q / nchunk_row, c = q - row * nchunk_row;
    const int64_t e0 = row * I + 8 * c;
    const float ma = e4m3_decode_hw(gs[row * (I >> 4) + (c >> 1)]) * gr[row];
    const float mb = e4m3_decode_hw(us[row * (I >> 4) + (c >> 1)]) * ur[row];
    uint4 oa, ob;
    silu_bwd_chunk(reinterpret_cast<const uint32_t*>(gc)[q], ma, reinterpret_cast<const uint32_t*>(uc)[q], mb,
                   load16(dh + e0), oa, ob);
    *reinterpret_cast<uint4*>(dgate + e0) = oa;
    *reinterpret_cast<uint4*>(dup + e0) = ob;
  }
}

// silu_mul_bwd with NVFP4 copies of both gradients: one 256-thread workgroup
// per row, NCH chunks per thread kept (as BF16) in registers until the row
// maxima are known.  MX: the saved state and the copies are MXFP4 (32-element
// blocks, E8M0 scales, no row scales: gr, ur, qgr, qur unused, no row maxima).
template <int NCH, bool MX>
__global__ __launch_bounds__(256) void k_silu_mul_bwd_quant(
    const uint8_t* __restrict__ gc, const uint8_t* __restrict__ gs, const float* __restrict__ gr,
    const uint8_t* __restrict__ uc, const uint8_t* __restrict__ us, const float* __restrict__ ur,
    const uint16_t* __restrict__ dh, int64_t I, uint16_t* __restrict__ dgate, uint16_t* __restrict__ dup,
    uint8_t* __restrict__ qgc, uint8_t* __restrict__ qgs, float* __restrict__ qgr, uint8_t* __restrict__ quc,
    uint8_t* __restrict__ qus, float* __restrict__ qur) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nchunk = (int)(I >> 3);
  const float rg = MX ? 1.0f : gr[row], ru = MX ? 1.0f : ur[row];
  constexpr int SSH = MX ? 5 : 4;                      // log2 of the block length
  uint4 oa[NCH], ob[NCH];
  float la = 0.0f, lb = 0.0f;
  // every chunk's inputs are loaded (branch-free) before any is used
  uint32_t wg[NCH], wu[NCH], sg[NCH], su[NCH];
  uint4 vdh[NCH];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    const bool ok = c < nchunk;
    const int64_t q = row * nchunk + c;
    wg[i] = load_or_zero(reinterpret_cast<const uint32_t*>(gc) + q, reinterpret_cast<const uint32_t*>(gc), ok);
    wu[i] = load_or_zero(reinterpret_cast<const uint32_t*>(uc) + q, reinterpret_cast<const uint32_t*>(uc), ok);
    sg[i] = load_or_zero(gs + row * (I >> SSH) + (c >> (SSH - 3)), gs, ok);
    su[i] = load_or_zero(us + row * (I >> SSH) + (c >> (SSH - 3)), us, ok);
    vdh[i] = load_or_zero(reinterpret_cast<const uint4*>(dh + row * I + 8 * c), reinterpret_cast<const uint4*>(dh), ok);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      const float ma = MX ? e8m0_decode(sg[i]) : e4m3_decode_hw(sg[i]) * rg;
      const float mb = MX ? e8m0_decode(su[i]) : e4m3_decode_hw(su[i]) * ru;
      silu_bwd_chunk(wg[i], ma, wu[i], mb, vdh[i], oa[i], ob[i]);
      *reinterpret_cast<uint4*>(dgate + row * I + 8 * c) = oa[i];
      *reinterpret_cast<uint4*>(dup + row * I + 8 * c) = ob[i];
      la = fmaxf(la, absmax_bf16x8(oa[i]));
      lb = fmaxf(lb, absmax_bf16x8(ob[i]));
    } else {
      oa[i] = make_uint4(0, 0, 0, 0);
      ob[i] = make_uint4(0, 0, 0, 0);
    }
  }
  if constexpr (MX) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + 256 * i;
      float f[8];
      unpack_bf16x8(oa[i], f);
      mx_quant_chunk(f, c < nchunk, qgc + row * (I >> 1), qgs + row * (I >> 5), c);
      unpack_bf16x8(ob[i], f);
      mx_quant_chunk(f, c < nchunk, quc + row * (I >> 1), qus + row * (I >> 5), c);
    }
    return;
  }
  const float amax_a = block_max_256(la, red);
  const float amax_b = block_max_256(lb, red);
  const int ea = row_exponent(amax_a), eb = row_exponent(amax_b);
  const float ra = pow2f(ea), ira = pow2f(-ea), rb = pow2f(eb), irb = pow2f(-eb);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    float f[8];
    unpack_bf16x8(oa[i], f);
    quant_chunk(f, c < nchunk, ra, ira, qgc + row * (I >> 1), qgs + row * (I >> 4), c);
    unpack_bf16x8(ob[i], f);
    quant_chunk(f, c < nchunk, rb, irb, quc + row * (I >> 1), qus + row * (I >> 4), c);
  }
  if (threadIdx.x == 0) {
    qgr[row] = ra;
    qur[row] = rb;
  }
}

// RMSNorm backward, optionally + residual gradient and + NVFP4 copy of the
// result.  One 256-thread workgroup per row; NCH 8-element chunks per thread.
// One row per WPR waves (the quantizer's row layout): lane l of the row's
// wave p owns the 16-element blocks l + 64 p + 64 WPR i.  Between passes it
// keeps the raw codes, scale byte and BF16 bits of its blocks and decodes them
// again where needed (the same operations, so the same values).
// MX: y_q and the copy are MXFP4 (32-element blocks on lanes 2p, 2p + 1, E8M0
// scales; yr and qr unused).
template <int NB, int WPR, bool MX>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint8_t* __restrict__ yc, const uint8_t* __restrict__ ys,
                                                     const float* __restrict__ yr, const float* __restrict__ rstd,
                                                     const uint16_t* __restrict__ gain, const uint16_t* __restrict__ dy,
                                                     int64_t M, int64_t H, const uint16_t* __restrict__ resid,
                                                     uint16_t* __restrict__ dx, uint8_t* __restrict__ qc,
                                                     uint8_t* __restrict__ qs, float* __restrict__ qr) {
  __shared__ double dred[2][4];
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = wave % WPR;
  const int64_t row0 = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
  const bool row_ok = row0 < M;                        // uniform per wave (no early exit: barriers below)
  const int64_t row = row_ok ? row0 : 0;
  const int nblk = (int)(H >> 4);
  const float rr = MX ? 1.0f : yr[row];
  uint2 cw[NB];                                        // 16 codes
  float sm[NB];                                        // block scale * row scale
  uint4 dv[NB][2];                                     // 16 BF16 dy
  uint32_t sb[NB];                                     // raw E4M3 block scales
  double sh = 0.0, sl = 0.0;                           // double-double partial of sum dy y^ (each product exact)
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    const bool ok = row_ok && blk < nblk;
    cw[i] = ok ? *reinterpret_cast<const uint2*>(yc + row * (H >> 1) + 8 * blk) : make_uint2(0, 0);
    sb[i] = MX ? load_or_zero(ys + row * (H >> 5) + (blk >> 1), ys, ok)
               : load_or_zero(ys + row * (H >> 4) + blk, ys, ok);      // decoded once every load is issued
    dv[i][0] = ok ? load16(dy + row * H + 16 * blk) : make_uint4(0, 0, 0, 0);
    dv[i][1] = ok ? load16(dy + row * H + 16 * blk + 8) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
    sm[i] = row_ok && lane + 64 * part + 64 * WPR * i < nblk ? (MX ? e8m0_decode(sb[i]) : e4m3_decode_hw(sb[i]) * rr)
                                                             : 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float y[8], d[8];
      decode8_f32(h ? cw[i].y : cw[i].x, sm[i], y);
      unpack_bf16x8(dv[i][h], d);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        double s2, e2;
        two_sum(sh, (double)d[t] * (double)y[t], s2, e2);
        sh = s2;
        sl += e2;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double oh = __shfl_xor(sh, o, 64), ol = __shfl_xor(sl, o, 64);
    double s2, e2;
    two_sum(sh, oh, s2, e2);
    sh = s2;
    sl = sl + ol + e2;
  }
  if constexpr (WPR > 1) {
    if (lane == 0) { dred[0][wave] = sh; dred[1][wave] = sl; }
    __syncthreads();
    const int w0 = wave - part;
    sh = dred[0][w0];
    sl = dred[1][w0];
    for (int k = 1; k < WPR; ++k) {
      double s2, e2;
      two_sum(sh, dred[0][w0 + k], s2, e2);
      sh = s2;
      sl = sl + dred[1][w0 + k] + e2;
    }
  }
  const double S = sh + sl;                            // the double-double value rounded once to float64
  const float mean = (float)(S / (double)H);
  const float rs = rstd[row];
  uint4 out[NB][2];
  float lmax = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    out[i][0] = out[i][1] = make_uint4(0, 0, 0, 0);
    if (!row_ok || blk >= nblk) continue;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float y[8], d[8], g[8], o[8];
      decode8_f32(h ? cw[i].y : cw[i].x, sm[i], y);
      unpack_bf16x8(dv[i][h], d);
      unpack_bf16x8(load16(gain + 16 * blk + 8 * h), g);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        o[t] = __fmul_rn(rs, __fsub_rn(__fmul_rn(g[t], d[t]), __fmul_rn(__fdiv_rn(y[t], g[t]), mean)));
      if (resid != nullptr) {
        float rv[8];
        unpack_bf16x8(load16(resid + row * H + 16 * blk + 8 * h), rv);
#pragma unroll
        for (int t = 0; t < 8; ++t) o[t] = __fadd_rn(__uint_as_float(f32_to_bf16_rne(o[t]) << 16), rv[t]);
      }
      uint4 v;
      v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
      v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
      *reinterpret_cast<uint4*>(dx + row * H + 16 * blk + 8 * h) = v;
      out[i][h] = v;
      lmax = fmaxf(lmax, absmax_bf16x8(v));
    }
  }
  if (MX && qc != nullptr) {
    if (!row_ok) return;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = lane + 64 * part + 64 * WPR * i;
      float f[16];
      unpack_bf16x8(out[i][0], f);
      unpack_bf16x8(out[i][1], f + 8);
      mx_quant_half(f, fmaxf(absmax8(f), absmax8(f + 8)), blk < nblk, qc + row * (H >> 1), qs + row * (H >> 5), blk);
    }
    return;
  }
  if (!MX && qc != nullptr) {                          // uniform: a kernel argument
    float amax = wave_max(lmax);
    if constexpr (WPR > 1) {
      if (lane == 0) red[wave] = amax;
      __syncthreads();
      const int w0 = wave - part;
#pragma unroll
      for (int k = 0; k < WPR; ++k) amax = fmaxf(amax, red[w0 + k]);
    }
    if (!row_ok) return;
    const int e = row_exponent(amax);
    const float r = pow2f(e), ir = pow2f(-e);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = lane + 64 * part + 64 * WPR * i;
      if (blk < nblk) {
        float f[16];
        unpack_bf16x8(out[i][0], f);
        unpack_bf16x8(out[i][1], f + 8);
        quant_block16(f, fmaxf(absmax8(f), absmax8(f + 8)), r, ir, qc + row * (H >> 1), qs + row * (H >> 4), blk);
      }
    }
    if (lane == 0 && part == 0) qr[row] = r;
  }
}

hipError_t launch_silu_mul_bwd(const uint8_t* gc, const uint8_t* gs, const float* gr, const uint8_t* uc,
                               const uint8_t* us, const float* ur, const uint16_t* dh, int64_t M, int64_t I,
                               uint16_t* dgate, uint16_t* dup, hipStream_t s) {
  const int64_t total = M * (I >> 3);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  k_silu_mul_bwd<<<(unsigned)blocks, 256, 0, s>>>(gc, gs, gr, uc, us, ur, dh, M, I, dgate, dup);
  return hipGetLastError();
}

hipError_t launch_silu_mul_bwd_quant(const uint8_t* gc, const uint8_t* gs, const float* gr, const uint8_t* uc,
                                     const uint8_t* us, const float* ur, const uint16_t* dh, int64_t M, int64_t I,
                                     uint16_t* dgate, uint16_t* dup, uint8_t* qgc, uint8_t* qgs, float* qgr,
                                     uint8_t* quc, uint8_t* qus, float* qur, int mx, hipStream_t s) {
  const int nch = (int)(((I >> 3) + 255) / 256);
  const dim3 grid((unsigned)M);
#define PACT_SMBQ(n)                                                                                         \
  do {                                                                                                      \
    if (mx) k_silu_mul_bwd_quant<n, true><<<grid, 256, 0, s>>>(gc, gs, gr, uc, us, ur, dh, I, dgate, dup, qgc, qgs,  \
                                                              qgr, quc, qus, qur);                          \
    else k_silu_mul_bwd_quant<n, false><<<grid, 256, 0, s>>>(gc, gs, gr, uc, us, ur, dh, I, dgate, dup, qgc, qgs,    \
                                                             qgr, quc, qus, qur);                           \
  } while (0)
  if (nch <= 1) PACT_SMBQ(1);
  else if (nch <= 2) PACT_SMBQ(2);
  else if (nch <= 4) PACT_SMBQ(4);
  else if (nch <= 8) PACT_SMBQ(8);
  else return hipErrorInvalidValue;
#undef PACT_SMBQ
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint8_t* yc, const uint8_t* ys, const float* yr, const float* rstd,
                              const uint16_t* gain, const uint16_t* dy, int64_t M, int64_t H,
                              const uint16_t* resid, uint16_t* dx, uint8_t* qc, uint8_t* qs, float* qr, int mx,
                              hipStream_t s) {
  // the quantizer's row layout: blocks per lane <= 4 (one wave per row up to
  // 4096 columns, two up to 8192, four up to 16384)
  const int64_t nblk = H >> 4;
  if (nblk > 1024) return hipErrorInvalidValue;
  const int wpr = nblk <= 256 ? 1 : (nblk <= 512 ? 2 : 4);
  const int64_t nb = (nblk + 64 * wpr - 1) / (64 * wpr);
  const dim3 grid((unsigned)((M + 4 / wpr - 1) / (4 / wpr)));
#define PACT_RMSB(N, W)                                                                                     \
  do {                                                                                                     \
    if (mx) k_rmsnorm_bwd<N, W, true><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, M, H, resid, dx, qc, qs, qr); \
    else k_rmsnorm_bwd<N, W, false><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, M, H, resid, dx, qc, qs, qr);  \
  } while (0)
  if (wpr == 1 && nb <= 1) PACT_RMSB(1, 1);
  else if (wpr == 1 && nb <= 2) PACT_RMSB(2, 1);
  else if (wpr == 1 && nb <= 3) PACT_RMSB(3, 1);
  else if (wpr == 1) PACT_RMSB(4, 1);
  else if (wpr == 2 && nb <= 3) PACT_RMSB(3, 2);
  else if (wpr == 2) PACT_RMSB(4, 2);
  else if (nb <= 3) PACT_RMSB(3, 4);
  else PACT_RMSB(4, 4);
#undef PACT_RMSB
  return hipGetLastError();
}

}  // namespace pact
