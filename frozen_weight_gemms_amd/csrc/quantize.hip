// BF16 -> NVFP4 quantizers and the fused RMSNorm / SiLU-multiply forward kernels.
//
// PACT quantizes activations and output gradients to NVFP4 for its native
// NVFP4 GEMMs and fuses RMSNorm and SiLU-multiply with that quantization,
// keeping the NVFP4 outputs (plus an FP32 per-token RMSNorm statistic) as the
// backward state (abstract; Appendix Table 7 rows "RMSNorm", "SiLU-multiply").
//
// Mapping on gfx950: one 256-thread workgroup per row.  Thread t owns the
// 8-element chunks t, t+256, ... of its row, loaded with one 16-byte load each
// and kept in registers (NCH chunks per thread), so each row is read from HBM
// exactly once.  A 16-element block is the chunk pair held by lanes 2p and
// 2p+1; its amax is one cross-lane exchange.  The row amax (needed before any
// block scale) is a wave64 butterfly plus a 4-entry LDS exchange.  Codes leave
// as one 32-bit store per chunk (coalesced across the wave), scales as bytes.
#include "mxfp4_device.h"
#include "pact_internal.h"
#include "row_ops.h"

namespace pact {

// --------------------------------------------------------------------------
// nvfp4_quantize, row-wise
// --------------------------------------------------------------------------
// Row-wise quantizer: WPR waves per row (1, 2 or 4), 4 / WPR rows per
// workgroup.  Lane l of the row's wave p owns the 16-element blocks
// l + 64 p + 64 WPR i (two 16-byte loads each), so every block's scale is set
// up once by the lane that holds it; the row maximum is a wave reduction,
// exchanged through LDS when a row spans several waves.  NB = blocks per lane.
// Workgroup `wg` of the row quantizer over one tensor (rows 4 / WPR wg ..).
template <int NB, int WPR>
__device__ __forceinline__ void quantize_rows_wg(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                 int64_t ldx, uint8_t* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, float* __restrict__ rscale,
                                                 int qmode, const float* __restrict__ tensor_amax, int64_t wg) {
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = wave % WPR;
  const int64_t row = wg * (4 / WPR) + wave / WPR;
  const bool row_ok = row < rows;                      // uniform per wave (no early exit: barrier below)
  const int nblk = (int)(cols >> 4);
  const uint16_t* xr = x + (row_ok ? row : 0) * ldx;
  uint4 v[NB][2];
  float bm[NB];
  float lmax = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    const bool ok = row_ok && blk < nblk;
    v[i][0] = ok ? load16(xr + 16 * blk) : make_uint4(0, 0, 0, 0);
    v[i][1] = ok ? load16(xr + 16 * blk + 8) : make_uint4(0, 0, 0, 0);
    float f[16];
    unpack_bf16x8(v[i][0], f);
    unpack_bf16x8(v[i][1], f + 8);
    bm[i] = fmaxf(absmax8(f), absmax8(f + 8));
    lmax = fmaxf(lmax, bm[i]);
  }
  float amax;
  if (tensor_amax != nullptr) {                        // a kernel argument, uniform: one scale for every row
    amax = *tensor_amax;
  } else {
    amax = wave_max(lmax);
    if constexpr (WPR > 1) {
      if (lane == 0) red[wave] = amax;
      __syncthreads();
      const int w0 = wave - part;
#pragma unroll
      for (int k = 0; k < WPR; ++k) amax = fmaxf(amax, red[w0 + k]);
    }
  }
  if (!row_ok) return;
  float r, inv_r;
  row_scale_pair(amax, qmode, r, inv_r);
  uint8_t* crow = codes + row * (cols >> 1);
  uint8_t* srow = scales + row * (cols >> 4);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    if (blk < nblk) {
      float f[16];
      unpack_bf16x8(v[i][0], f);
      unpack_bf16x8(v[i][1], f + 8);
      quant_block16(f, bm[i], r, inv_r, crow, srow, blk, (qmode & kQuantRoundUp) != 0);
    }
  }
  if (lane == 0 && part == 0) rscale[row] = r;
}

template <int NB, int WPR>
__global__ __launch_bounds__(kThreads) void k_quantize_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ rscale, int qmode,
                                                            const float* __restrict__ tensor_amax) {
  quantize_rows_wg<NB, WPR>(x, rows, cols, ldx, codes, scales, rscale, qmode, tensor_amax, (int64_t)blockIdx.x);
}

// Several independent row-wise quantizations (default recipe) of at most 3072
// columns in one launch: workgroup w belongs to the first problem whose
// cumulative workgroup count exceeds w, and runs that problem's one-wave-per-
// row body, so every problem's outputs equal its own launch's.  (Up to 3
// blocks per lane: the 4-block body's registers would lower every problem's
// occupancy.)
__global__ __launch_bounds__(kThreads) void k_quantize_rows_batch(QuantBatch b) {
  int i = 0;
  while (i + 1 < b.n && (int64_t)blockIdx.x >= b.wg_end[i]) ++i;
  const int64_t wg = (int64_t)blockIdx.x - (i > 0 ? b.wg_end[i - 1] : 0);
  switch (b.nb[i]) {
    case 1: quantize_rows_wg<1, 1>(b.x[i], b.rows[i], b.cols[i], b.ldx[i], b.codes[i], b.scales[i], b.rscale[i], 0,
                                   nullptr, wg); break;
    case 2: quantize_rows_wg<2, 1>(b.x[i], b.rows[i], b.cols[i], b.ldx[i], b.codes[i], b.scales[i], b.rscale[i], 0,
                                   nullptr, wg); break;
    default: quantize_rows_wg<3, 1>(b.x[i], b.rows[i], b.cols[i], b.ldx[i], b.codes[i], b.scales[i], b.rscale[i], 0,
                                    nullptr, wg); break;
  }
}

__global__ __launch_bounds__(kThreads) void k_quantize_rows_long(const uint16_t* __restrict__ x, int64_t cols,
                                                                 int64_t ldx, uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 float* __restrict__ rscale, int qmode,
                                                                 const float* __restrict__ tensor_amax) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int nchunk = (int)(cols >> 3);
  const uint16_t* xr = x + row * ldx;
  float lmax = 0.0f;
  for (int c = threadIdx.x; c < nchunk; c += kThreads) {
    float f[8];
    unpack_bf16x8(load16(xr + 8 * c), f);
    lmax = fmaxf(lmax, absmax8(f));
  }
  const float amax = tensor_amax != nullptr ? *tensor_amax : block_max_256(lmax, red);
  float r, inv_r;
  row_scale_pair(amax, qmode, r, inv_r);
  uint8_t* crow = codes + row * (cols >> 1);
  uint8_t* srow = scales + row * (cols >> 4);
  const int nround = (nchunk + kThreads - 1) / kThreads;
  for (int i = 0; i < nround; ++i) {
    const int c = threadIdx.x + kThreads * i;
    float f[8];
    uint4 v = c < nchunk ? load16(xr + 8 * c) : make_uint4(0, 0, 0, 0);
    unpack_bf16x8(v, f);
    quant_chunk(f, c < nchunk, r, inv_r, crow, srow, c, (qmode & kQuantRoundUp) != 0);
  }
  if (threadIdx.x == 0) rscale[row] = r;
}

// --------------------------------------------------------------------------
// nvfp4_quantize with transpose: output row i is column i of x [cols x rows].
// Used offline for the cached backward weight layout W_bwd = Q(W^T).  A
// workgroup owns 64 consecutive output rows; lane i of each wave reads
// x[j][i0 + i] so that a wave's loads are 128 contiguous bytes per j.
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_quantize_cols(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ rscale, int qmode,
                                                            const float* __restrict__ tensor_amax) {
  __shared__ float red[4][64];
  const int li = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + li;
  const bool ok = i < rows;
  const int64_t ic = ok ? i : rows - 1;
  const int64_t nblk = cols >> 4;
  float lmax = 0.0f;
  for (int64_t j = g; j < cols; j += 4) lmax = fmaxf(lmax, fabsf(bf16_lo(x[j * ldx + ic])));
  red[g][li] = lmax;
  __syncthreads();
  const float amax = tensor_amax != nullptr ? *tensor_amax
                                            : fmaxf(fmaxf(red[0][li], red[1][li]), fmaxf(red[2][li], red[3][li]));
  float r, inv_r;
  row_scale_pair(amax, qmode, r, inv_r);
  for (int64_t b = g; b < nblk; b += 4) {
    float f[16];
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      f[t] = bf16_lo(x[(16 * b + t) * ldx + ic]);
      m = fmaxf(m, fabsf(f[t]));
    }
    const BlockQ q = block_setup(m, r, inv_r, (qmode & kQuantRoundUp) != 0);
    const uint32_t w0 = encode8(f, q), w1 = encode8(f + 8, q);
    if (ok) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + i * (cols >> 1) + 8 * b);
      dst[0] = w0;
      dst[1] = w1;
      scales[i * nblk + b] = (uint8_t)q.sc;
    }
  }
  if (ok && g == 0) rscale[i] = r;
}

// --------------------------------------------------------------------------
// rmsnorm_quant
// --------------------------------------------------------------------------
// RMSNorm -> NVFP4 in the row layout of the quantizer: WPR waves per row,
// lane l of the row's wave p owns the 16-element blocks l + 64 p + 64 WPR i.
// Sums over the row are wave reductions, exchanged through LDS (in wave
// order) when a row spans several waves.
template <int NB, int WPR>
__device__ __forceinline__ double row_sum_f64(double v, double* dred, int wave, int part) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  if constexpr (WPR > 1) {
    if ((threadIdx.x & 63) == 0) dred[wave] = v;
    __syncthreads();
    v = dred[wave - part];
#pragma unroll
    for (int k = 1; k < WPR; ++k) v += dred[wave - part + k];
    __syncthreads();
  }
  return v;
}

// MX: the output is MXFP4 (32-element blocks, E8M0 scales, no row scale;
// rscale unused) instead of NVFP4; the FP32 sequence is the same.
template <int NB, int WPR, bool MX>
__global__ __launch_bounds__(kThreads) void k_rmsnorm_quant(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ gain, float eps,
                                                            int64_t M, int64_t H, int64_t ldx,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            float* __restrict__ rscale,
                                                            float* __restrict__ rstd_out, int force_exact) {
  __shared__ double dred[2][4];
  __shared__ float red[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = wave % WPR;
  const int64_t row = (int64_t)blockIdx.x * (4 / WPR) + wave / WPR;
  const bool row_ok = row < M;                         // uniform per wave (no early exit: barriers below)
  const int nblk = (int)(H >> 4);
  const uint16_t* xr = x + (row_ok ? row : 0) * ldx;
  uint4 v[NB][2];
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    const bool ok = row_ok && blk < nblk;
    v[i][0] = ok ? load16(xr + 16 * blk) : make_uint4(0, 0, 0, 0);
    v[i][1] = ok ? load16(xr + 16 * blk + 8) : make_uint4(0, 0, 0, 0);
    float f[16];
    unpack_bf16x8(v[i][0], f);
    unpack_bf16x8(v[i][1], f + 8);
    // the square is exact in float64, so fma(d, d, ss) rounds exactly as ss + d*d
#pragma unroll
    for (int t = 0; t < 16; ++t) ss = __builtin_fma((double)f[t], (double)f[t], ss);
  }
  double S = row_sum_f64<NB, WPR>(ss, dred[0], wave, part);
  // The FP32 result depends on S only through fp32(S/H).  The float64 sum above
  // is within (H + 64) * 2^-53 * S of the exactly rounded sum; unless fp32(S/H)
  // is that close to an FP32 rounding boundary, it is the exactly rounded
  // value.  Otherwise (rarely), recompute S as an error-free double-double sum.
  {
    const double q = S / (double)H;
    const float f = (float)q;
    // neighbours of f (f >= 0 and finite): adjacent bit patterns
    const uint32_t fb = __float_as_uint(f);
    const double lo = fb > 0u ? (double)__uint_as_float(fb - 1u) : 0.0;
    const double hi = (double)__uint_as_float(fb + 1u);
    const double dist = fmin(q - 0.5 * (lo + (double)f), 0.5 * ((double)f + hi) - q);
    const double margin = ((double)H + 64.0) * 2.220446049250313e-16 * q;   // (H+64) * 2^-52 * q
    bool exact = force_exact != 0 || (q > 0.0 && !(dist > margin));
    // uniform per wave; with several waves per row every wave of the
    // workgroup takes the exact path if any row needs it (barriers inside)
    if constexpr (WPR > 1) exact = __syncthreads_or(exact) != 0;
    if (exact) {
      double sh = 0.0, sl = 0.0;
#pragma unroll
      for (int i = 0; i < NB; ++i) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          // scheduling fences keep this rarely taken path from raising the
          // kernel's register count (it would otherwise widen every element to
          // float64 at once)
          __builtin_amdgcn_sched_barrier(0);
          // an opaque copy of the raw bits: stops the compiler from sharing the
          // unpacked values with the passes below and keeping them all live
          uint4 w = v[i][h];
          asm volatile("" : "+v"(w.x), "+v"(w.y), "+v"(w.z), "+v"(w.w));
          float f8[8];
          unpack_bf16x8(w, f8);
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            double s2, e2;
            two_sum(sh, (double)f8[t] * (double)f8[t], s2, e2);
            sh = s2;
            sl += e2;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
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
        __syncthreads();
      }
      S = sh + sl;   // the double-double value rounded once to float64
    }
  }
  const float ms = (float)(S / (double)H);
  const float var = __fadd_rn(ms, eps);
  const float sd = (float)__builtin_sqrt((double)var);        // RN64 then RN32 of sqrt: equals sqrt_rn in FP32
  const float rstd = __fdiv_rn(1.0f, sd);
  // y = (x * rstd) * g: formed once for the block maxima and again, by the same
  // operations, in the quantization pass (cheaper than holding it in registers)
  uint4 gv[NB][2];
  float bm[NB];
  float lmax = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    const bool ok = blk < nblk;
    gv[i][0] = ok ? load16(gain + 16 * blk) : make_uint4(0, 0, 0, 0);
    gv[i][1] = ok ? load16(gain + 16 * blk + 8) : make_uint4(0, 0, 0, 0);
    float f[16], g[16], y[16];
    unpack_bf16x8(v[i][0], f);
    unpack_bf16x8(v[i][1], f + 8);
    unpack_bf16x8(gv[i][0], g);
    unpack_bf16x8(gv[i][1], g + 8);
#pragma unroll
    for (int t = 0; t < 16; ++t) y[t] = __fmul_rn(__fmul_rn(f[t], rstd), g[t]);
    bm[i] = fmaxf(absmax8(y), absmax8(y + 8));
    lmax = fmaxf(lmax, bm[i]);
  }
  if constexpr (MX) {
    // MXFP4: a 32-element block is the 16-element blocks of lanes 2p, 2p + 1
    // (H % 32 == 0, so both halves are in the row or neither); no row scale
    if (!row_ok) return;
    uint8_t* crow = codes + row * (H >> 1);
    uint8_t* srow = scales + row * (H >> 5);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int blk = lane + 64 * part + 64 * WPR * i;
      float f[16], g[16], y[16];
      unpack_bf16x8(v[i][0], f);
      unpack_bf16x8(v[i][1], f + 8);
      unpack_bf16x8(gv[i][0], g);
      unpack_bf16x8(gv[i][1], g + 8);
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = __fmul_rn(__fmul_rn(f[t], rstd), g[t]);
      mx_quant_half(y, bm[i], blk < nblk, crow, srow, blk);
    }
    if (lane == 0 && part == 0) rstd_out[row] = rstd;
    return;
  }
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
  const float r = pow2f(e), inv_r = pow2f(-e);
  uint8_t* crow = codes + row * (H >> 1);
  uint8_t* srow = scales + row * (H >> 4);
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = lane + 64 * part + 64 * WPR * i;
    if (blk < nblk) {
      float f[16], g[16], y[16];
      unpack_bf16x8(v[i][0], f);
      unpack_bf16x8(v[i][1], f + 8);
      unpack_bf16x8(gv[i][0], g);
      unpack_bf16x8(gv[i][1], g + 8);
#pragma unroll
      for (int t = 0; t < 16; ++t) y[t] = __fmul_rn(__fmul_rn(f[t], rstd), g[t]);
      quant_block16(y, bm[i], r, inv_r, crow, srow, blk);
    }
  }
  if (lane == 0 && part == 0) {
    rscale[row] = r;
    rstd_out[row] = rstd;
  }
}

// --------------------------------------------------------------------------
// silu_mul_quant
// --------------------------------------------------------------------------
// MX: MXFP4 outputs (32-element blocks on lanes 4p .. 4p + 3, E8M0 scales, no
// row scales or row maxima; the r* arguments are unused).
template <int NCH, bool MX>
__global__ __launch_bounds__(kThreads) void k_silu_mul_quant(const uint16_t* __restrict__ gate,
                                                             const uint16_t* __restrict__ up, int64_t I,
                                                             int64_t ld, uint8_t* __restrict__ hc,
                                                             uint8_t* __restrict__ hs, float* __restrict__ hr,
                                                             uint8_t* __restrict__ gc, uint8_t* __restrict__ gs,
                                                             float* __restrict__ gr, uint8_t* __restrict__ uc,
                                                             uint8_t* __restrict__ us, float* __restrict__ ur) {
  __shared__ float red[3][4];
  const int64_t row = blockIdx.x;
  const int nchunk = (int)(I >> 3);
  uint4 va[NCH], vb[NCH];
  float h[NCH][8];
  float ma = 0.0f, mb = 0.0f, mh = 0.0f;
  // every chunk's loads are issued (branch-free) before any is used
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const bool ok = c < nchunk;
    va[i] = load_or_zero(reinterpret_cast<const uint4*>(gate + row * ld + 8 * c), reinterpret_cast<const uint4*>(gate), ok);
    vb[i] = load_or_zero(reinterpret_cast<const uint4*>(up + row * ld + 8 * c), reinterpret_cast<const uint4*>(up), ok);
  }
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    float a[8], b[8];
    unpack_bf16x8(va[i], a);
    unpack_bf16x8(vb[i], b);
    silu_mul8(a, b, h[i]);
    ma = fmaxf(ma, absmax8(a));
    mb = fmaxf(mb, absmax8(b));
    mh = fmaxf(mh, absmax8(h[i]));
  }
  if constexpr (MX) {
    const int64_t co = row * (I >> 1), so = row * (I >> 5);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = threadIdx.x + kThreads * i;
      const bool ok = c < nchunk;                  // I % 32 == 0: uniform over a block's four lanes
      float a[8], b[8];
      unpack_bf16x8(va[i], a);
      unpack_bf16x8(vb[i], b);
      mx_quant_chunk(h[i], ok, hc + co, hs + so, c);
      mx_quant_chunk(a, ok, gc + co, gs + so, c);
      mx_quant_chunk(b, ok, uc + co, us + so, c);
    }
    return;
  }
  ma = wave_max(ma);
  mb = wave_max(mb);
  mh = wave_max(mh);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][w] = mh; red[1][w] = ma; red[2][w] = mb; }
  __syncthreads();
  float amx[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) amx[k] = fmaxf(fmaxf(red[k][0], red[k][1]), fmaxf(red[k][2], red[k][3]));
  float r[3], ir[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    const int e = row_exponent(amx[k]);
    r[k] = pow2f(e);
    ir[k] = pow2f(-e);
  }
  const int64_t co = row * (I >> 1), so = row * (I >> 4);
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const bool ok = c < nchunk;
    float a[8], b[8];
    unpack_bf16x8(va[i], a);
    unpack_bf16x8(vb[i], b);
    quant_chunk(h[i], ok, r[0], ir[0], hc + co, hs + so, c);
    quant_chunk(a, ok, r[1], ir[1], gc + co, gs + so, c);
    quant_chunk(b, ok, r[2], ir[2], uc + co, us + so, c);
  }
  if (threadIdx.x == 0) { hr[row] = r[0]; gr[row] = r[1]; ur[row] = r[2]; }
}

// --------------------------------------------------------------------------
// Device self-test of the arithmetic shortcuts the kernels rely on, checked
// exhaustively over every input bit pattern in the stated range against the
// IEEE operation they replace (counts of disagreements, one per check):
//   0: recip_rn(d) == 1/d               d in [2^-126, 2^126)
//   1: div6_rn(x) == x/6                x in [6 * 2^-126, FLT_MAX] (normal quotient)
//   2: sigmoid_pinned(a) == 1/(1 + E(-a)), IEEE division   every non-NaN a
//   3: f32_to_bf16_rne(x) == integer RNE of the bit pattern  every non-NaN x
//   4: e4m3_encode_hw(t) == e4m3_encode(t)   every t in [0, 448]; and
//      e4m3_decode_hw(c) == e4m3_decode(c)   every code c in [0, 0x7E]
// --------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_selftest_arith(int which, uint64_t lo, uint64_t hi,
                                                             unsigned long long* __restrict__ count) {
  const uint64_t step = (uint64_t)gridDim.x * kThreads;
  unsigned long long bad = 0;
  for (uint64_t u = lo + (uint64_t)blockIdx.x * kThreads + threadIdx.x; u <= hi; u += step) {
    const float x = __uint_as_float((uint32_t)u);
    if (x != x) continue;
    bool ok;
    if (which == 0) {
      ok = __float_as_uint(recip_rn(x)) == __float_as_uint(__fdiv_rn(1.0f, x));
    } else if (which == 1) {
      ok = __float_as_uint(div6_rn(x)) == __float_as_uint(__fdiv_rn(x, 6.0f));
    } else if (which == 2) {
      const float ref = __fdiv_rn(1.0f, __fadd_rn(1.0f, exp_pinned(-x)));
      ok = __float_as_uint(sigmoid_pinned(x)) == __float_as_uint(ref);
    } else if (which == 3) {
      const uint32_t b = __float_as_uint(x);
      ok = f32_to_bf16_rne(x) == ((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
    } else {
      ok = e4m3_encode_hw(x) == e4m3_encode(x);
      if (u <= 0x7Eu) ok = ok && __float_as_uint(e4m3_decode_hw((uint32_t)u)) == __float_as_uint(e4m3_decode((uint32_t)u));
    }
    bad += ok ? 0ull : 1ull;
  }
  bad = (unsigned long long)wave_sum_u64(bad);
  if ((threadIdx.x & 63) == 0 && bad != 0) atomicAdd(count + which, bad);
}

__global__ void k_zero_u64x5(unsigned long long* p) {
  if (threadIdx.x < 5) p[threadIdx.x] = 0ull;
}

hipError_t launch_selftest_arith(unsigned long long* counts, hipStream_t s) {
  k_zero_u64x5<<<1, 64, 0, s>>>(counts);
  const uint64_t lo[5] = {0x00800000ull, 0x01C00000ull, 0ull, 0ull, 0ull};
  const uint64_t hi[5] = {0x7E7FFFFFull, 0x7F7FFFFFull, 0xFFFFFFFFull, 0xFFFFFFFFull, 0x43E00000ull};   // 448
  for (int w = 0; w < 5; ++w) k_selftest_arith<<<8192, kThreads, 0, s>>>(w, lo[w], hi[w], counts);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// launchers
// --------------------------------------------------------------------------
static int chunks_per_thread(int64_t cols) { return (int)(((cols >> 3) + kThreads - 1) / kThreads); }

// Tensor amax for the per-tensor scale recipe: max |x| over the logical
// matrix [rows x cols] (row stride ldx), written to *amax (non-negative, so the
// float's bit pattern orders like an unsigned integer and an unsigned atomic
// max combines the workgroups in any order with the same result).
__global__ void k_zero_f32(float* p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p = 0.0f;
}
__global__ __launch_bounds__(kThreads) void k_absmax_vec(const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
                                                         int64_t ldx, unsigned* __restrict__ amax) {
  const int64_t cpr = cols >> 3, total = rows * cpr;
  float m = 0.0f;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total; q += (int64_t)gridDim.x * kThreads) {
    const int64_t row = q / cpr, c = q - row * cpr;
    float f[8];
    unpack_bf16x8(load16(x + row * ldx + 8 * c), f);
    m = fmaxf(m, absmax8(f));
  }
  __shared__ float red[4];
  m = block_max_256(m, red);                   // one atomic per workgroup
  if (threadIdx.x == 0) atomicMax(amax, __float_as_uint(m));
}
__global__ __launch_bounds__(kThreads) void k_absmax_scalar(const uint16_t* __restrict__ x, int64_t rows,
                                                            int64_t cols, int64_t ldx, unsigned* __restrict__ amax) {
  const int64_t total = rows * cols;
  float m = 0.0f;
  for (int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x; q < total; q += (int64_t)gridDim.x * kThreads) {
    const int64_t row = q / cols, c = q - row * cols;
    m = fmaxf(m, fabsf(bf16_lo(x[row * ldx + c])));
  }
  __shared__ float red[4];
  m = block_max_256(m, red);
  if (threadIdx.x == 0) atomicMax(amax, __float_as_uint(m));
}

hipError_t launch_tensor_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* amax,
                                hipStream_t s) {
  k_zero_f32<<<1, 64, 0, s>>>(amax);
  const bool vec = (cols % 8) == 0 && (ldx % 8) == 0 && (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
  const int64_t work = vec ? rows * (cols >> 3) : rows * cols;
  int64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 1024) blocks = 1024;                 // 4 per CU; one atomic each
  if (blocks < 1) blocks = 1;
  unsigned* a = reinterpret_cast<unsigned*>(amax);
  if (vec) k_absmax_vec<<<(unsigned)blocks, kThreads, 0, s>>>(x, rows, cols, ldx, a);
  else k_absmax_scalar<<<(unsigned)blocks, kThreads, 0, s>>>(x, rows, cols, ldx, a);
  return hipGetLastError();
}

hipError_t launch_quantize_ex(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                              int qmode, const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                              float* rscale, hipStream_t s) {
  if (transpose) {
    const unsigned grid = (unsigned)((rows + 63) / 64);
    k_quantize_cols<<<grid, kThreads, 0, s>>>(x, rows, cols, ldx, codes, scales, rscale, qmode, tensor_amax);
    return hipGetLastError();
  }
  // blocks per lane <= 4: one wave per row up to 4096 columns, two up to 8192, four up to 16384
  const int64_t nblk = cols >> 4;
  const int wpr = nblk <= 256 ? 1 : (nblk <= 512 ? 2 : 4);
  const int64_t nb = (nblk + 64 * wpr - 1) / (64 * wpr);
  const dim3 grid((unsigned)((rows + 4 / wpr - 1) / (4 / wpr)));
#define PACT_QR(N, W) \
  k_quantize_rows<N, W><<<grid, kThreads, 0, s>>>(x, rows, cols, ldx, codes, scales, rscale, qmode, tensor_amax)
  if (nblk > 1024) k_quantize_rows_long<<<dim3((unsigned)rows), kThreads, 0, s>>>(x, cols, ldx, codes, scales, rscale,
                                                                                  qmode, tensor_amax);
  else if (wpr == 1 && nb <= 1) PACT_QR(1, 1);
  else if (wpr == 1 && nb <= 2) PACT_QR(2, 1);
  else if (wpr == 1 && nb <= 3) PACT_QR(3, 1);
  else if (wpr == 1) PACT_QR(4, 1);
  else if (wpr == 2 && nb <= 3) PACT_QR(3, 2);
  else if (wpr == 2) PACT_QR(4, 2);
  else if (nb <= 3) PACT_QR(3, 4);
  else PACT_QR(4, 4);
#undef PACT_QR
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                           uint8_t* codes, uint8_t* scales, float* rscale, hipStream_t s) {
  return launch_quantize_ex(x, rows, cols, ldx, transpose, 0, nullptr, codes, scales, rscale, s);
}

hipError_t launch_quantize_batch(int n, const uint16_t* const* x, const int64_t* rows, const int64_t* cols,
                                 const int64_t* ldx, uint8_t* const* codes, uint8_t* const* scales,
                                 float* const* rscale, hipStream_t s) {
  QuantBatch b{};
  int64_t wgs = 0;
  for (int i = 0; i < n; ++i) {
    if (rows[i] == 0) continue;
    const int64_t nblk = cols[i] >> 4;
    if (nblk > 192) {
      // more than 3 blocks per lane: a launch of its own
      const hipError_t e = launch_quantize(x[i], rows[i], cols[i], ldx[i], 0, codes[i], scales[i], rscale[i], s);
      if (e != hipSuccess) return e;
      continue;
    }
    const int k = b.n++;
    b.x[k] = x[i];
    b.rows[k] = rows[i];
    b.cols[k] = cols[i];
    b.ldx[k] = ldx[i];
    b.codes[k] = codes[i];
    b.scales[k] = scales[i];
    b.rscale[k] = rscale[i];
    b.nb[k] = nblk > 64 ? (int)((nblk + 63) / 64) : 1;
    wgs += (rows[i] + 3) / 4;
    b.wg_end[k] = wgs;
  }
  if (b.n == 0) return hipSuccess;
  k_quantize_rows_batch<<<dim3((unsigned)wgs), kThreads, 0, s>>>(b);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t H,
                                int64_t ldx, uint8_t* codes, uint8_t* scales, float* rscale, float* rstd,
                                int force_exact, int mx, hipStream_t s) {
  // the quantizer's row layout: blocks per lane <= 4 (one wave per row up to
  // 4096 columns, two up to 8192, four up to 16384)
  const int64_t nblk = H >> 4;
  if (nblk > 1024) return hipErrorInvalidValue;
  const int wpr = nblk <= 256 ? 1 : (nblk <= 512 ? 2 : 4);
  const int64_t nb = (nblk + 64 * wpr - 1) / (64 * wpr);
  const dim3 grid((unsigned)((M + 4 / wpr - 1) / (4 / wpr)));
#define PACT_RMS(N, W)                                                                                          \
  do {                                                                                                         \
    if (mx) k_rmsnorm_quant<N, W, true><<<grid, kThreads, 0, s>>>(x, gain, eps, M, H, ldx, codes, scales, rscale,   \
                                                               rstd, force_exact);                             \
    else k_rmsnorm_quant<N, W, false><<<grid, kThreads, 0, s>>>(x, gain, eps, M, H, ldx, codes, scales, rscale,     \
                                                                rstd, force_exact);                            \
  } while (0)
  if (wpr == 1 && nb <= 1) PACT_RMS(1, 1);
  else if (wpr == 1 && nb <= 2) PACT_RMS(2, 1);
  else if (wpr == 1 && nb <= 3) PACT_RMS(3, 1);
  else if (wpr == 1) PACT_RMS(4, 1);
  else if (wpr == 2 && nb <= 3) PACT_RMS(3, 2);
  else if (wpr == 2) PACT_RMS(4, 2);
  else if (nb <= 3) PACT_RMS(3, 4);
  else PACT_RMS(4, 4);
#undef PACT_RMS
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t I, int64_t ld,
                                 uint8_t* hc, uint8_t* hs, float* hr, uint8_t* gc, uint8_t* gs, float* gr,
                                 uint8_t* uc, uint8_t* us, float* ur, int mx, hipStream_t s) {
  const int nch = chunks_per_thread(I);
  const dim3 grid((unsigned)M);
#define PACT_SILU(N)                                                                                         \
  do {                                                                                                      \
    if (mx) k_silu_mul_quant<N, true><<<grid, kThreads, 0, s>>>(gate, up, I, ld, hc, hs, hr, gc, gs, gr, uc, us, ur); \
    else k_silu_mul_quant<N, false><<<grid, kThreads, 0, s>>>(gate, up, I, ld, hc, hs, hr, gc, gs, gr, uc, us, ur);  \
  } while (0)
  if (nch <= 1) PACT_SILU(1);
  else if (nch <= 2) PACT_SILU(2);
  else if (nch <= 4) PACT_SILU(4);
  else if (nch <= 8) PACT_SILU(8);
  else return hipErrorInvalidValue;
#undef PACT_SILU
  return hipGetLastError();
}

}  // namespace pact
