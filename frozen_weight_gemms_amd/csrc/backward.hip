// SiLU-multiply and RMSNorm backward from the saved NVFP4 state (PACT,
// Appendix Table 7: "FP32 reconstruction and derivatives, BF16 gradients" for
// SiLU-multiply; "FP32 reconstruction and reduction, BF16 gradient" for
// RMSNorm).  Both are HBM-bound elementwise / row-reduction kernels.
//
//   silu_mul_bwd: a^ = deq(gate_q), b^ = deq(up_q), sigma = 1/(1+e^-a^)
//                 dgate = dh b^ sigma (1 + a^ (1 - sigma)),  dup = dh a^ sigma
//   rmsnorm_bwd:  y^ = deq(y_q)
//                 dx = rstd (g dy - (y^ / g) (1/H) sum_j dy_j y^_j)
#include "pact_internal.h"

namespace pact {

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
    const uint32_t wa = reinterpret_cast<const uint32_t*>(gc)[q];
    const uint32_t wb = reinterpret_cast<const uint32_t*>(uc)[q];
    const float ma = __builtin_amdgcn_cvt_f32_fp8((int)gs[row * (I >> 4) + (c >> 1)], 0) * gr[row];
    const float mb = __builtin_amdgcn_cvt_f32_fp8((int)us[row * (I >> 4) + (c >> 1)], 0) * ur[row];
    float a[8], b[8], d[8];
    decode8_f32(wa, ma, a);
    decode8_f32(wb, mb, b);
    unpack_bf16x8(*reinterpret_cast<const uint4*>(dh + e0), d);
    float da[8], db[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float en = expf(-fabsf(a[t]));                 // no overflow for either sign
      const float sig = a[t] >= 0.0f ? 1.0f / (1.0f + en) : en / (1.0f + en);
      const float tt = 1.0f + a[t] * (1.0f - sig);
      da[t] = ((d[t] * b[t]) * sig) * tt;
      db[t] = (d[t] * a[t]) * sig;
    }
    uint4 oa, ob;
    oa.x = pack_bf16x2(da[0], da[1]); oa.y = pack_bf16x2(da[2], da[3]);
    oa.z = pack_bf16x2(da[4], da[5]); oa.w = pack_bf16x2(da[6], da[7]);
    ob.x = pack_bf16x2(db[0], db[1]); ob.y = pack_bf16x2(db[2], db[3]);
    ob.z = pack_bf16x2(db[4], db[5]); ob.w = pack_bf16x2(db[6], db[7]);
    *reinterpret_cast<uint4*>(dgate + e0) = oa;
    *reinterpret_cast<uint4*>(dup + e0) = ob;
  }
}

// One 256-thread workgroup per row; NCH 8-element chunks per thread in registers.
template <int NCH>
__global__ __launch_bounds__(256) void k_rmsnorm_bwd(const uint8_t* __restrict__ yc, const uint8_t* __restrict__ ys,
                                                     const float* __restrict__ yr, const float* __restrict__ rstd,
                                                     const uint16_t* __restrict__ gain, const uint16_t* __restrict__ dy,
                                                     int64_t H, uint16_t* __restrict__ dx) {
  __shared__ double red[4];
  const int64_t row = blockIdx.x;
  const int nchunk = (int)(H >> 3);
  float y[NCH][8], d[NCH][8];
  double dot = 0.0;
  const float rr = yr[row];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c < nchunk) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(yc + row * (H >> 1) + 4 * c);
      const float m = __builtin_amdgcn_cvt_f32_fp8((int)ys[row * (H >> 4) + (c >> 1)], 0) * rr;
      decode8_f32(w, m, y[i]);
      unpack_bf16x8(*reinterpret_cast<const uint4*>(dy + row * H + 8 * c), d[i]);
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) { y[i][t] = 0.0f; d[i][t] = 0.0f; }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) dot += (double)d[i][t] * (double)y[i][t];
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dot;
  __syncthreads();
  const float mean = (float)(((red[0] + red[1]) + (red[2] + red[3])) / (double)H);
  const float rs = rstd[row];
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = threadIdx.x + 256 * i;
    if (c >= nchunk) continue;
    float g[8], o[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(gain + 8 * c), g);
#pragma unroll
    for (int t = 0; t < 8; ++t) o[t] = rs * (g[t] * d[i][t] - (y[i][t] / g[t]) * mean);
    uint4 v;
    v.x = pack_bf16x2(o[0], o[1]); v.y = pack_bf16x2(o[2], o[3]);
    v.z = pack_bf16x2(o[4], o[5]); v.w = pack_bf16x2(o[6], o[7]);
    *reinterpret_cast<uint4*>(dx + row * H + 8 * c) = v;
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

hipError_t launch_rmsnorm_bwd(const uint8_t* yc, const uint8_t* ys, const float* yr, const float* rstd,
                              const uint16_t* gain, const uint16_t* dy, int64_t M, int64_t H, uint16_t* dx,
                              hipStream_t s) {
  const int nch = (int)(((H >> 3) + 255) / 256);
  const dim3 grid((unsigned)M);
  if (nch <= 1) k_rmsnorm_bwd<1><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, H, dx);
  else if (nch <= 2) k_rmsnorm_bwd<2><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, H, dx);
  else if (nch <= 4) k_rmsnorm_bwd<4><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, H, dx);
  else if (nch <= 8) k_rmsnorm_bwd<8><<<grid, 256, 0, s>>>(yc, ys, yr, rstd, gain, dy, H, dx);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pact
