// BF16 rank-r LoRA branch on the reconstructed input (PACT, Appendix Table 7
// row "LoRA branch": BF16 GEMMs on reconstructed inputs forward; BF16 adapter
// gradients and input gradients backward; saved state is the shared NVFP4
// input and the BF16 adapters; Figure 3's caption describes the same split).
//
//   lora_down : T  = bf16(X~ A^T)             X~ = deq(X_q), exact in BF16
//   lora_bwd  : T  = bf16(X~ A^T)             (recomputed into the dT buffer)
//               dB = bf16(s dY^T T)
//               dT = bf16(s dY B)             (overwrites T)
//               dA = bf16(dT^T X~)
// (the input-gradient term dT A is added inside the dgrad GEMM's epilogue).
//
// All four are skinny products Out[P x r] = sum over a long axis R, r <= 128,
// on v_mfma_f32_16x16x32_bf16 with FP32 accumulation:
//   * row-reduction kernel (lora_down, dT): the long operand is read along its
//     rows; a 256-thread workgroup owns 16 output rows and its 4 waves split R,
//     then reduce through LDS.
//   * column-reduction kernel (dB, dA^T): the long operand is read along its
//     columns; a workgroup owns 64 output rows (64 columns of the long operand,
//     one 128-byte row segment for BF16), stages 32 x 64 tiles of it in LDS and
//     each wave reads its 16 columns from there.
#include "pact_internal.h"

namespace pact {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kMaxRank = 128;
constexpr int kNT = kMaxRank / 16;   // max 16-wide output tiles along r

__device__ __forceinline__ __bf16 bfbits(uint16_t v) { return __builtin_bit_cast(__bf16, v); }
__device__ __forceinline__ uint16_t bf16_exact(float f) { return (uint16_t)(__float_as_uint(f) >> 16); }

// 8 dequantized NVFP4 elements times m (= s or s * r), as BF16 (exact).
__device__ __forceinline__ bf16x8_t deq8_bf16(uint32_t w, float m) {
  float f[8];
  decode8_f32(w, m, f);
  bf16x8_t r;
#pragma unroll
  for (int t = 0; t < 8; ++t) r[t] = bfbits(bf16_exact(f[t]));
  return r;
}

// ---------------------------------------------------------------------------
// Row reduction: Out[p][j] = post(p) * sum_R L[p][R] * W(R, j)
//   L_NVFP4: L = deq(x) without the row scale; post(p) = scale * rscale[p]
//   else   : L = BF16 matrix [P x R] (leading dim ldl); post(p) = scale
//   W(R, j) = w[R * wsR + j * wsJ]
// ---------------------------------------------------------------------------
template <bool L_NVFP4>
__global__ __launch_bounds__(256) void k_lora_rowred(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                     const float* __restrict__ xr, const uint16_t* __restrict__ lb,
                                                     int64_t ldl, int64_t P, int64_t R, const uint16_t* __restrict__ w,
                                                     int64_t wsR, int64_t wsJ, int64_t r, float scale,
                                                     uint16_t* __restrict__ out) {
  __shared__ float red[4][16][kMaxRank + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * 16;
  int64_t p = p0 + i;
  p = p < P ? p : P - 1;
  const int ntile = (int)((r + 15) / 16);
  floatx4 acc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) acc[t] = floatx4{0, 0, 0, 0};

  const int64_t nsteps = (R + 31) / 32;
  for (int64_t st = wave; st < nsteps; st += 4) {
    const int64_t k = st * 32 + 8 * g;         // this lane's 8 elements along R
    const bool kin = k < R;                    // R % 16 == 0 for NVFP4; BF16 R % 8 == 0
    bf16x8_t af;
    if (L_NVFP4) {
      uint32_t wd = 0;
      float sc = 0.0f;
      if (kin) {
        wd = *reinterpret_cast<const uint32_t*>(xc + p * (R >> 1) + (k >> 1));
        sc = __builtin_amdgcn_cvt_f32_fp8((int)xs[p * (R >> 4) + (k >> 4)], 0);
      }
      af = deq8_bf16(wd, sc);
    } else {
      uint4 v = kin ? *reinterpret_cast<const uint4*>(lb + p * ldl + k) : make_uint4(0, 0, 0, 0);
      af = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      if (t < ntile) {
        const int64_t j = t * 16 + i;
        bf16x8_t bf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool ok = kin && j < r;
          bf[e] = bfbits(ok ? w[(k + e) * wsR + j * wsJ] : (uint16_t)0);
        }
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[t], 0, 0, 0);
      }
    }
  }
  // accumulator layout: element (row, col) at lane col + 16 * (row / 4), reg row % 4
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (t < ntile) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[wave][4 * g + e][t * 16 + i] = acc[t][e];
    }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 16 * r; q += 256) {
    const int row = q / (int)r, col = q % (int)r;
    const int64_t pp = p0 + row;
    if (pp < P) {
      const float s = red[0][row][col] + red[1][row][col] + red[2][row][col] + red[3][row][col];
      const float post = L_NVFP4 ? scale * xr[pp] : scale;
      out[pp * r + col] = (uint16_t)f32_to_bf16_rne(s * post);
    }
  }
}

// ---------------------------------------------------------------------------
// Column reduction: Out(p, j) = scale * sum_R Z[R][p] * W[R][j]
//   Z_NVFP4: Z = deq(x) [R x P] including row scales; else BF16 [R x P] (ld ldz)
//   W: BF16 [R x r] row-major.  Out(p, j) is stored at out[p * osP + j * osJ].
// ---------------------------------------------------------------------------
constexpr int ZPAD = 72;   // LDS row stride (elements) of the staged Z tile [32 x 64]

template <bool Z_NVFP4>
__global__ __launch_bounds__(256) void k_lora_colred(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                     const float* __restrict__ xr, const uint16_t* __restrict__ zb,
                                                     int64_t ldz, int64_t R, int64_t P, const uint16_t* __restrict__ w,
                                                     int64_t r, float scale, uint16_t* __restrict__ out, int64_t osP,
                                                     int64_t osJ) {
  __shared__ uint16_t zt[32][ZPAD];
  __shared__ uint16_t wt[32][kMaxRank + 8];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  const int ntile = (int)((r + 15) / 16);
  floatx4 acc[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t) acc[t] = floatx4{0, 0, 0, 0};

  for (int64_t R0 = 0; R0 < R; R0 += 32) {
    // stage Z[R0 .. R0+32][p0 .. p0+64] as BF16
    if (Z_NVFP4) {
      // 32 rows x 8 chunks of 8 elements: one chunk per thread
      const int row = tid >> 3, ch = tid & 7;
      const int64_t Rr = R0 + row, pc = p0 + 8 * ch;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (Rr < R && pc < P) {
        const uint32_t wd = *reinterpret_cast<const uint32_t*>(xc + Rr * (P >> 1) + (pc >> 1));
        const float m = __builtin_amdgcn_cvt_f32_fp8((int)xs[Rr * (P >> 4) + (pc >> 4)], 0) * xr[Rr];
        float f[8];
        decode8_f32(wd, m, f);
        v.x = bf16_exact(f[0]) | ((uint32_t)bf16_exact(f[1]) << 16);
        v.y = bf16_exact(f[2]) | ((uint32_t)bf16_exact(f[3]) << 16);
        v.z = bf16_exact(f[4]) | ((uint32_t)bf16_exact(f[5]) << 16);
        v.w = bf16_exact(f[6]) | ((uint32_t)bf16_exact(f[7]) << 16);
      }
      *reinterpret_cast<uint4*>(&zt[row][8 * ch]) = v;
    } else {
      const int row = tid >> 3, ch = tid & 7;
      const int64_t Rr = R0 + row, pc = p0 + 8 * ch;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (Rr < R && pc < P) v = *reinterpret_cast<const uint4*>(zb + Rr * ldz + pc);
      *reinterpret_cast<uint4*>(&zt[row][8 * ch]) = v;
    }
    for (int q = tid; q < 32 * r; q += 256) {
      const int row = q / (int)r, col = q % (int)r;
      const int64_t Rr = R0 + row;
      wt[row][col] = Rr < R ? w[Rr * r + col] : (uint16_t)0;
    }
    __syncthreads();
    bf16x8_t af;
#pragma unroll
    for (int e = 0; e < 8; ++e) af[e] = bfbits(zt[8 * g + e][16 * wave + i]);
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      if (t < ntile) {
        const int j = t * 16 + i;
        bf16x8_t bf;
#pragma unroll
        for (int e = 0; e < 8; ++e) bf[e] = bfbits(j < r ? wt[8 * g + e][j] : (uint16_t)0);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int t = 0; t < kNT; ++t) {
    if (t < ntile) {
      const int64_t j = t * 16 + i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t p = p0 + 16 * wave + 4 * g + e;
        if (p < P && j < r) out[p * osP + j * osJ] = (uint16_t)f32_to_bf16_rne(acc[t][e] * scale);
      }
    }
  }
}

hipError_t launch_lora_down(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                            const uint16_t* A, int64_t r, uint16_t* T, hipStream_t s) {
  const unsigned grid = (unsigned)((M + 15) / 16);
  k_lora_rowred<true><<<grid, 256, 0, s>>>(xc, xs, xr, nullptr, 0, M, K, A, 1, K, r, 1.0f, T);
  return hipGetLastError();
}

hipError_t launch_lora_bwd(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                           const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                           int64_t N, uint16_t* dT, uint16_t* dA, uint16_t* dB, hipStream_t s) {
  // T into the dT buffer
  hipError_t e = launch_lora_down(xc, xs, xr, M, K, A, r, dT, s);
  if (e != hipSuccess) return e;
  // dB[n][j] = s * sum_m dY[m][n] T[m][j]
  k_lora_colred<false><<<(unsigned)((N + 63) / 64), 256, 0, s>>>(nullptr, nullptr, nullptr, dy, N, M, N, dT, r,
                                                                 scale, dB, r, 1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dT[m][j] = s * sum_n dY[m][n] B[n][j]
  k_lora_rowred<false><<<(unsigned)((M + 15) / 16), 256, 0, s>>>(nullptr, nullptr, nullptr, dy, N, M, N, B, r, 1,
                                                                 r, scale, dT);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dA[j][k] = sum_m dT[m][j] X~[m][k]
  k_lora_colred<true><<<(unsigned)((K + 63) / 64), 256, 0, s>>>(xc, xs, xr, nullptr, 0, M, K, dT, r, 1.0f, dA, 1,
                                                                K);
  return hipGetLastError();
}

}  // namespace pact
