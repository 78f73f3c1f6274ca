// BF16 rank-r LoRA branch on the reconstructed input (PACT, Appendix Table 7
// row "LoRA branch": BF16 GEMMs on reconstructed inputs forward; BF16 adapter
// gradients and input gradients backward; saved state is the shared NVFP4
// input and the BF16 adapters; Figure 3's caption describes the same split).
//
//   lora_down : T  = bf16(X~ A^T)             X~ = deq(X_q), exact in BF16
//   lora_bwd  : T  = bf16(X~ A^T)             (recomputed, kept in the workspace)
//               dT = bf16(s dY B)
//               dB = bf16(s dY^T T)
//               dA = bf16(dT^T X~)
// (the input-gradient term dT A is added inside the dgrad GEMM's epilogue).
//
// All of these are skinny products, Out[P x r] = sum over a long axis R with
// r <= 128, on v_mfma_f32_16x16x32_bf16 with FP32 accumulation.  lora_bwd is
// three launches:
//   * the row kernel reduces along rows (T over K from X_q, dT over N from dY):
//     a workgroup owns 16 token rows; each of its waves streams 8 consecutive
//     elements per lane per MFMA step over its share of the long axis, with 8
//     steps of loads in flight, and the waves reduce through LDS;
//   * the column kernel contracts over the token axis M (dB from dY and T, dA
//     from X_q and dT), split over M: a workgroup stages 128-row x 64-column
//     tiles of the long operand in LDS transposed and writes an FP32 partial
//     [64 x r]; a third, small launch sums the partials in split order and
//     writes BF16, so results do not depend on scheduling.
#include "pact_internal.h"

namespace pact {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ __bf16 bfbits(uint16_t v) { return __builtin_bit_cast(__bf16, v); }
__device__ __forceinline__ uint32_t bf16_exact(float f) { return __float_as_uint(f) >> 16; }

// 8 dequantized NVFP4 elements times m (= s or s * r), packed as BF16 (exact).
__device__ __forceinline__ uint4 deq8_bf16_packed(uint32_t w, float m) {
  float f[8];
  decode8_f32(w, m, f);
  uint4 v;
  v.x = bf16_exact(f[0]) | (bf16_exact(f[1]) << 16);
  v.y = bf16_exact(f[2]) | (bf16_exact(f[3]) << 16);
  v.z = bf16_exact(f[4]) | (bf16_exact(f[5]) << 16);
  v.w = bf16_exact(f[6]) | (bf16_exact(f[7]) << 16);
  return v;
}

// ---------------------------------------------------------------------------
// Row kernel.
//   part 0 (waves [0, NW/2) or all waves when DO_DT is false):
//       T[p][j]  = bf16(xr[p] * sum_k (e*s)[p][k] * A[j][k])      (X_q [P x K], A [r x K])
//   part 1 (waves [NW/2, NW), when DO_DT):
//       dT[p][j] = bf16(scale * sum_n dY[p][n] * B[n][j])          (dY [P x N], B [N x r])
// ---------------------------------------------------------------------------
template <int NT>
struct RowUnroll {
  static constexpr int value = NT <= 2 ? 8 : (NT <= 4 ? 4 : 2);   // steps of loads in flight
};

template <int NT, int NWP>
__device__ __forceinline__ void rowred_part(bool nvfp4, const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                            const uint16_t* __restrict__ lb, int64_t p, int64_t R,
                                            const uint16_t* __restrict__ w, int64_t wsR, int64_t wsJ, int64_t r,
                                            int wpart, int i, int g, floatx4* acc) {
  int64_t jrow[NT];
  bool jok[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t j = t * 16 + i;
    jok[t] = j < r;
    jrow[t] = jok[t] ? j : 0;
  }
  const int64_t nsteps = (R + 31) / 32;
  const int64_t per = (nsteps + NWP - 1) / NWP;
  const int64_t st0 = wpart * per, st1 = st0 + per < nsteps ? st0 + per : nsteps;
  constexpr int RR_UNROLL = RowUnroll<NT>::value;
  for (int64_t sb = st0; sb < st1; sb += RR_UNROLL) {
    uint4 lv[RR_UNROLL];
    float ls[RR_UNROLL];
    bf16x8_t bv[RR_UNROLL][NT];
#pragma unroll
    for (int u = 0; u < RR_UNROLL; ++u) {
      const int64_t k = (sb + u) * 32 + 8 * g;
      const bool kin = (sb + u) < st1 && k < R;
      if (nvfp4) {
        lv[u].x = kin ? *reinterpret_cast<const uint32_t*>(xc + p * (R >> 1) + (k >> 1)) : 0u;
        ls[u] = kin ? __builtin_amdgcn_cvt_f32_fp8((int)xs[p * (R >> 4) + (k >> 4)], 0) : 0.0f;
      } else {
        lv[u] = kin ? *reinterpret_cast<const uint4*>(lb + p * R + k) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (wsR == 1) {   // small operand K-contiguous (A [r x K])
          const uint4 v = (kin && jok[t]) ? *reinterpret_cast<const uint4*>(w + jrow[t] * wsJ + k)
                                          : make_uint4(0, 0, 0, 0);
          bv[u][t] = __builtin_bit_cast(bf16x8_t, v);
        } else {          // small operand rank-contiguous (B [N x r]): 8 rows of one column
#pragma unroll
          for (int e = 0; e < 8; ++e)
            bv[u][t][e] = bfbits((kin && jok[t]) ? w[(k + e) * wsR + jrow[t]] : (uint16_t)0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RR_UNROLL; ++u) {
      const uint4 av = nvfp4 ? deq8_bf16_packed(lv[u].x, ls[u]) : lv[u];
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int t = 0; t < NT; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bv[u][t], acc[t], 0, 0, 0);
    }
  }
}

template <int NT, bool DO_DT>
__global__ __launch_bounds__(512) void k_lora_rows(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                   const float* __restrict__ xr, int64_t P, int64_t K,
                                                   const uint16_t* __restrict__ A, int64_t r,
                                                   uint16_t* __restrict__ T, const uint16_t* __restrict__ dy,
                                                   int64_t N, const uint16_t* __restrict__ B, float scale,
                                                   uint16_t* __restrict__ dT) {
  constexpr int NW = 8;
  constexpr int RT = 16 * NT;
  __shared__ float red[NW][16][RT + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t p0 = (int64_t)blockIdx.x * 16;
  int64_t p = p0 + i;
  p = p < P ? p : P - 1;

  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0, 0, 0, 0};
  constexpr int NWP = DO_DT ? NW / 2 : NW;          // waves per part
  const int part = DO_DT ? wave / NWP : 0;
  const int wpart = wave - part * NWP;
  if (part == 0)
    rowred_part<NT, NWP>(true, xc, xs, nullptr, p, K, A, 1, K, r, wpart, i, g, acc);
  else
    rowred_part<NT, NWP>(false, nullptr, nullptr, dy, p, N, B, r, 1, r, wpart, i, g, acc);
  // accumulator layout: (row, col) at lane col + 16 * (row / 4), reg row % 4
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * g + e][t * 16 + i] = acc[t][e];
  __syncthreads();
  for (int q = threadIdx.x; q < (DO_DT ? 2 : 1) * 16 * RT; q += 512) {
    const int prt = q / (16 * RT);
    const int row = (q / RT) % 16, col = q % RT;
    const int64_t pp = p0 + row;
    if (pp < P && col < r) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NWP; ++w) sum += red[prt * NWP + w][row][col];
      if (prt == 0) T[pp * r + col] = (uint16_t)f32_to_bf16_rne(sum * xr[pp]);
      else dT[pp * r + col] = (uint16_t)f32_to_bf16_rne(sum * scale);
    }
  }
}

// ---------------------------------------------------------------------------
// Column kernel: for column strip c (64 columns) and M-split s,
//   part[s][p][j] = sum_{m in split s} Z[m][p] * W[m][j]
// with (Z, W, output) = (dY [M x N], T, dB [N x r] scaled by `scale`) for the
// first nstrip_b strips, and (X~ [M x K], dT, dA [r x K]) for the rest.
// ---------------------------------------------------------------------------
constexpr int CR_ROWS = 128;           // rows of Z staged per iteration
constexpr int CR_PAD = CR_ROWS + 8;    // LDS row stride (elements) of the transposed tiles

template <int NT>
__device__ __forceinline__ void colred_strip(bool nvfp4, const uint8_t* __restrict__ xc,
                                             const uint8_t* __restrict__ xs, const float* __restrict__ xr,
                                             const uint16_t* __restrict__ zb, int64_t P, int64_t Rb, int64_t Re,
                                             int64_t p0, const uint16_t* __restrict__ w, int64_t r, uint16_t (*zt)[CR_PAD],
                                             uint16_t (*wtl)[CR_PAD], floatx4* acc) {
  constexpr int RT = 16 * NT;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  for (int64_t R0 = Rb; R0 < Re; R0 += CR_ROWS) {
    uint4 zv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid >> 3) + 32 * u, ch = tid & 7;
      const int64_t Rr = R0 + row, pc = p0 + 8 * ch;
      zv[u] = make_uint4(0, 0, 0, 0);
      if (Rr < Re && pc < P) {
        if (nvfp4) {
          const uint32_t wd = *reinterpret_cast<const uint32_t*>(xc + Rr * (P >> 1) + (pc >> 1));
          const float m = __builtin_amdgcn_cvt_f32_fp8((int)xs[Rr * (P >> 4) + (pc >> 4)], 0) * xr[Rr];
          zv[u] = deq8_bf16_packed(wd, m);
        } else {
          zv[u] = *reinterpret_cast<const uint4*>(zb + Rr * P + pc);
        }
      }
    }
    uint16_t wv[CR_ROWS * RT / 256];
#pragma unroll
    for (int u = 0; u < CR_ROWS * RT / 256; ++u) {
      const int q = tid + 256 * u;
      const int row = q / RT, col = q % RT;
      const int64_t Rr = R0 + row;
      wv[u] = (Rr < Re && col < r) ? w[Rr * r + col] : (uint16_t)0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row = (tid >> 3) + 32 * u, ch = tid & 7;
      const uint32_t e[4] = {zv[u].x, zv[u].y, zv[u].z, zv[u].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        zt[8 * ch + 2 * t][row] = (uint16_t)(e[t] & 0xFFFFu);
        zt[8 * ch + 2 * t + 1][row] = (uint16_t)(e[t] >> 16);
      }
    }
#pragma unroll
    for (int u = 0; u < CR_ROWS * RT / 256; ++u) {
      const int q = tid + 256 * u;
      wtl[q % RT][q / RT] = wv[u];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < CR_ROWS / 32; ++kk) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&zt[16 * wave + i][kk * 32 + 8 * g]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8_t bf = *reinterpret_cast<const bf16x8_t*>(&wtl[t * 16 + i][kk * 32 + 8 * g]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();
  }
}

template <int NT>
__global__ __launch_bounds__(256) void k_lora_cols(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                   const float* __restrict__ xr, int64_t M, int64_t K,
                                                   const uint16_t* __restrict__ dy, int64_t N,
                                                   const uint16_t* __restrict__ T, const uint16_t* __restrict__ dT,
                                                   int64_t r, int nstrip_b, int64_t rows_per_split,
                                                   float* __restrict__ part_b, float* __restrict__ part_a) {
  constexpr int RT = 16 * NT;
  __shared__ __attribute__((aligned(16))) uint16_t zt[64][CR_PAD];
  __shared__ __attribute__((aligned(16))) uint16_t wtl[RT][CR_PAD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  const bool is_b = (int)blockIdx.x < nstrip_b;
  const int strip = is_b ? (int)blockIdx.x : (int)blockIdx.x - nstrip_b;
  const int64_t P = is_b ? N : K;
  const int64_t p0 = (int64_t)strip * 64;
  const int64_t Rb = (int64_t)blockIdx.y * rows_per_split;
  const int64_t Re = Rb + rows_per_split < M ? Rb + rows_per_split : M;
  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0, 0, 0, 0};
  if (is_b) colred_strip<NT>(false, nullptr, nullptr, nullptr, dy, P, Rb, Re, p0, T, r, zt, wtl, acc);
  else colred_strip<NT>(true, xc, xs, xr, nullptr, P, Rb, Re, p0, dT, r, zt, wtl, acc);

  // this split's partial for the strip: part[s][p][j], FP32
  float* part = (is_b ? part_b : part_a) + (int64_t)blockIdx.y * P * r;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t j = t * 16 + i;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t pp = p0 + 16 * wave + 4 * g + e;
      if (pp < P && j < r) part[pp * r + j] = acc[t][e];
    }
  }
}

// Sum of the split partials in split order, rounded to BF16: dB [N x r]
// (times `scale`) for q < N*r, then dA [r x K] (stored transposed from the
// [K x r] partials).
__global__ __launch_bounds__(256) void k_lora_reduce(const float* __restrict__ part_b,
                                                     const float* __restrict__ part_a, int nsplit, int64_t N,
                                                     int64_t K, int64_t r, float scale, uint16_t* __restrict__ dB,
                                                     uint16_t* __restrict__ dA) {
  const int64_t nb = N * r, total = nb + K * r;
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const bool is_b = q < nb;
    const int64_t qq = is_b ? q : q - nb;
    const int64_t stride = is_b ? nb : K * r;
    const float* base = is_b ? part_b : part_a;
    float sum = 0.0f;
    for (int s = 0; s < nsplit; ++s) sum += base[(int64_t)s * stride + qq];
    if (is_b) {
      dB[qq] = (uint16_t)f32_to_bf16_rne(sum * scale);
    } else {
      const int64_t k = qq / r, j = qq - k * r;
      dA[j * K + k] = (uint16_t)f32_to_bf16_rne(sum);
    }
  }
}

__global__ __launch_bounds__(256) void k_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256) p[q] = 0;
}

// ---------------------------------------------------------------------------
// launchers and workspace layout
// ---------------------------------------------------------------------------
static int rank_tiles(int64_t r) { return (int)((r + 15) / 16); }

struct LoraWs {
  int64_t nsplit, rows_per_split;
  int nstrip_b, nstrip_a;
  size_t off_T, off_pdB, off_pdA, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static LoraWs lora_ws(int64_t M, int64_t K, int64_t N, int64_t r) {
  LoraWs w;
  int64_t ns = (M + 255) / 256;                 // >= 256 token rows per split
  ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
  w.rows_per_split = (M + ns - 1) / ns;
  w.rows_per_split = (w.rows_per_split + CR_ROWS - 1) / CR_ROWS * CR_ROWS;
  if (w.rows_per_split < CR_ROWS) w.rows_per_split = CR_ROWS;
  w.nsplit = (M + w.rows_per_split - 1) / w.rows_per_split;
  if (w.nsplit < 1) w.nsplit = 1;
  w.nstrip_b = (int)((N + 63) / 64);
  w.nstrip_a = (int)((K + 63) / 64);
  size_t off = 0;
  w.off_T = off;   off = align256(off + (size_t)M * r * 2);
  w.off_pdB = off; off = align256(off + (size_t)w.nsplit * N * r * 4);
  w.off_pdA = off; off = align256(off + (size_t)w.nsplit * K * r * 4);
  w.total = off;
  return w;
}

size_t lora_bwd_workspace(int64_t M, int64_t K, int64_t N, int64_t r) { return lora_ws(M, K, N, r).total; }

template <bool DO_DT>
static void rows(int nt, unsigned grid, hipStream_t s, const uint8_t* xc, const uint8_t* xs, const float* xr,
                 int64_t M, int64_t K, const uint16_t* A, int64_t r, uint16_t* T, const uint16_t* dy, int64_t N,
                 const uint16_t* B, float scale, uint16_t* dT) {
#define PACT_ROWS(NT) k_lora_rows<NT, DO_DT><<<grid, 512, 0, s>>>(xc, xs, xr, M, K, A, r, T, dy, N, B, scale, dT)
  if (nt <= 1) PACT_ROWS(1);
  else if (nt <= 2) PACT_ROWS(2);
  else if (nt <= 4) PACT_ROWS(4);
  else PACT_ROWS(8);
#undef PACT_ROWS
}

hipError_t launch_lora_down(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                            const uint16_t* A, int64_t r, uint16_t* T, hipStream_t s) {
  rows<false>(rank_tiles(r), (unsigned)((M + 15) / 16), s, xc, xs, xr, M, K, A, r, T, nullptr, 0, nullptr, 0.0f,
              nullptr);
  return hipGetLastError();
}

hipError_t launch_lora_bwd(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                           const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                           int64_t N, uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, hipStream_t s) {
  const LoraWs w = lora_ws(M, K, N, r);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* T = reinterpret_cast<uint16_t*>(ws + w.off_T);
  float* pdB = reinterpret_cast<float*>(ws + w.off_pdB);
  float* pdA = reinterpret_cast<float*>(ws + w.off_pdA);
  const int nt = rank_tiles(r);
  const int ncnt = w.nstrip_b + w.nstrip_a;
  if (M == 0) {
    // empty token axis: every gradient is an empty sum (a fill kernel, not a
    // memset, so the call can be captured in a graph)
    if (N * r > 0) k_zero_u16<<<(unsigned)((N * r + 255) / 256 < 4096 ? (N * r + 255) / 256 : 4096), 256, 0, s>>>(dB, N * r);
    if (K * r > 0) k_zero_u16<<<(unsigned)((K * r + 255) / 256 < 4096 ? (K * r + 255) / 256 : 4096), 256, 0, s>>>(dA, K * r);
    return hipGetLastError();
  }
  // T (workspace) and dT
  rows<true>(nt, (unsigned)((M + 15) / 16), s, xc, xs, xr, M, K, A, r, T, dy, N, B, scale, dT);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ncnt == 0) return e;
  const dim3 grid((unsigned)ncnt, (unsigned)w.nsplit);
#define PACT_COLS(NT) k_lora_cols<NT><<<grid, 256, 0, s>>>(xc, xs, xr, M, K, dy, N, T, dT, r, w.nstrip_b, \
                                                           w.rows_per_split, pdB, pdA)
  if (nt <= 1) PACT_COLS(1);
  else if (nt <= 2) PACT_COLS(2);
  else if (nt <= 4) PACT_COLS(4);
  else PACT_COLS(8);
#undef PACT_COLS
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t tot = (N + K) * r;
  k_lora_reduce<<<(unsigned)((tot + 255) / 256 < 4096 ? (tot + 255) / 256 : 4096), 256, 0, s>>>(
      pdB, pdA, (int)w.nsplit, N, K, r, scale, dB, dA);
  return hipGetLastError();
}

}  // namespace pact
