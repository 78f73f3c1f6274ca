// BF16 rank-r LoRA branch on the reconstructed input (PACT, Appendix Table 7
// row "LoRA branch": the adapter products run in BF16 on the dequantized
// NVFP4 input in both directions, and backward keeps only that NVFP4 input
// and the BF16 adapters; Figure 3's caption draws the same split).
//
//   lora_down : T  = bf16(X~ A^T)             X~ = deq(X_q), exact in BF16
//   lora_bwd  : T  = bf16(X~ A^T)             (recomputed, kept in the workspace)
//               dT = bf16(s dY B)
//               dB = bf16(s dY^T T)
//               dA = bf16(dT^T X~)
// (the input-gradient term dT A is added inside the dgrad GEMM's epilogue).
//
// All of these are skinny products with r <= 128 on v_mfma_f32_16x16x32_bf16
// with FP32 accumulation, bound by streaming the long operand (X_q or dY) from
// HBM.  Two kernel shapes:
//   * the row kernel reduces along a row of the long operand (T over K from
//     X_q, dT over N from dY).  A workgroup owns 16 token rows; its 8 waves
//     take interleaved 128-element chunks of the row, each lane loading 32
//     consecutive elements of a row per chunk (16 bytes of codes, or four
//     16-byte BF16 loads) and the matching 32 elements of the small operand
//     (A read rank-major; B transposed through LDS);
//   * the column kernel contracts over the token axis (dB from dY and T, dA
//     from X_q and dT).  Each lane loads an 8-row x CPL-column block of the
//     long operand and transposes it in registers, so MFMA instance c takes
//     columns q0 + CPL i + c (i = lane % 16) with no LDS round trip for the big
//     operand; T and dT come rank-major from the row kernel.  Each workgroup
//     writes an FP32 partial for its column strip and token split; a small
//     reduce launch sums the partials in split order, so results do not depend
//     on scheduling.
#include "pact_internal.h"

#include <mutex>
#include <type_traits>

namespace pact {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16_exact(float f) { return __float_as_uint(f) >> 16; }
__device__ __forceinline__ uint32_t pack2(float a, float b) { return bf16_exact(a) | (bf16_exact(b) << 16); }

// 8 NVFP4 elements of one code word times m (= s or s * r), packed as BF16:
// exact, because e * s has at most 6 significant bits and r is a power of two.
__device__ __forceinline__ uint4 deq8_bf16(uint32_t w, float m) {
  const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const float2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const float2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  return make_uint4(pack2(a.x * m, a.y * m), pack2(b.x * m, b.y * m), pack2(c.x * m, c.y * m),
                    pack2(d.x * m, d.y * m));
}

__device__ __forceinline__ float e4m3_f32(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }


// ---------------------------------------------------------------------------
// Row kernel.  Block (tile, part) with 16 token rows p0 .. p0 + 15:
//   part 0:  T[p][j]  = bf16(xr[p] * sum_k (e*s)[p][k] * A[j][k])     X_q [P x K], A [r x K]
//   part 1:  dT[p][j] = bf16(scale * sum_n dY[p][n] * B[n][j])         dY [P x N], B [N x r]
// Chunk c of the long axis is elements [128c, 128c + 128); waves take chunks
// wave, wave + 8, ...  The chunk of the long operand (16 rows) is loaded with
// row-contiguous 16-byte loads (four rows of 256 bytes per BF16 instruction,
// sixteen rows of 64 bytes of codes per NVFP4 instruction) into a wave-private
// LDS tile and read back in the MFMA layout: sub-step u (0..3) gives lane
// (i, g) row i, elements 128c + 32u + 8g + (0..7).  The small operand must
// reach lane (i, g) as rank 16t + i at those same 8 elements:
//   * A [r x K] is rank-major, so it is read directly in that layout (it is
//     small and cache-resident);
//   * B [N x r] is element-major: its 128 x 16 slice for the chunk and rank
//     tile t is copied as loaded (32 bytes a row) into the wave's tile once the
//     long operand has been read out of it, and read back with
//     ds_read_b64_tr_b16.  That instruction transposes within each 16-lane
//     group: output lane i, element a, is element i % 4 of source lane
//     4a + i / 4, so source lane 4a + c (group g, half h) addresses row
//     32u + 8g + 4h + a, columns 4c .. 4c + 3, and output lane i receives
//     column i of the four rows 32u + 8g + 4h + (0..3).
// The global loads of CH chunks are issued before any of them is used.
// ---------------------------------------------------------------------------
template <int NT>
struct RowCfg {
  static constexpr int CH = NT <= 2 ? 2 : 1;
};
constexpr int RL_STRIDE = 272;              // BF16 tile row stride in LDS (256 B + 16: conflict-free b128 reads)
constexpr int RQ_STRIDE = 80;               // NVFP4 code tile row stride (64 B + 16: conflict-free b32 reads)
constexpr int RQ_SCALES = 16 * RQ_STRIDE;   // then 16 rows x 8 scale bytes
constexpr int RSTAGE = 16 * RL_STRIDE;      // bytes of one wave's staging tile (>= 128 rows x 32 bytes of B)

typedef short short4_t __attribute__((ext_vector_type(4)));

// Row n, columns col .. col + 7 of B [N x r] (zeros outside the matrix);
// 16-byte loads when rows are 16-byte aligned (r % 8 == 0).
__device__ __forceinline__ uint4 load_b8(const uint16_t* __restrict__ B, int64_t n, int64_t col, int64_t N,
                                         int64_t r, bool ok) {
  const bool in = ok && n < N && col < r;
  const uint16_t* p = B + n * r + col;
  if ((r & 7) == 0)
    return load_or_zero(reinterpret_cast<const uint4*>(p), reinterpret_cast<const uint4*>(B), in);
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t lo = load_or_zero(p + 2 * k, B, in && col + 2 * k < r);
    const uint32_t hi = load_or_zero(p + 2 * k + 1, B, in && col + 2 * k + 1 < r);
    w[k] = lo | (hi << 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// A of lora_down / the T part is loaded row-contiguously and laid out for the
// MFMA through LDS up to 4 rank tiles (8 would spill)
template <int NT>
constexpr bool kRowTileA = NT <= 4;

template <int NT, bool NVFP4>
__device__ __forceinline__ void row_reduce(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                           const uint16_t* __restrict__ lb, int64_t p0, int64_t P, int64_t R,
                                           const uint16_t* __restrict__ S, int64_t r, int wave, int lane,
                                           uint8_t* stage, floatx4* acc) {
  constexpr int CH = RowCfg<NT>::CH;
  const int i = lane & 15, g = lane >> 4;
  const int64_t nchunk = (R + 127) / 128;
  for (int64_t cb = wave; cb < nchunk; cb += 8 * CH) {
    uint4 lv[CH][4];          // BF16: instruction v holds rows 4v + lane/16, elements 8 (lane % 16) + (0..7)
    uint32_t lsc[CH][2];      // NVFP4: scale bytes of row lane/4, blocks 2 (lane % 4) and + 1
    uint4 sv[CH][NT][4];      // A: rows 16t + 4v + lane/16, elements 8 (lane % 16) + (0..7) (NT <= 4; else the
                              // MFMA operand of sub-step u); B: rows 32v + lane/2, columns 16t + 8 (lane % 2) + (0..7)
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      const int64_t c = cb + 8 * q;
      const bool cin = c < nchunk;
      if constexpr (NVFP4) {
        // lane -> row lane / 4, bytes 16 (lane % 4) .. + 16 of the chunk's 64 code bytes
        const int64_t row = p0 + (lane >> 2);
        const int64_t k0 = c * 128 + 32 * (lane & 3);
        const bool rin = cin && row < P;
        const bool full = rin && k0 + 32 <= R, half = rin && k0 + 16 <= R;
        const uint8_t* cp = xc + row * (R >> 1) + (k0 >> 1);
        const uint2* c2 = reinterpret_cast<const uint2*>(xc);
        const uint2 w01 = load_or_zero(reinterpret_cast<const uint2*>(cp), c2, half);
        const uint2 w23 = load_or_zero(reinterpret_cast<const uint2*>(cp + 8), c2, full);
        lv[q][0] = make_uint4(w01.x, w01.y, w23.x, w23.y);
        const uint8_t* sp = xs + row * (R >> 4) + (k0 >> 4);
        lsc[q][0] = load_or_zero(sp, xs, half);
        lsc[q][1] = load_or_zero(sp + 1, xs, full);
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t row = p0 + 4 * v + (lane >> 4);
          const int64_t k = c * 128 + 8 * (lane & 15);
          const bool ok = cin && row < P && k + 8 <= R;
          lv[q][v] = load_or_zero(reinterpret_cast<const uint4*>(lb + row * R + k),
                                  reinterpret_cast<const uint4*>(lb), ok);
        }
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (NVFP4 && kRowTileA<NT>) {
          // A rows 16 t + 4 v + lane / 16, elements 8 (lane % 16) .. + 7 of the
          // chunk: four whole rows per instruction (full cache lines); the MFMA
          // layout is formed through the wave's LDS tile below
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int64_t j = 16 * t + 4 * v + (lane >> 4);
            const int64_t k = c * 128 + 8 * (lane & 15);
            const bool ok = cin && j < r && k + 8 <= R;
            sv[q][t][v] = load_or_zero(reinterpret_cast<const uint4*>(S + j * R + k),
                                       reinterpret_cast<const uint4*>(S), ok);
          }
        } else if constexpr (NVFP4) {
          // A in the MFMA layout directly (lane (i, g): row 16 t + i, elements
          // 32 u + 8 g .. + 7), half a cache line per row and instruction
          const int64_t j = 16 * t + i;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int64_t k = c * 128 + 32 * u + 8 * g;
            const bool ok = cin && j < r && k + 8 <= R;
            sv[q][t][u] = load_or_zero(reinterpret_cast<const uint4*>(S + j * R + k),
                                       reinterpret_cast<const uint4*>(S), ok);
          }
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v)
            sv[q][t][v] = load_b8(S, c * 128 + 32 * v + (lane >> 1), 16 * t + 8 * (lane & 1), R, r, cin);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      // stage the chunk in this wave's LDS tile, then read it back in the MFMA layout
      // (the tile is the wave's own and a wave's LDS accesses execute in
      // order, so a read sees the writes before it and a later write
      // cannot overtake a read: no waits, only compiler barriers)
      if constexpr (NVFP4) {
        *reinterpret_cast<uint4*>(stage + (lane >> 2) * RQ_STRIDE + 16 * (lane & 3)) = lv[q][0];
        stage[RQ_SCALES + (lane >> 2) * 8 + 2 * (lane & 3)] = (uint8_t)lsc[q][0];
        stage[RQ_SCALES + (lane >> 2) * 8 + 2 * (lane & 3) + 1] = (uint8_t)lsc[q][1];
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          *reinterpret_cast<uint4*>(stage + (4 * v + (lane >> 4)) * RL_STRIDE + 16 * (lane & 15)) = lv[q][v];
      }
      __builtin_amdgcn_wave_barrier();
      uint4 av[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (NVFP4) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(stage + i * RQ_STRIDE + 16 * u + 4 * g);
          const uint32_t sb = stage[RQ_SCALES + i * 8 + 2 * u + (g >> 1)];
          av[u] = deq8_bf16(w, e4m3_f32(sb));
        } else {
          av[u] = *reinterpret_cast<const uint4*>(stage + i * RL_STRIDE + 64 * u + 16 * g);
        }
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint4 bv[4];
        if constexpr (NVFP4 && kRowTileA<NT>) {
          // A tile (16 rows x 256 bytes) into the wave's LDS tile as loaded, read
          // back as lane (i, g): row 16 t + i, elements 32 u + 8 g .. + 7
#pragma unroll
          for (int v = 0; v < 4; ++v)
            *reinterpret_cast<uint4*>(stage + (4 * v + (lane >> 4)) * RL_STRIDE + 16 * (lane & 15)) = sv[q][t][v];
          __builtin_amdgcn_wave_barrier();
#pragma unroll
          for (int u = 0; u < 4; ++u) bv[u] = *reinterpret_cast<const uint4*>(stage + i * RL_STRIDE + 64 * u + 16 * g);
          __builtin_amdgcn_wave_barrier();
        } else if constexpr (NVFP4) {
#pragma unroll
          for (int u = 0; u < 4; ++u) bv[u] = sv[q][t][u];
        } else {
          // B slice (128 rows x 32 bytes) into the tile as loaded, read back transposed
#pragma unroll
          for (int v = 0; v < 4; ++v)
            *reinterpret_cast<uint4*>(stage + (32 * v + (lane >> 1)) * 32 + 16 * (lane & 1)) = sv[q][t][v];
          __builtin_amdgcn_wave_barrier();
          const int l16 = lane & 15;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            short4_t h2[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              uint8_t* a = stage + (32 * u + 8 * g + 4 * h + (l16 >> 2)) * 32 + 8 * (l16 & 3);
              h2[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)a);
            }
            const uint2 lo = __builtin_bit_cast(uint2, h2[0]), hi = __builtin_bit_cast(uint2, h2[1]);
            bv[u] = make_uint4(lo.x, lo.y, hi.x, hi.y);
          }
          __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av[u]),
                                                           __builtin_bit_cast(bf16x8_t, bv[u]), acc[t], 0, 0, 0);
      }
    }
  }
}

// Part 0 writes T (row-major, if T != NULL) and Tt (rank-major with leading
// dimension ldt, if Tt != NULL); part 1 writes dT and dTt; part 2 copies a
// given dT (dT_in) into dTt.  The rank-major copies get zeros in their padding
// columns [P, ldt), which the column kernel reads.  Block row y runs part
// (parts >> 4y) & 15.
// One workgroup of the row kernel: token rows 16 bx .. 16 bx + 15, `part`.
template <int NT>
__device__ __forceinline__ void lora_rows_block(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                const float* __restrict__ xr, int64_t P, int64_t K,
                                                const uint16_t* __restrict__ A, int64_t r,
                                                uint16_t* __restrict__ T, uint16_t* __restrict__ Tt, int64_t ldt,
                                                const uint16_t* __restrict__ dy, int64_t N,
                                                const uint16_t* __restrict__ B, float scale,
                                                uint16_t* __restrict__ dT, uint16_t* __restrict__ dTt,
                                                const uint16_t* __restrict__ dT_in, int part, int64_t bx) {
  constexpr int NW = 8;
  constexpr int RT = 16 * NT;
  __shared__ float red[NW][16][RT + 1];
  __shared__ __attribute__((aligned(16))) uint8_t stage[NW][RSTAGE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15, g = lane >> 4;
  const int64_t p0 = bx * 16;
  if (part == 2) {
    // rank-major copy of the given dT rows p0 .. p0 + 15 (and the padding)
    for (int q = threadIdx.x; q < 16 * r; q += 512) {
      const int64_t pp = p0 + q / r, j = q % r;
      if (pp < P) dTt[j * ldt + pp] = dT_in[pp * r + j];
    }
    if (p0 + 16 >= P && ldt > P) {
      const int64_t pad = ldt - P;
      for (int64_t q = threadIdx.x; q < r * pad; q += 512) dTt[(q / pad) * ldt + P + q % pad] = 0;
    }
    return;
  }

  floatx4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = floatx4{0, 0, 0, 0};
  if (part == 0) row_reduce<NT, true>(xc, xs, nullptr, p0, P, K, A, r, wave, lane, stage[wave], acc);
  else row_reduce<NT, false>(nullptr, nullptr, dy, p0, P, N, B, r, wave, lane, stage[wave], acc);

  // accumulator layout (16x16): (row, col) at lane col + 16 * (row / 4), register row % 4
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave][4 * g + e][t * 16 + i] = acc[t][e];
  __syncthreads();
  uint16_t* out = part == 0 ? T : dT;
  uint16_t* outt = part == 0 ? Tt : dTt;
  for (int q = threadIdx.x; q < 16 * RT; q += 512) {
    const int row = q / RT, col = q % RT;
    const int64_t pp = p0 + row;
    if (pp < P && col < r) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w][row][col];
      const uint16_t v = (uint16_t)f32_to_bf16_rne(part == 0 ? sum * xr[pp] : sum * scale);
      if (out != nullptr) out[pp * r + col] = v;
      if (outt != nullptr) outt[col * ldt + pp] = v;
    }
  }
  if (outt != nullptr && p0 + 16 >= P && ldt > P) {
    // last row tile: zero the padding columns [P, ldt) of the rank-major copy
    const int64_t pad = ldt - P;
    for (int64_t q = threadIdx.x; q < r * pad; q += 512) outt[(q / pad) * ldt + P + q % pad] = 0;
  }
}

template <int NT>
__global__ __launch_bounds__(512) void k_lora_rows(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                   const float* __restrict__ xr, int64_t P, int64_t K,
                                                   const uint16_t* __restrict__ A, int64_t r,
                                                   uint16_t* __restrict__ T, uint16_t* __restrict__ Tt, int64_t ldt,
                                                   const uint16_t* __restrict__ dy, int64_t N,
                                                   const uint16_t* __restrict__ B, float scale,
                                                   uint16_t* __restrict__ dT, uint16_t* __restrict__ dTt,
                                                   int parts, const uint16_t* __restrict__ dT_in) {
  lora_rows_block<NT>(xc, xs, xr, P, K, A, r, T, Tt, ldt, dy, N, B, scale, dT, dTt, dT_in,
                      (parts >> (4 * (int)blockIdx.y)) & 15, (int64_t)blockIdx.x);
}

// ---------------------------------------------------------------------------
// Column kernel: for column strip x (16 CPL columns of the long operand) and
// token split y,
//   part[y][q][j] = sum_{m in split y} Z[m][q] * Wt[j][m]
// with (Z, Wt) = (dY [M x N], T^T) for the first nstrip_b strips (dB; the
// reduce applies `scale`) and (X~ [M x K], dT^T) for the rest (dA).  A wave
// step covers 32 token rows: lane (i, g) loads rows m0 + 8g + (0..7) at
// columns q0 + CPL i + (0..CPL-1) and transposes the block in registers; MFMA
// instance c (row i <-> column q0 + CPL i + c) contracts the 32 rows against
// Wt.  The 4 waves of a workgroup take interleaved steps of the split and are
// summed through LDS in wave order.
// ---------------------------------------------------------------------------
template <int NT>
struct ColCfg {
  static constexpr int CPL = NT <= 2 ? 8 : (NT <= 4 ? 4 : 2);   // columns per lane
};

// v_perm_b32 byte selects: (lo16(a), lo16(b)) and (hi16(a), hi16(b)) packed as lo | hi << 16
__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// rows[e] holds CPL consecutive BF16 columns of row e (two per dword);
// out[c] = the 8 rows of column c (two per dword).
template <int CPL>
__device__ __forceinline__ void transpose_rows(const uint32_t (&rows)[8][CPL / 2], uint4 (&out)[CPL]) {
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int d = c >> 1;
    uint32_t v[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      v[t] = (c & 1) ? hi_pair(rows[2 * t][d], rows[2 * t + 1][d]) : lo_pair(rows[2 * t][d], rows[2 * t + 1][d]);
    out[c] = make_uint4(v[0], v[1], v[2], v[3]);
  }
}

// One wave step's long-operand block (8 rows x CPL columns per lane, as BF16
// pairs) and its rank-major small operand.
template <int NT, int CPL>
struct ColStep {
  uint32_t rows[8][CPL / 2];
  uint4 wv[NT];
};

template <int NT, int CPL, bool is_b>
__device__ __forceinline__ void col_load(ColStep<NT, CPL>& st, const uint8_t* __restrict__ xc,
                                         const uint8_t* __restrict__ xs, const float* __restrict__ xr, int64_t K,
                                         const uint16_t* __restrict__ dy, int64_t N, const uint16_t* __restrict__ Wt,
                                         int64_t ldt, int64_t r, int64_t m0, int64_t Re, int64_t qc, bool qok,
                                         int lane) {
  const int i = lane & 15, g = lane >> 4;
  // row scales of the step's 32 rows, one per lane (dA strips only)
  float xr_step = 0.0f;
  if constexpr (!is_b) xr_step = load_or_zero(xr + m0 + (lane & 31), xr, m0 + (lane & 31) < Re);
  if constexpr (is_b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t m = m0 + 8 * g + e;
      const bool ok = qok && m < Re;
      const uint16_t* src = dy + m * N + qc;
      if constexpr (CPL == 8) {
        const uint4 v = load_or_zero(reinterpret_cast<const uint4*>(src), reinterpret_cast<const uint4*>(dy), ok);
        st.rows[e][0] = v.x; st.rows[e][1] = v.y; st.rows[e][2] = v.z; st.rows[e][3] = v.w;
      } else if constexpr (CPL == 4) {
        const uint2 v = load_or_zero(reinterpret_cast<const uint2*>(src), reinterpret_cast<const uint2*>(dy), ok);
        st.rows[e][0] = v.x; st.rows[e][1] = v.y;
      } else {
        st.rows[e][0] = load_or_zero(reinterpret_cast<const uint32_t*>(src), reinterpret_cast<const uint32_t*>(dy), ok);
      }
    }
  } else {
    // X~ = e * s * r: CPL codes of row m (within one block), dequantized to
    // BF16; the row scale of row m0 + 8g + e comes from lane 8g + e.  All 8
    // rows' codes and scale bytes are loaded before any is used.
    uint32_t cw[8], sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t m = m0 + 8 * g + e;
      const bool ok = qok && m < Re;
      const uint8_t* cp = xc + m * (K >> 1) + (qc >> 1);
      sc[e] = load_or_zero(xs + m * (K >> 4) + (qc >> 4), xs, ok);
      if constexpr (CPL == 8) cw[e] = load_or_zero(reinterpret_cast<const uint32_t*>(cp), reinterpret_cast<const uint32_t*>(xc), ok);
      else if constexpr (CPL == 4) cw[e] = load_or_zero(reinterpret_cast<const uint16_t*>(cp), reinterpret_cast<const uint16_t*>(xc), ok);
      else cw[e] = load_or_zero(cp, xc, ok);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int64_t m = m0 + 8 * g + e;
      const bool ok = qok && m < Re;
      const float rr = __shfl(xr_step, 8 * g + e, 64);
      const float mlt = ok ? e4m3_f32(sc[e]) * rr : 0.0f;
      const uint32_t w = cw[e];
      if constexpr (CPL == 8) {
        const uint4 v = deq8_bf16(w, mlt);
        st.rows[e][0] = v.x; st.rows[e][1] = v.y; st.rows[e][2] = v.z; st.rows[e][3] = v.w;
      } else if constexpr (CPL == 4) {
        const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        const float2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
        st.rows[e][0] = pack2(a.x * mlt, a.y * mlt);
        st.rows[e][1] = pack2(b.x * mlt, b.y * mlt);
      } else {
        const float2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
        st.rows[e][0] = pack2(a.x * mlt, a.y * mlt);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int64_t j = 16 * t + i;
    // Wt rows are zero-padded up to ldt (M rounded up to 32), and m0 + 32 <= ldt
    st.wv[t] = load_or_zero(reinterpret_cast<const uint4*>(Wt + j * ldt + m0 + 8 * g), reinterpret_cast<const uint4*>(Wt),
                            j < r);
  }
}

template <int NT, int CPL>
__device__ __forceinline__ void col_mma(const ColStep<NT, CPL>& st, floatx4 (&acc)[CPL][NT]) {
  uint4 zt[CPL];
  transpose_rows<CPL>(st.rows, zt);
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int t = 0; t < NT; ++t)
      acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, zt[c]),
                                                          __builtin_bit_cast(bf16x8_t, st.wv[t]), acc[c][t], 0, 0, 0);
}

// Column kernel.  Blocks [0, nstrip_b * nsplit_b) are (strip, split) pairs of
// dB, the rest of dA; each writes the FP32 partial of its strip and split.
// One workgroup of the column kernel: block `blk` of the `nblk` blocks of
// one problem's launch (blocks of different problems start at multiples of 8,
// so block ids map to XCDs as in a launch of its own).
template <int NT>
__device__ __forceinline__ void lora_cols_block(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                const float* __restrict__ xr, int64_t M, int64_t K,
                                                const uint16_t* __restrict__ dy, int64_t N,
                                                const uint16_t* __restrict__ Tt, const uint16_t* __restrict__ dTt,
                                                int64_t ldt, int64_t r, int nstrip_b, int nsplit_b,
                                                int64_t rows_b, int nstrip_a, int64_t rows_a,
                                                float* __restrict__ part_b, float* __restrict__ part_a, int blk,
                                                int nblk) {
  constexpr int CPL = ColCfg<NT>::CPL;
  constexpr int SW = 16 * CPL;
  __shared__ floatx4 red[4][CPL][NT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15;
  // Consecutive block ids go to different XCDs; the remap gives each XCD a
  // contiguous run of (strip, split) pairs, i.e. adjacent strips of the same
  // token rows, so the cache lines of a row (codes, scales, BF16) that
  // neighbouring strips share are fetched into one L2.
  const int nb = nstrip_b * nsplit_b;
  const bool is_b = blk < nb;
  int bid = is_b ? blk : blk - nb;
  const int nstrip = is_b ? nstrip_b : nstrip_a;
  const int npart = is_b ? nb : nblk - nb;
  if ((npart & 7) == 0 && ((is_b ? 0 : nb) & 7) == 0) bid = (bid & 7) * (npart >> 3) + (bid >> 3);
  const int strip = bid % nstrip, split = bid / nstrip;
  const int64_t rows_per_split = is_b ? rows_b : rows_a;
  const int64_t P = is_b ? N : K;
  const int64_t q0 = (int64_t)strip * SW;
  const int64_t qc = q0 + CPL * i;                          // this lane's first column
  const bool qok = qc + CPL <= P;                           // P % 16 == 0: all CPL columns or none
  const int64_t Rb = (int64_t)split * rows_per_split;
  const int64_t Re = Rb + rows_per_split < M ? Rb + rows_per_split : M;
  const uint16_t* Wt = is_b ? Tt : dTt;

  floatx4 acc[CPL][NT];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[c][t] = floatx4{0, 0, 0, 0};

  // a wave step covers 32 token rows; the 4 waves interleave steps
  auto run = [&](auto tag) {
    constexpr bool B_PART = decltype(tag)::value;
    for (int64_t m0 = Rb + 32 * wave; m0 < Re; m0 += 128) {
      ColStep<NT, CPL> st;
      col_load<NT, CPL, B_PART>(st, xc, xs, xr, K, dy, N, Wt, ldt, r, m0, Re, qc, qok, lane);
      col_mma<NT, CPL>(st, acc);
    }
  };
  if (is_b) run(std::true_type{});
  else run(std::false_type{});

#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][c][t][lane] = acc[c][t];
  __syncthreads();
  // output (q, j): q = q0 + CPL ir + c is C row ir of instance c, j = 16 t + jc its C column;
  // C (ir, jc) sits at lane jc + 16 (ir / 4), register ir % 4
  float* part = (is_b ? part_b : part_a) + (int64_t)split * P * r;
  for (int q = tid; q < SW * NT * 16; q += 256) {
    const int ql = q / (NT * 16), jr = q % (NT * 16);
    const int ir = ql / CPL, c = ql % CPL;
    const int t = jr / 16, jc = jr % 16;
    const int ln = jc + 16 * (ir / 4), e = ir % 4;
    const int64_t qq = q0 + ql;
    if (qq < P && jr < r) {
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) sum += red[w][c][t][ln][e];
      part[qq * r + jr] = sum;
    }
  }

}

template <int NT>
__global__ __launch_bounds__(256) void k_lora_cols(const uint8_t* __restrict__ xc, const uint8_t* __restrict__ xs,
                                                   const float* __restrict__ xr, int64_t M, int64_t K,
                                                   const uint16_t* __restrict__ dy, int64_t N,
                                                   const uint16_t* __restrict__ Tt, const uint16_t* __restrict__ dTt,
                                                   int64_t ldt, int64_t r, int nstrip_b, int nsplit_b,
                                                   int64_t rows_b, int nstrip_a, int64_t rows_a,
                                                   float* __restrict__ part_b, float* __restrict__ part_a) {
  lora_cols_block<NT>(xc, xs, xr, M, K, dy, N, Tt, dTt, ldt, r, nstrip_b, nsplit_b, rows_b, nstrip_a, rows_a, part_b,
                      part_a, (int)blockIdx.x, (int)gridDim.x);
}

// Sum of the split partials in split order, rounded to BF16: dB [N x r]
// (times `scale`) for the first N*r elements, then dA [r x K] (stored
// transposed from the [K x r] partials).  A thread owns 4 consecutive elements
// and issues the loads of 8 splits before adding them, in split order.
// Block `blk` of `nblk` of one problem's reduce (a grid-stride loop, so every
// output is formed by one thread in the same order whatever the grid).
__device__ __forceinline__ void lora_reduce_block(const float* __restrict__ part_b, const float* __restrict__ part_a,
                                                  int nsplit_b, int nsplit_a, int64_t N, int64_t K, int64_t r,
                                                  float scale, uint16_t* __restrict__ dB, uint16_t* __restrict__ dA,
                                                  int64_t blk, int64_t nblk) {
  const int64_t nb4 = N * r / 4, total4 = nb4 + K * r / 4;       // N * r and K * r are multiples of 16
  for (int64_t q = blk * 256 + threadIdx.x; q < total4; q += nblk * 256) {
    const bool is_b = q < nb4;
    const int64_t qq = is_b ? q : q - nb4;
    const int64_t stride = is_b ? N * r : K * r;
    const float* base = (is_b ? part_b : part_a) + 4 * qq;
    const int nsplit = is_b ? nsplit_b : nsplit_a;
    float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int sb = 0; sb < nsplit; sb += 8) {
      float4 pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pv[u] = load_or_zero(reinterpret_cast<const float4*>(base + (int64_t)(sb + u) * stride),
                             reinterpret_cast<const float4*>(base), sb + u < nsplit);
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (sb + u < nsplit) {
          sum.x += pv[u].x; sum.y += pv[u].y; sum.z += pv[u].z; sum.w += pv[u].w;
        }
    }
    const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = 4 * qq + u;
      if (is_b) {
        dB[e] = (uint16_t)f32_to_bf16_rne(sv[u] * scale);
      } else {
        const int64_t k = e / r, j = e - k * r;
        dA[j * K + k] = (uint16_t)f32_to_bf16_rne(sv[u]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_lora_reduce(const float* __restrict__ part_b,
                                                     const float* __restrict__ part_a, int nsplit_b, int nsplit_a,
                                                     int64_t N, int64_t K, int64_t r, float scale,
                                                     uint16_t* __restrict__ dB, uint16_t* __restrict__ dA) {
  lora_reduce_block(part_b, part_a, nsplit_b, nsplit_a, N, K, r, scale, dB, dA, (int64_t)blockIdx.x,
                    (int64_t)gridDim.x);
}

// ---------------------------------------------------------------------------
// Batched adapter gradients: dA and dB of up to kLoraBatch problems (each with
// its own X_q, A, dY, dT, workspace and shapes; one token count M and one
// scale) in three launches, each problem's blocks running exactly the
// single-problem code above, so the results are those of lora_bwd_ab.
// ---------------------------------------------------------------------------
struct LoraProb {
  const uint8_t* xc;
  const uint8_t* xs;
  const float* xr;
  const uint16_t* T;                     // [M x r], leading dimension ldT
  const uint16_t* dy;
  const uint16_t* dT;
  uint16_t* dA;
  uint16_t* dB;
  uint16_t* Tt;
  uint16_t* dTt;
  float* pdB;
  float* pdA;
  int64_t K, N, r, ldT, ldt, rows_b, rows_a;
  int nstrip_b, nsplit_b, nstrip_a, nsplit_a;
  int cols_begin, cols_end;              // block range in the column launch (begin % 8 == 0)
  int red_begin, red_end;                // block range in the reduce launch
};
struct LoraBatch {
  LoraProb p[kLoraBatch];
  int n;
  int64_t M;
  float scale;
};

// The rank-major copies the column kernel reads, of every problem of a batch:
// Tt[j][m] = T[m][j] (T with leading dimension ldT) and dTt[j][m] = dT[m][j],
// with zeros in the padding columns [M, ldt).  Workgroup (x, p): rows
// 64 x .. 64 x + 63 of problem p; consecutive threads write consecutive rows.
__global__ __launch_bounds__(256) void k_lora_tt_batch(LoraBatch b) {
  const LoraProb& q = b.p[blockIdx.y];
  const int64_t P = b.M, r = q.r;
  const int64_t p0 = (int64_t)blockIdx.x * 64;
  for (int64_t k = threadIdx.x; k < 64 * r; k += 256) {
    const int64_t j = k >> 6, pp = p0 + (k & 63);
    if (pp < P) {
      q.Tt[j * q.ldt + pp] = q.T[pp * q.ldT + j];
      q.dTt[j * q.ldt + pp] = q.dT[pp * r + j];
    }
  }
  if (p0 + 64 >= P && q.ldt > P) {
    const int64_t pad = q.ldt - P;
    for (int64_t k = threadIdx.x; k < r * pad; k += 256) {
      q.Tt[(k / pad) * q.ldt + P + k % pad] = 0;
      q.dTt[(k / pad) * q.ldt + P + k % pad] = 0;
    }
  }
}

template <int NT>
__global__ __launch_bounds__(256) void k_lora_cols_batch(LoraBatch b) {
  const int g = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < b.n && g >= b.p[pi + 1].cols_begin) ++pi;
  const LoraProb& q = b.p[pi];
  if (g >= q.cols_end) return;                        // alignment padding: the whole block leaves
  lora_cols_block<NT>(q.xc, q.xs, q.xr, b.M, q.K, q.dy, q.N, q.Tt, q.dTt, q.ldt, q.r, q.nstrip_b, q.nsplit_b,
                      q.rows_b, q.nstrip_a, q.rows_a, q.pdB, q.pdA, g - q.cols_begin, q.cols_end - q.cols_begin);
}

__global__ __launch_bounds__(256) void k_lora_reduce_batch(LoraBatch b) {
  const int g = (int)blockIdx.x;
  int pi = 0;
  while (pi + 1 < b.n && g >= b.p[pi + 1].red_begin) ++pi;
  const LoraProb& q = b.p[pi];
  lora_reduce_block(q.pdB, q.pdA, q.nsplit_b, q.nsplit_a, q.N, q.K, q.r, b.scale, q.dB, q.dA,
                    (int64_t)(g - q.red_begin), (int64_t)(q.red_end - q.red_begin));
}

__global__ __launch_bounds__(256) void k_zero_u16(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < n; q += (int64_t)gridDim.x * 256) p[q] = 0;
}

// ---------------------------------------------------------------------------
// launchers and workspace layout
// ---------------------------------------------------------------------------
static int nt_class(int64_t r) {
  const int nt = (int)((r + 15) / 16);
  return nt <= 1 ? 1 : nt <= 2 ? 2 : nt <= 4 ? 4 : 8;
}
static int cols_per_lane(int ntc) { return ntc <= 2 ? 8 : (ntc <= 4 ? 4 : 2); }

struct LoraWs {
  int64_t ldt, nsplit_b, nsplit_a, rows_b, rows_a;
  int nstrip_b, nstrip_a;
  size_t off_Tt, off_dTt, off_pdB, off_pdA, total;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// token splits for `strips` column strips: about `target` workgroups, at least
// 128 token rows (one step per wave) per split, split length a multiple of 32
static void token_splits(int64_t M, int64_t strips, int64_t target, int64_t* nsplit, int64_t* rows) {
  int64_t ns = strips > 0 ? (target + strips - 1) / strips : 1;
  const int64_t max_ns = (M + 127) / 128;
  ns = ns > max_ns ? max_ns : ns;
  ns = ns < 1 ? 1 : (ns > 64 ? 64 : ns);
  int64_t rp = ((M + ns - 1) / ns + 31) / 32 * 32;
  if (rp < 32) rp = 32;
  *rows = rp;
  *nsplit = (M + rp - 1) / rp < 1 ? 1 : (M + rp - 1) / rp;
}

static LoraWs lora_ws(int64_t M, int64_t K, int64_t N, int64_t r) {
  LoraWs w;
  const int64_t sw = 16 * cols_per_lane(nt_class(r));
  w.nstrip_b = (int)((N + sw - 1) / sw);
  w.nstrip_a = (int)((K + sw - 1) / sw);
  w.ldt = (M + 31) / 32 * 32;
  // dB strips stream BF16 dY (long steps); dA strips dequantize X_q (shorter splits)
  token_splits(M, w.nstrip_b, 384, &w.nsplit_b, &w.rows_b);
  token_splits(M, w.nstrip_a, 384, &w.nsplit_a, &w.rows_a);
  size_t off = 0;
  w.off_Tt = off;  off = align256(off + (size_t)r * w.ldt * 2);
  w.off_dTt = off; off = align256(off + (size_t)r * w.ldt * 2);
  w.off_pdB = off; off = align256(off + (size_t)w.nsplit_b * N * r * 4);
  w.off_pdA = off; off = align256(off + (size_t)w.nsplit_a * K * r * 4);
  w.total = off;
  return w;
}

size_t lora_bwd_workspace(int64_t M, int64_t K, int64_t N, int64_t r) { return lora_ws(M, K, N, r).total; }

static void rows(int ntc, dim3 grid, hipStream_t s, const uint8_t* xc, const uint8_t* xs, const float* xr,
                 int64_t M, int64_t K, const uint16_t* A, int64_t r, uint16_t* T, uint16_t* Tt, int64_t ldt,
                 const uint16_t* dy, int64_t N, const uint16_t* B, float scale, uint16_t* dT, uint16_t* dTt,
                 int parts = 0x10, const uint16_t* dT_in = nullptr) {
#define PACT_ROWS(NT) \
  k_lora_rows<NT><<<grid, 512, 0, s>>>(xc, xs, xr, M, K, A, r, T, Tt, ldt, dy, N, B, scale, dT, dTt, parts, dT_in)
  if (ntc <= 1) PACT_ROWS(1);
  else if (ntc <= 2) PACT_ROWS(2);
  else if (ntc <= 4) PACT_ROWS(4);
  else PACT_ROWS(8);
#undef PACT_ROWS
}

static unsigned grid_for(int64_t n) { return (unsigned)((n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096); }

hipError_t launch_lora_down(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                            const uint16_t* A, int64_t r, uint16_t* T, hipStream_t s) {
  rows(nt_class(r), dim3((unsigned)((M + 15) / 16), 1), s, xc, xs, xr, M, K, A, r, T, nullptr, 0, nullptr, 0,
       nullptr, 0.0f, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_lora_bwd_dt(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* B, int64_t r, float scale,
                              uint16_t* dT, hipStream_t s) {
  if (M == 0) return hipSuccess;
  rows(nt_class(r), dim3((unsigned)((M + 15) / 16), 1), s, nullptr, nullptr, nullptr, M, 0, nullptr, r, nullptr,
       nullptr, 0, dy, N, B, scale, dT, nullptr, 0x1);
  return hipGetLastError();
}

hipError_t launch_lora_bwd(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                           const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                           int64_t N, uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, hipStream_t s) {
  return launch_lora_bwd_impl(xc, xs, xr, M, K, A, B, r, scale, dy, N, dT, nullptr, dA, dB, workspace, s);
}

hipError_t launch_lora_bwd_ab(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                              const uint16_t* A, int64_t r, float scale, const uint16_t* dy, int64_t N,
                              const uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, hipStream_t s) {
  return launch_lora_bwd_impl(xc, xs, xr, M, K, A, nullptr, r, scale, dy, N, nullptr, dT, dA, dB, workspace, s);
}

// dT_in == nullptr: the whole backward (dT from dY and B); else dT is given
// (lora_bwd_dt's output) and only dA and dB are formed, with identical results.
hipError_t launch_lora_bwd_impl(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                                const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                                int64_t N, uint16_t* dT, const uint16_t* dT_in, uint16_t* dA, uint16_t* dB,
                                void* workspace, hipStream_t s) {
  const LoraWs w = lora_ws(M, K, N, r);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* Tt = reinterpret_cast<uint16_t*>(ws + w.off_Tt);
  uint16_t* dTt = reinterpret_cast<uint16_t*>(ws + w.off_dTt);
  float* pdB = reinterpret_cast<float*>(ws + w.off_pdB);
  float* pdA = reinterpret_cast<float*>(ws + w.off_pdA);
  const int ntc = nt_class(r);
  if (M == 0) {
    // empty token axis: every gradient is an empty sum (a fill kernel, not a
    // memset, so the call can be captured in a graph)
    if (N * r > 0) k_zero_u16<<<grid_for(N * r), 256, 0, s>>>(dB, N * r);
    if (K * r > 0) k_zero_u16<<<grid_for(K * r), 256, 0, s>>>(dA, K * r);
    return hipGetLastError();
  }
  // T^T (workspace), dT and dT^T (workspace); or T^T and the copy of the given dT
  rows(ntc, dim3((unsigned)((M + 15) / 16), 2), s, xc, xs, xr, M, K, A, r, nullptr, Tt, w.ldt, dy, N, B, scale, dT,
       dTt, dT_in != nullptr ? 0x20 : 0x10, dT_in);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nblk = (int64_t)w.nstrip_b * w.nsplit_b + (int64_t)w.nstrip_a * w.nsplit_a;
  if (nblk == 0) return hipSuccess;
#define PACT_COLS(NT)                                                                                          \
  k_lora_cols<NT><<<(unsigned)nblk, 256, 0, s>>>(xc, xs, xr, M, K, dy, N, Tt, dTt, w.ldt, r, w.nstrip_b,           \
                                                 (int)w.nsplit_b, w.rows_b, w.nstrip_a, w.rows_a,                  \
                                                 pdB, pdA)
  if (ntc <= 1) PACT_COLS(1);
  else if (ntc <= 2) PACT_COLS(2);
  else if (ntc <= 4) PACT_COLS(4);
  else PACT_COLS(8);
#undef PACT_COLS
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t tot4 = (N + K) * r / 4;
  k_lora_reduce<<<grid_for(tot4), 256, 0, s>>>(pdB, pdA, (int)w.nsplit_b, (int)w.nsplit_a, N, K, r, scale, dB, dA);
  return hipGetLastError();
}

bool lora_same_rank_class(int64_t r0, int64_t r1) { return nt_class(r0) == nt_class(r1); }

hipError_t launch_lora_bwd_ab_batch(int n, const uint8_t* const* xc, const uint8_t* const* xs,
                                    const float* const* xr, int64_t M, const int64_t* K,
                                    const uint16_t* const* T, const int64_t* ldT, const int64_t* r, float scale,
                                    const uint16_t* const* dy, const int64_t* N, const uint16_t* const* dT,
                                    uint16_t* const* dA, uint16_t* const* dB, void* const* ws, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (M == 0) {
    for (int i = 0; i < n; ++i) {
      if (N[i] * r[i] > 0) k_zero_u16<<<grid_for(N[i] * r[i]), 256, 0, s>>>(dB[i], N[i] * r[i]);
      if (K[i] * r[i] > 0) k_zero_u16<<<grid_for(K[i] * r[i]), 256, 0, s>>>(dA[i], K[i] * r[i]);
    }
    return hipGetLastError();
  }
  LoraBatch b{};
  b.n = n;
  b.M = M;
  b.scale = scale;
  int cols = 0, red = 0;
  for (int i = 0; i < n; ++i) {
    const LoraWs w = lora_ws(M, K[i], N[i], r[i]);
    uint8_t* base = static_cast<uint8_t*>(ws[i]);
    LoraProb& q = b.p[i];
    q.xc = xc[i]; q.xs = xs[i]; q.xr = xr[i]; q.T = T[i]; q.dy = dy[i]; q.dT = dT[i]; q.dA = dA[i]; q.dB = dB[i];
    q.Tt = reinterpret_cast<uint16_t*>(base + w.off_Tt);
    q.dTt = reinterpret_cast<uint16_t*>(base + w.off_dTt);
    q.pdB = reinterpret_cast<float*>(base + w.off_pdB);
    q.pdA = reinterpret_cast<float*>(base + w.off_pdA);
    q.K = K[i]; q.N = N[i]; q.r = r[i]; q.ldT = ldT[i]; q.ldt = w.ldt; q.rows_b = w.rows_b; q.rows_a = w.rows_a;
    q.nstrip_b = w.nstrip_b; q.nsplit_b = (int)w.nsplit_b; q.nstrip_a = w.nstrip_a; q.nsplit_a = (int)w.nsplit_a;
    const int nblk = (int)((int64_t)w.nstrip_b * w.nsplit_b + (int64_t)w.nstrip_a * w.nsplit_a);
    q.cols_begin = cols;
    q.cols_end = cols + nblk;
    cols = (q.cols_end + 7) / 8 * 8;
    q.red_begin = red;
    q.red_end = red + (int)grid_for((N[i] + K[i]) * r[i] / 4);
    red = q.red_end;
  }
  k_lora_tt_batch<<<dim3((unsigned)((M + 63) / 64), (unsigned)n), 256, 0, s>>>(b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (cols > 0) {
    const int ntc = nt_class(r[0]);
    if (ntc <= 1) k_lora_cols_batch<1><<<(unsigned)cols, 256, 0, s>>>(b);
    else if (ntc <= 2) k_lora_cols_batch<2><<<(unsigned)cols, 256, 0, s>>>(b);
    else if (ntc <= 4) k_lora_cols_batch<4><<<(unsigned)cols, 256, 0, s>>>(b);
    else k_lora_cols_batch<8><<<(unsigned)cols, 256, 0, s>>>(b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  k_lora_reduce_batch<<<(unsigned)red, 256, 0, s>>>(b);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// lora_bwd without a caller workspace: the same launches, with the workspace
// in a fixed device array.  Every byte of the workspace that a launch reads is
// written earlier in the same call (T^T and dT^T by the row kernel for rows
// < M, each split's partials by the column kernel), so nothing is cleared
// between calls.  One array per device, shared by every call on that device:
// calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kLoraScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};     // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t lora_scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));      // with `dev` current: this device's copy
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return hipSuccess;
}

}  // namespace pact
