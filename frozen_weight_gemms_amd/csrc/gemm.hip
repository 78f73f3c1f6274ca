// NVFP4 x NVFP4 -> BF16 GEMM for the frozen projections: C = A B^T with both
// operands row-blocked NVFP4 (PACT, Appendix Table 7 row "Frozen projections":
// both the forward product and the input gradient are NVFP4 GEMMs that sum in
// FP32 and write BF16, each over its own cached NVFP4 copy of the weight).  With
// W_fwd = Q(W) and W_bwd = Q(W^T) both directions are this one product:
//   forward  Y  = X_q  W_fwd^T   (A = X_q  [M x K],  B = W_fwd [N x K])
//   dgrad    dX = dY_q W_bwd^T   (A = dY_q [M x N],  B = W_bwd [K x N])
//
// How NVFP4 maps onto CDNA4 matrix cores.  An NVFP4 element times its E4M3
// block scale, e * s, has at most 2 + 4 = 6 significant bits and magnitude in
// [2^-10, 2688], so it is exact in FP16.  The kernel dequantizes each 16-element
// block in registers to FP16 (v_cvt_scalef32_pk_f16_fp4 for the E2M1 values,
// then one v_pk_mul_f16 by the block scale) and runs
// v_mfma_f32_32x32x16_f16 with FP32 accumulation, so every product is exact
// and only the FP32 accumulation rounds.  The power-of-two row scales of A and
// B multiply the accumulator in the epilogue (exact).  The scaled FP4 MFMA of
// gfx950 takes power-of-two (E8M0) scales per 32 elements; NVFP4's E4M3 scales
// per 16 elements cannot be expressed through it without error, so the
// contraction runs at the FP16 matrix rate.
//
// Tiling.  A workgroup of 4 waves (2 x 2) computes a BM x BN tile, each wave
// (BM/2) x (BN/2) as WTM x WTN MFMA tiles of 32 x 32.  Two kernels:
//   * the generic one (any K % 16 == 0) advances K in stages of 128 (8 NVFP4
//     blocks, 64 code bytes per row), double-buffered through registers into
//     LDS; lane half h owns K range [64h, 64h + 64) of a stage and MFMA step s
//     takes K = 64h + 8s + t (t = 0..7) from both operands;
//   * the fast one (K % 256 == 0, below) advances K in stages of 256 loaded
//     straight into two LDS buffers with LDS-direct buffer loads; lane half h
//     owns K range [128h, 128h + 128) and step s takes K = 128h + 8s + t.
// Both take the same consistent permutation of K for the two operands.
#include <type_traits>

#include "epilogue.h"
#include "lds_dma.h"
#include "mfma_fp16.h"
#include "pact_internal.h"

namespace pact {

constexpr int KT = 128;            // K elements per stage
#ifndef PACT_VALU_PER_MFMA
#define PACT_VALU_PER_MFMA 6
#endif
constexpr int CODE_STRIDE = 80;    // LDS bytes per row of codes (64 data + 16 pad: conflict-free b128 reads)
constexpr int SCALE_STRIDE = 48;   // LDS bytes per row of FP16 scale pairs (32 data + 16 pad)

template <int WTM, int WTN>
struct TileCfg {
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 64 * WTN;
  static constexpr int A_CODES = 0;
  static constexpr int B_CODES = A_CODES + BM * CODE_STRIDE;
  static constexpr int A_SC = B_CODES + BN * CODE_STRIDE;
  static constexpr int B_SC = A_SC + BM * SCALE_STRIDE;
  static constexpr int STAGE = B_SC + BN * SCALE_STRIDE;
  static constexpr int NCODE_A = BM * 8 / 256;   // 8-byte code chunks per thread per stage
  static constexpr int NCODE_B = BN * 8 / 256;
  static constexpr int NSC = (BM + BN + 255) / 256;
};

__device__ __forceinline__ uint32_t scale_pair(uint32_t e4m3) {
  const float f = __builtin_amdgcn_cvt_f32_fp8((int)e4m3, 0);
  const _Float16 h = (_Float16)f;                       // exact: E4M3 values are FP16 values
  const uint32_t hb = (uint32_t)__builtin_bit_cast(uint16_t, h);
  return hb | (hb << 16);
}

template <int WTM, int WTN>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4(GemmArgs p, int tiles_m, int tiles_n) {
  using C = TileCfg<WTM, WTN>;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  // ---- tile index: consecutive tiles per XCD, then grouped along M ----
  const int nwg = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((nwg & 7) == 0) tile = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  constexpr int GM = 4;
  const int group = tile / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = tile - group * GM * tiles_n;
  const int tile_m = first_m + in_group % gm;
  const int tile_n = in_group / gm;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kb = K >> 4;                 // blocks per row
  const int64_t crow = K >> 1;               // code bytes per row
  const int nk = (int)((K + KT - 1) / KT);
  const bool sc_aligned = (K % KT) == 0;

  floatx16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- optional rank-r term, accumulated first and rescaled by s / (rA rB) ----
  if (p.lora_t != nullptr) {
    const int64_t r = p.lora_r;
    for (int64_t k0 = 0; k0 < r; k0 += 16) {
      bf16x8_t tf[WTM], uf[WTN];
      // every element from a clamped, valid index, selected afterwards (a
      // conditional load compiles to a branch and a wait of its own)
      uint16_t et[WTM][8], eu[WTN][8];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
        m = m < M ? m : M - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          et[i][t] = p.lora_t[m * r + (j < r ? j : r - 1)];
        }
      }
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
        n = n < N ? n : N - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          eu[i][t] = p.lora_u[(j < r ? j : r - 1) * p.u_stride_j + n * p.u_stride_n];
        }
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) tf[i][t] = bf16_of(k0 + 8 * h + t < r ? et[i][t] : (uint16_t)0);
#pragma unroll
      for (int i = 0; i < WTN; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t) uf[i][t] = bf16_of(k0 + 8 * h + t < r ? eu[i][t] : (uint16_t)0);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], uf[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      int64_t n = n0 + wn * (BN / 2) + j * 32 + li;
      n = n < N ? n : N - 1;
      const float inv_b = 1.0f / p.b_rscale[n];
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          int64_t m = m0 + wm * (BM / 2) + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
          m = m < M ? m : M - 1;
          const float f = (p.lora_scale * (1.0f / p.a_rscale[m])) * inv_b;
          acc[i][j][rr] *= f;
        }
    }
  }

  // ---- global -> register staging ----
  uint2 ga[C::NCODE_A], gb[C::NCODE_B];
  uint2 gs[C::NSC];
  auto load_stage = [&](int kt) {
#pragma unroll
    for (int it = 0; it < C::NCODE_A; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 3, blk = q & 7;
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      const int64_t b = (int64_t)kt * 8 + blk;
      ga[it] = load_or_zero(reinterpret_cast<const uint2*>(p.a_codes + m * crow + (b < kb ? b : 0) * 8),
                            reinterpret_cast<const uint2*>(p.a_codes), b < kb);
    }
#pragma unroll
    for (int it = 0; it < C::NCODE_B; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 3, blk = q & 7;
      int64_t n = n0 + row;
      n = n < N ? n : N - 1;
      const int64_t b = (int64_t)kt * 8 + blk;
      gb[it] = load_or_zero(reinterpret_cast<const uint2*>(p.b_codes + n * crow + (b < kb ? b : 0) * 8),
                            reinterpret_cast<const uint2*>(p.b_codes), b < kb);
    }
#pragma unroll
    for (int it = 0; it < C::NSC; ++it) {
      const int row = tid + 256 * it;
      gs[it] = make_uint2(0, 0);
      if (row < BM + BN) {
        const uint8_t* base;
        if (row < BM) {
          int64_t m = m0 + row;
          m = m < M ? m : M - 1;
          base = p.a_scales + m * kb;
        } else {
          int64_t n = n0 + (row - BM);
          n = n < N ? n : N - 1;
          base = p.b_scales + n * kb;
        }
        const int64_t b0 = (int64_t)kt * 8;
        if (sc_aligned) {
          gs[it] = *reinterpret_cast<const uint2*>(base + b0);
        } else {
          uint32_t lo = 0, hi = 0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (b0 + t < kb) lo |= (uint32_t)base[b0 + t] << (8 * t);
            if (b0 + 4 + t < kb) hi |= (uint32_t)base[b0 + 4 + t] << (8 * t);
          }
          gs[it] = make_uint2(lo, hi);
        }
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* st = smem + buf * C::STAGE;
#pragma unroll
    for (int it = 0; it < C::NCODE_A; ++it) {
      const int q = tid + 256 * it;
      *reinterpret_cast<uint2*>(st + C::A_CODES + (q >> 3) * CODE_STRIDE + (q & 7) * 8) = ga[it];
    }
#pragma unroll
    for (int it = 0; it < C::NCODE_B; ++it) {
      const int q = tid + 256 * it;
      *reinterpret_cast<uint2*>(st + C::B_CODES + (q >> 3) * CODE_STRIDE + (q & 7) * 8) = gb[it];
    }
#pragma unroll
    for (int it = 0; it < C::NSC; ++it) {
      const int row = tid + 256 * it;
      if (row < BM + BN) {
        uint8_t* dst = row < BM ? st + C::A_SC + row * SCALE_STRIDE : st + C::B_SC + (row - BM) * SCALE_STRIDE;
        uint4 lo, hi;
        lo.x = scale_pair(gs[it].x & 0xFF); lo.y = scale_pair((gs[it].x >> 8) & 0xFF);
        lo.z = scale_pair((gs[it].x >> 16) & 0xFF); lo.w = scale_pair(gs[it].x >> 24);
        hi.x = scale_pair(gs[it].y & 0xFF); hi.y = scale_pair((gs[it].y >> 8) & 0xFF);
        hi.z = scale_pair((gs[it].y >> 16) & 0xFF); hi.w = scale_pair(gs[it].y >> 24);
        reinterpret_cast<uint4*>(dst)[0] = lo;
        reinterpret_cast<uint4*>(dst)[1] = hi;
      }
    }
  };

  if (nk > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const uint8_t* st = smem + buf * C::STAGE;
    uint4 ca0[WTM], ca1[WTM], sa[WTM], cb0[WTN], cb1[WTN], sb[WTN];
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = wm * (BM / 2) + i * 32 + li;
      const uint8_t* cp = st + C::A_CODES + row * CODE_STRIDE + 32 * h;
      ca0[i] = reinterpret_cast<const uint4*>(cp)[0];
      ca1[i] = reinterpret_cast<const uint4*>(cp)[1];
      sa[i] = *reinterpret_cast<const uint4*>(st + C::A_SC + row * SCALE_STRIDE + 16 * h);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int row = wn * (BN / 2) + j * 32 + li;
      const uint8_t* cp = st + C::B_CODES + row * CODE_STRIDE + 32 * h;
      cb0[j] = reinterpret_cast<const uint4*>(cp)[0];
      cb1[j] = reinterpret_cast<const uint4*>(cp)[1];
      sb[j] = *reinterpret_cast<const uint4*>(st + C::B_SC + row * SCALE_STRIDE + 16 * h);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      half8_t af[WTM], bf[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const uint4& c = s < 4 ? ca0[i] : ca1[i];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        const uint32_t sp = (s >> 1) == 0 ? sa[i].x : (s >> 1) == 1 ? sa[i].y : (s >> 1) == 2 ? sa[i].z : sa[i].w;
        af[i] = dequant8(w, sp);
      }
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const uint4& c = s < 4 ? cb0[j] : cb1[j];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        const uint32_t sp = (s >> 1) == 0 ? sb[j].x : (s >> 1) == 1 ? sb[j].y : (s >> 1) == 2 ? sb[j].z : sb[j].w;
        bf[j] = dequant8(w, sp);
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_stage(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: row scales, optional accumulate, BF16 rounding ----
#pragma unroll
  for (int j = 0; j < WTN; ++j) {
    const int64_t n = n0 + wn * (BN / 2) + j * 32 + li;
    if (n >= N) continue;
    const float rb = p.b_rscale[n];
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int64_t m = m0 + wm * (BM / 2) + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        if (m < M) {
          float v = acc[i][j][rr] * (p.a_rscale[m] * rb);
          uint16_t* dst = p.out + m * p.ldo + n;
          if (p.accumulate) v += __uint_as_float((uint32_t)*dst << 16);
          *dst = (uint16_t)f32_to_bf16_rne(v);
        }
      }
  }
}

// ===========================================================================
// Fast path (K % 256 == 0): global -> LDS direct loads, two LDS stages of
// K = 256.
//
// Each stage holds, for the BM + BN rows of the tile, 128 bytes of codes and
// 16 bytes of raw E4M3 scales per row.  The loads are buffer loads with the
// LDS-direct modifier (16 bytes per lane; each instruction fills 1 KB of LDS at
// the wave-uniform address in M0), so no registers stage the data and rows
// past the end of an operand read as zeros through the buffer range check.  A
// row's eight 16-byte code chunks are stored XOR-swizzled by (row >> 1) & 7,
// which spreads the 16 rows of every 256-byte LDS access over all banks.
// Lane half h of a wave owns K range [128h, 128h + 128) of a stage; K step s
// (0..15) takes K = 128h + 8s + t (t = 0..7) from both operands.
// ===========================================================================
constexpr int KT2 = 256;           // K elements per stage of the fast path

template <int WTM, int WTN>
struct FastCfg {
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 64 * WTN;
  static constexpr int ROWS = BM + BN;
  static constexpr int CODES = 0;                       // [ROWS][128] swizzled
  static constexpr int SCALES = ROWS * 128;             // [ROWS][16]
  static constexpr int NC = ROWS / 32;                  // code load instructions per wave per stage (8 rows each)
  static constexpr int NS_TOTAL = ROWS / 64;            // scale load instructions per stage (64 rows each)
  static constexpr int NS = (NS_TOTAL + 3) / 4;         // per wave; surplus ones fill a pad region with zeros
  static constexpr int PAD = SCALES + ROWS * 16;
  static constexpr int STAGE = PAD + (NS * 4 - NS_TOTAL) * 1024;
  static constexpr int LOADS = NC + NS;                 // vector-memory instructions per stage per wave
  // epilogue: per wave, one 32-row slab of its (BN/2)-column tile as FP32
  static constexpr int EPI_LD = BN / 2 + 4;             // floats per staged row (pad breaks bank aliasing)
  static constexpr int EPI_WAVE = 32 * EPI_LD * 4;      // bytes per wave
  static constexpr int MAIN = 2 * STAGE > 4 * EPI_WAVE ? 2 * STAGE : 4 * EPI_WAVE;
  static constexpr int RSC = MAIN;                      // row scales of A (BM floats) then B (BN floats)
  static constexpr int TOTAL = RSC + ROWS * 4;
  static constexpr int NR_TOTAL = ROWS / 64;            // row-scale load instructions (64 rows each)
  static constexpr int NR = (NR_TOTAL + 3) / 4;         // per wave
  static_assert(ROWS % 64 == 0 && BM % 64 == 0, "tile rows");
};

// With SEG, the contraction runs over up to kMaxSeg segments (sg), each with
// its own A and B operands, contraction length (a multiple of the stage) and
// row scales: the input gradient summed over several projections that read
// the same X.  The accumulator holds each segment's partial sum in units of
// the current segment's row scales; at a segment boundary it is rescaled by
// the power of two r_A,old r_B,old / (r_A,new r_B,new) (v_ldexp: exact in the
// FP32 range), so the epilogue applies the last segment's scales.  Row scales
// that are not powers of two (the FP32 tensor-scale recipe) cannot be carried
// across segments this way: with two or more segments the epilogue checks
// every segment's row scales of the tile and writes NaN to the tile if one of
// them is not a power of two
// (such operands take one nvfp4_gemm_dgrad launch per projection, with
// accumulate, instead).  Without SEG every segment branch compiles away.
template <int WTM, int WTN, bool SEG = false>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_fast(GemmArgs p, int tiles_m, int tiles_n, SegArgs sg) {
  using C = FastCfg<WTM, WTN>;
  constexpr int BM = C::BM, BN = C::BN;
  constexpr int NSEG_LDS = SEG ? kMaxSeg : 1;            // row-scale areas (one per segment)
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::TOTAL + (NSEG_LDS - 1) * C::ROWS * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int li = lane & 31, h = lane >> 5;

  const int nwg = tiles_m * tiles_n;
  int tile = blockIdx.x;
  if ((nwg & 7) == 0) tile = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  constexpr int GM = 4;
  const int group = tile / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(tiles_m - first_m, GM);
  const int in_group = tile - group * GM * tiles_n;
  const int tile_m = first_m + in_group % gm;
  const int tile_n = in_group / gm;
  const int64_t m0 = (int64_t)tile_m * BM, n0 = (int64_t)tile_n * BN;

  const int64_t M = p.M, N = p.N, K = p.K;
  uint32_t crow = (uint32_t)(K >> 1), srow = (uint32_t)(K >> 4);
  const int nk = (int)(K / KT2);

  floatx16 acc[WTM][WTN];

  // ---- load addressing ----
  // Code instruction c of this wave covers tile rows 8 (wave + 4c) .. +7: lane
  // -> row 8 (wave + 4c) + lane / 8, LDS slot lane % 8, global chunk
  // slot ^ ((row >> 1) & 7) (independent of c).  Rows below BM are A rows.
  int4v_t ra_c = buffer_rsrc(p.a_codes, (uint32_t)(M * crow));
  int4v_t rb_c = buffer_rsrc(p.b_codes, (uint32_t)(N * crow));
  int4v_t ra_s = buffer_rsrc(p.a_scales, (uint32_t)(M * srow));
  int4v_t rb_s = buffer_rsrc(p.b_scales, (uint32_t)(N * srow));
  const int crow0 = 8 * wave + (lane >> 3);              // tile row of instruction 0
  const uint32_t cchunk = (uint32_t)(((lane & 7) ^ ((crow0 >> 1) & 7)) << 4);
  // voffset of code instruction c: the row term must sit in voffset so that
  // rows past the operand end fail the range check
  auto code_voff = [&](int c) -> uint32_t {
    const int row = crow0 + 32 * c;
    if (row < BM) {
      const int64_t m = m0 + row;
      return m < M ? (uint32_t)m * crow + cchunk : 0xfffffff0u;
    }
    const int64_t n = n0 + (row - BM);
    return n < N ? (uint32_t)n * crow + cchunk : 0xfffffff0u;
  };
  uint32_t cvo[C::NC];
  uint32_t svo[C::NS];
  // scale instruction c of this wave: tile rows 64 (wave + 4c) + lane
  auto set_voffsets = [&]() __attribute__((always_inline)) {
#pragma unroll
  for (int c = 0; c < C::NC; ++c) cvo[c] = code_voff(c);
#pragma unroll
  for (int c = 0; c < C::NS; ++c) {
    const int q = wave + 4 * c;
    const int row = 64 * q + lane;
    uint32_t v = 0xfffffff0u;                              // surplus instruction: zeros into the pad
    if (q < C::NS_TOTAL) {
      if (row < BM) {
        const int64_t m = m0 + row;
        if (m < M) v = (uint32_t)m * srow;
      } else {
        const int64_t n = n0 + (row - BM);
        if (n < N) v = (uint32_t)n * srow;
      }
    }
    svo[c] = v;
  }
  };
  set_voffsets();
  // load descriptors and voffsets of segment sgi's operands
  auto set_segment = [&](int sgi) __attribute__((always_inline)) {
    if constexpr (SEG) {
      const int64_t Ks = sg.s[sgi].K;
      crow = (uint32_t)(Ks >> 1);
      srow = (uint32_t)(Ks >> 4);
      ra_c = buffer_rsrc(sg.s[sgi].a_codes, (uint32_t)(M * crow));
      rb_c = buffer_rsrc(sg.s[sgi].b_codes, (uint32_t)(N * crow));
      ra_s = buffer_rsrc(sg.s[sgi].a_scales, (uint32_t)(M * srow));
      rb_s = buffer_rsrc(sg.s[sgi].b_scales, (uint32_t)(N * srow));
      set_voffsets();
    }
  };
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  // load instruction q (< LOADS) of stage kt into LDS buffer buf
  auto issue_one = [&](int kt, int buf, int q) {
    const uint32_t st = lds0 + (uint32_t)(buf * C::STAGE);
    if (q < C::NC) {
      const bool is_a = 8 * (4 * q + 3) + 7 < BM;          // all four waves' rows of instruction q are A rows
      const bool is_b = 8 * (4 * q) >= BM;
      static_assert(BM % 32 == 0, "A/B split on an instruction boundary");
      const uint32_t dst = st + C::CODES + (uint32_t)(wave_s + 4 * q) * 1024u;
      const uint32_t soff = (uint32_t)kt * 128u;
      if (is_a) lds_dma_buf16(ra_c, cvo[q], soff, dst);
      else if (is_b) lds_dma_buf16(rb_c, cvo[q], soff, dst);
    } else {
      const int c = q - C::NC;
      const int qq = wave_s + 4 * c;
      const uint32_t dst = qq < C::NS_TOTAL ? st + C::SCALES + (uint32_t)qq * 1024u
                                            : st + C::PAD + (uint32_t)(qq - C::NS_TOTAL) * 1024u;
      const uint32_t soff = (uint32_t)kt * 16u;
      // scale instruction c covers rows 64 (wave + 4c) ..: A rows iff 64 (4c + 3) + 63 < BM, B rows iff 256 c >= BM
      if (64 * (4 * c + 3) + 63 < BM) lds_dma_buf16(ra_s, svo[c], soff, dst);
      else if (256 * c >= BM) lds_dma_buf16(rb_s, svo[c], soff, dst);
      else if (qq * 64 < BM) lds_dma_buf16(ra_s, svo[c], soff, dst);   // split by wave: uniform branch
      else lds_dma_buf16(rb_s, svo[c], soff, dst);
    }
  };
  auto issue_stage = [&](int kt, int buf) {
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q) issue_one(kt, buf, q);
  };

  // ---- fragment reads from LDS ----
  uint4 ca[WTM][2], cb[WTN][2];
  uint2 sra[WTM], srb[WTN], sra_n[WTM], srb_n[WTN];
  half2_t sa[WTM][2], sb[WTN][2];
  // codes chunk c (K steps 4c .. 4c + 3) into register slot c & 1
  auto read_codes = [&](const uint8_t* st, int c) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = wm * (BM / 2) + i * 32 + li;
      ca[i][c & 1] = *reinterpret_cast<const uint4*>(st + C::CODES + row * 128 + (((4 * h + c) ^ ((row >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int row = BM + wn * (BN / 2) + j * 32 + li;
      cb[j][c & 1] = *reinterpret_cast<const uint4*>(st + C::CODES + row * 128 + (((4 * h + c) ^ ((row >> 1) & 7)) << 4));
    }
  };
  auto read_scales = [&](const uint8_t* st, uint2* a_out, uint2* b_out) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
      a_out[i] = *reinterpret_cast<const uint2*>(st + C::SCALES + (wm * (BM / 2) + i * 32 + li) * 16 + 8 * h);
#pragma unroll
    for (int j = 0; j < WTN; ++j)
      b_out[j] = *reinterpret_cast<const uint2*>(st + C::SCALES + (BM + wn * (BN / 2) + j * 32 + li) * 16 + 8 * h);
  };
  // FP16 scale pair for chunk c (blocks 8h + 2c, 8h + 2c + 1) into slot c & 1
  auto pair = [](uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  };
  auto cvt_chunk_scales = [&](int c) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) sa[i][c & 1] = pair((c >> 1) ? sra[i].y : sra[i].x, (c & 1) != 0);
#pragma unroll
    for (int j = 0; j < WTN; ++j) sb[j][c & 1] = pair((c >> 1) ? srb[j].y : srb[j].x, (c & 1) != 0);
  };
  // K step s of a stage: dequantize the A and B fragments (codes word s % 4 of
  // chunk s / 4, block scale 8h + s / 2)
  half8_t af[2][WTM], bf[2][WTN];
  auto deq_step = [&](int s, half8_t* a_out, half8_t* b_out) {
    const int c = s >> 2;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const uint4& q = ca[i][c & 1];
      const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
      a_out[i] = dequant8h(w, (s >> 1) & 1 ? sa[i][c & 1].yy : sa[i][c & 1].xx);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const uint4& q = cb[j][c & 1];
      const uint32_t w = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
      b_out[j] = dequant8h(w, (s >> 1) & 1 ? sb[j][c & 1].yy : sb[j][c & 1].xx);
    }
  };
  // MFMAs of K step s.  With dma set, the loads of stage dma_kt into buffer
  // dma_buf are spread over the MFMAs of steps 13-15 (one instruction every
  // DMA_SP MFMAs), so the wave's vector-memory issue overlaps the matrix core
  // (step 12 carries the LDS reads that follow the stage's barrier).
  constexpr int DMA_SP = (3 * WTM * WTN) / C::LOADS;
  static_assert(DMA_SP >= 1, "DMA spacing");
  auto mfma_step = [&](int s, int dma_kt, int dma_buf, bool dma) {
#pragma unroll
    for (int k = 0; k < WTM * WTN; ++k) {
      const int i = k / WTN, j = k % WTN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
      const int g = (s - 13) * WTM * WTN + k;
      if (dma && s >= 13 && g % DMA_SP == 0 && g / DMA_SP < C::LOADS) issue_one(dma_kt, dma_buf, g / DMA_SP);
    }
  };
  // one MFMA : PACT_VALU_PER_MFMA VALU, front-loading the dequantization of
  // the next step under the first MFMAs of this one; nr LDS reads of the step
  // go one (or two) after each of its first MFMAs, so the wave's in-order
  // issue never waits behind a burst of reads
  auto interleave = [&](int nr) __attribute__((always_inline)) {
    constexpr int NM = WTM * WTN;
#pragma unroll
    for (int k = 0; k < NM; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (k < nr - NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (k < nr) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, PACT_VALU_PER_MFMA, 0);
    }
  };

  // Stage kt lives in LDS buffer kt % 2.  Its loads are issued during steps
  // 13-15 of stage kt - 2 (stages 0 and 1 in the prologue) and published by the
  // barrier at step 12 of stage kt - 1.  Each wave reads codes one chunk ahead:
  // chunk c + 1 during chunk c, and chunk 0 plus the scales of stage kt + 1
  // during chunk 3 of stage kt.  By the barrier at step 12 of stage kt every
  // wave has consumed all of stage kt's LDS data (chunk 3 is dequantized at
  // step 11), so the loads of stage kt + 2 go into its buffer right after it.
  const float* const rsc0 = reinterpret_cast<const float*>(smem + C::RSC);
  // accumulator from units of segment cseg's row scales to those of cseg + 1
  auto rescale_acc = [&](int cseg) __attribute__((always_inline)) {
    if constexpr (SEG) {
      // this lane's rows are wm (BM / 2) + 4h + (a compile-time offset), its
      // columns BM + wn (BN / 2) + li + 32 j: one base address each, so every
      // read takes an immediate offset
      const float* ro = rsc0 + cseg * C::ROWS + wm * (BM / 2) + 4 * h;
      const float* rn = ro + C::ROWS;
      const float* co = rsc0 + cseg * C::ROWS + BM + wn * (BN / 2) + li;
      const float* cn = co + C::ROWS;
      auto ex = [](float v) { return (int)((__float_as_uint(v) >> 23) & 255u); };
      int dcol[WTN];
#pragma unroll
      for (int j = 0; j < WTN; ++j) dcol[j] = ex(co[j * 32]) - ex(cn[j * 32]);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          __builtin_amdgcn_sched_barrier(0);               // a few live exponents at a time
          const int off = i * 32 + 8 * (rr >> 2) + (rr & 3);
          const int drow = ex(ro[off]) - ex(rn[off]);
#pragma unroll
          for (int j = 0; j < WTN; ++j) acc[i][j][rr] = __builtin_ldexpf(acc[i][j][rr], drow + dcol[j]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto run_stage = [&](int kt, auto dma_tag) {
    constexpr bool DMA = decltype(dma_tag)::value;
    const uint8_t* st = smem + (kt & 1) * C::STAGE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int s = 4 * c; s < 4 * c + 4; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        // the first step of chunk c reads chunk c + 1 (at chunk 3: the next
        // stage's chunk 0 and scales), spread over its MFMAs
        int nr = 0;
        if (s == 4 * c) {
          if (c < 3) {
            read_codes(st, c + 1);
            nr = WTM + WTN;
          } else {
            // publish stage kt + 1 (the only loads in flight); after the last
            // stage the reads below fetch a stale in-bounds buffer, never used
            PACT_WAIT_VMCNT(0);
            __syncthreads();
            const uint8_t* stn = smem + ((kt + 1) & 1) * C::STAGE;
            read_codes(stn, 0);
            read_scales(stn, sra_n, srb_n);
            nr = 2 * (WTM + WTN);
          }
        }
        if (s == 15) {
#pragma unroll
          for (int i = 0; i < WTM; ++i) sra[i] = sra_n[i];
#pragma unroll
          for (int j = 0; j < WTN; ++j) srb[j] = srb_n[j];
          cvt_chunk_scales(0);
          deq_step(0, af[0], bf[0]);
        } else {
          if (((s + 1) & 3) == 0) cvt_chunk_scales((s + 1) >> 2);
          deq_step(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
        }
        mfma_step(s, kt + 2, kt & 1, DMA);
        interleave(nr);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- prologue ----
  // Row scales of the tile's A rows then B rows go straight into LDS (4 bytes
  // per lane, 64 rows per instruction; rows past an operand's end read as 0
  // and are never stored), ahead of the first two stages.
  float* rsc = reinterpret_cast<float*>(smem + C::RSC);
  for (int sgi = 0; sgi < (SEG ? sg.nseg : 1); ++sgi) {
    const int4v_t ra_r = buffer_rsrc(SEG ? sg.s[sgi].a_rscale : p.a_rscale, (uint32_t)(M * 4));
    const int4v_t rb_r = buffer_rsrc(SEG ? sg.s[sgi].b_rscale : p.b_rscale, (uint32_t)(N * 4));
    const uint32_t rdst = lds0 + (uint32_t)C::RSC + (uint32_t)(sgi * C::ROWS * 4);
#pragma unroll
    for (int c = 0; c < C::NR; ++c) {
      const int q = wave_s + 4 * c;                      // instruction q: tile rows 64q .. 64q + 63
      if (q < C::NR_TOTAL) {
        if (64 * q < BM) {
          const int64_t m = m0 + 64 * q + lane;
          lds_dma_buf4(ra_r, m < M ? (uint32_t)m * 4u : 0xfffffff0u, 0u, rdst + (uint32_t)q * 256u);
        } else {
          const int64_t n = n0 + (64 * q - BM) + lane;
          lds_dma_buf4(rb_r, n < N ? (uint32_t)n * 4u : 0xfffffff0u, 0u, rdst + (uint32_t)q * 256u);
        }
      }
    }
  }
  const int nk0 = SEG ? (int)(sg.s[0].K / KT2) : nk;   // stages of the first (or only) segment
  issue_stage(0, 0);

  // The LoRA term is formed while those loads are in flight: acc starts as
  // (lora_scale / (rA rB)) * T U, so the epilogue's row-scale multiply turns
  // it into lora_scale * T U.  The T rows are scaled by f_m = lora_scale / rA
  // and the U columns by 1/rB as they are loaded (exact for power-of-two row
  // scales; see lora_factors for others), so the MFMAs produce the term
  // directly and the accumulator is never rescaled.  With a power-of-two lora_scale, T f_m is exact in BF16 (which
  // has FP32's exponent range).  Otherwise x = fl32(T f_m) is split into three
  // BF16 values hi + mid + lo = x exactly (each residual is exact in FP32 and
  // the last has at most 8 significant bits), and the term runs three MFMA
  // passes, one per piece.  (The compiler's wait for the T/U loads also covers
  // stage 0's loads issued above; stage 1's are issued after the term, so the
  // prologue never waits for them: they are needed from step 12 of stage 0.)
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  // 1/r of a power of two, exact, computed on the exponent
  auto inv_pow2 = [](float v) { return __uint_as_float((254u << 23) - __float_as_uint(v)); };
  auto is_pow2 = [](float v) { return (__float_as_uint(v) & 0x7FFFFFu) == 0u; };
  const uint32_t s_bits = __float_as_uint(p.lora_scale);
  const uint32_t s_exp = (s_bits >> 23) & 255u;
  const int npieces = ((s_bits & 0x7FFFFFu) == 0 && s_exp >= 1u && s_exp <= 254u) ? 1 : 3;
  // row scales the accumulator's units refer to (the first segment's with SEG)
  const float* const lra = SEG ? sg.s[0].a_rscale : p.a_rscale;
  const float* const lrb = SEG ? sg.s[0].b_rscale : p.b_rscale;
  // eight BF16 values times f; piece 0, 1, 2 of the exact three-way split
  auto scaled = [](uint4 v, float f, int piece) __attribute__((always_inline)) {
    auto one = [&](float x) {
      const float hi = __uint_as_float(f32_to_bf16_rne(x) << 16);
      if (piece == 0) return hi;
      const float r1 = x - hi;
      const float mid = __uint_as_float(f32_to_bf16_rne(r1) << 16);
      return piece == 1 ? mid : r1 - mid;
    };
    uint4 o;
    o.x = pack_bf16x2(one(bf16_lo(v.x) * f), one(bf16_hi(v.x) * f));
    o.y = pack_bf16x2(one(bf16_lo(v.y) * f), one(bf16_hi(v.y) * f));
    o.z = pack_bf16x2(one(bf16_lo(v.z) * f), one(bf16_hi(v.z) * f));
    o.w = pack_bf16x2(one(bf16_lo(v.w) * f), one(bf16_hi(v.w) * f));
    return __builtin_bit_cast(bf16x8_t, o);
  };
  // T row and U column factors of this lane's fragments.  A row scale of the
  // wave's rows or columns that is not a power of two (the FP32 tensor-scale
  // recipe) has no exact reciprocal on the exponent, and U / rB would not be
  // exact in BF16: such a wave ("odd") writes NaN to its part of the tile
  // (the register-staged kernel, which scales the term in FP32 after its
  // MFMAs, serves those operands).
  float fa[WTM], fb[WTN];
  bool odd_wave = false;                               // wave-uniform
  auto lora_factors = [&]() __attribute__((always_inline)) {
    bool odd = false;
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
      m = m < M ? m : M - 1;
      const float ra = lra[m];
      odd = odd || !is_pow2(ra);
      fa[i] = p.lora_scale * inv_pow2(ra);
    }
#pragma unroll
    for (int i = 0; i < WTN; ++i) {
      int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
      n = n < N ? n : N - 1;
      const float rb = lrb[n];
      odd = odd || !is_pow2(rb);
      fb[i] = inv_pow2(rb);
    }
    odd_wave = __ballot(odd) != 0ull;
  };
  // Fragments of T (rows) and U (columns) for ranks k0 .. k0 + 15.  Where a
  // fragment is not one aligned 16-byte run, its 8 elements are gathered with
  // clamped indices and selected afterwards (no branches), and every
  // fragment's loads are issued before any is used, so they are in flight
  // together.
  auto lora_load = [&](const uint16_t* lt, const uint16_t* lu, int64_t r, int64_t k0, uint4 (&tv)[WTM],
                       uint4 (&uv)[WTN]) __attribute__((always_inline)) {
    const bool t_vec = (r & 15) == 0;                          // T rows: 16-byte aligned runs of 8 ranks
    const bool u_vec = t_vec && p.u_stride_j == 1;             // U(j, n) = B[n][j]: same for B rows
    if (t_vec) {
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
        m = m < M ? m : M - 1;
        tv[i] = *reinterpret_cast<const uint4*>(lt + m * r + k0 + 8 * h);
      }
    } else {
      uint32_t e[WTM][8];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
        m = m < M ? m : M - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          e[i][t] = lt[m * r + (j < r ? j : r - 1)];
        }
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        uint32_t w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) w[t] = k0 + 8 * h + t < r ? e[i][t] : 0u;
        tv[i] = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
      }
    }
    if (u_vec) {
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
        n = n < N ? n : N - 1;
        uv[i] = *reinterpret_cast<const uint4*>(lu + n * p.u_stride_n + k0 + 8 * h);
      }
    } else {
      uint32_t e[WTN][8];
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
        n = n < N ? n : N - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          e[i][t] = lu[(j < r ? j : r - 1) * p.u_stride_j + n * p.u_stride_n];
        }
      }
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        uint32_t w[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) w[t] = k0 + 8 * h + t < r ? e[i][t] : 0u;
        uv[i] = make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16));
      }
    }
  };
  // the MFMAs of one loaded rank chunk (after lora_factors)
  auto lora_mma = [&](const uint4 (&tv)[WTM], const uint4 (&uv)[WTN]) __attribute__((always_inline)) {
    bf16x8_t uf[WTN];
    // pieces (U piece pu, T piece pt): (0, 0 .. npieces-1), or for an odd
    // wave every pair with pu + pt <= 2 (the others are below 2^-24 of the term)
#pragma unroll
    for (int i = 0; i < WTN; ++i) uf[i] = scaled(uv[i], fb[i], 0);
    for (int piece = 0; piece < npieces; ++piece) {
      bf16x8_t tf[WTM];
#pragma unroll
      for (int i = 0; i < WTM; ++i) tf[i] = scaled(tv[i], fa[i], piece);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], uf[j], acc[i][j], 0, 0, 0);
    }
  };
  // one rank-r term (T, U), a chunk of 16 ranks at a time
  auto lora_term = [&](const uint16_t* lt, const uint16_t* lu, int64_t r) __attribute__((always_inline)) {
    for (int64_t k0 = 0; k0 < r; k0 += 16) {
      uint4 tv[WTM], uv[WTN];
      lora_load(lt, lu, r, k0, tv, uv);
      lora_mma(tv, uv);
    }
  };
  bool any_lora = p.lora_t != nullptr;
  if constexpr (SEG) {
    any_lora = false;
    for (int lp = 0; lp < sg.nseg; ++lp) any_lora = any_lora || sg.s[lp].lora_t != nullptr;
  }
  if (any_lora) {
    if constexpr (SEG) {
      lora_factors();
      for (int lp = 0; lp < sg.nseg; ++lp)
        if (sg.s[lp].lora_t != nullptr) lora_term(sg.s[lp].lora_t, sg.s[lp].lora_u, sg.s[lp].lora_r);
    } else {
      // the loads of the first rank chunk go out before lora_factors' row-scale
      // loads, so both wait for memory together (a second chunk in flight as
      // well costs a register spill in the 256 x 256 tile)
      const int64_t r = p.lora_r;
      uint4 tv0[WTM], uv0[WTN];
      lora_load(p.lora_t, p.lora_u, r, 0, tv0, uv0);
      lora_factors();
      lora_mma(tv0, uv0);
      for (int64_t k0 = 16; k0 < r; k0 += 16) {
        uint4 tv[WTM], uv[WTN];
        lora_load(p.lora_t, p.lora_u, r, k0, tv, uv);
        lora_mma(tv, uv);
      }
    }
  }
  if (nk0 > 1) issue_stage(1, 1);
  if constexpr (!SEG) {
    // stage 0 (and the row scales) complete and visible
    if (nk > 1) PACT_WAIT_VMCNT(C::LOADS);
    else PACT_WAIT_VMCNT(0);
    __syncthreads();
    read_codes(smem, 0);
    read_scales(smem, sra, srb);
    cvt_chunk_scales(0);
    deq_step(0, af[0], bf[0]);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) run_stage(kt, std::true_type{});
    for (; kt < nk; ++kt) run_stage(kt, std::false_type{});
  } else {
    // one pass of the stage pipeline per segment (its first two stages'
    // loads in flight); before a later segment every wave is past its reads
    // of the stage buffers, and the accumulator changes to the segment's
    // row-scale units (one copy of the pipeline serves every segment)
    for (int sgi = 0; sgi < sg.nseg; ++sgi) {
      int nks = nk0;
      if (sgi > 0) {
        PACT_WAIT_VMCNT(0);
        __syncthreads();
        rescale_acc(sgi - 1);
        set_segment(sgi);
        nks = (int)(sg.s[sgi].K / KT2);
        issue_stage(0, 0);
        if (nks > 1) issue_stage(1, 1);
      }
      if (nks > 1) PACT_WAIT_VMCNT(C::LOADS);
      else PACT_WAIT_VMCNT(0);
      __syncthreads();
      read_codes(smem, 0);
      read_scales(smem, sra, srb);
      cvt_chunk_scales(0);
      deq_step(0, af[0], bf[0]);
      int kt = 0;
      for (; kt + 2 < nks; ++kt) run_stage(kt, std::true_type{});
      for (; kt < nks; ++kt) run_stage(kt, std::false_type{});
    }
  }
  PACT_WAIT_VMCNT(0);

  // ---- epilogue: row scales, optional accumulate, BF16 rounding ----
  // Each wave stages one 32-row slab of its tile at a time in LDS as FP32
  // (MFMA layout in, row-major out), then every lane writes 8 consecutive
  // columns of a row with one 16-byte store.
  // NaN instead of a rounded result: a wave whose LoRA term met a row scale
  // that is not a power of two poisons its part of the tile; with two or more
  // segments, a tile whose row scales (of any segment) are not all powers of
  // two poisons all of it (rows past an operand's end read as 0, a
  // power-of-two pattern)
  float poison = odd_wave ? __uint_as_float(0x7FC00000u) : 1.0f;
  if constexpr (SEG) {
    uint32_t odd = 0u;
    if (sg.nseg > 1)
      for (int q = tid; q < sg.nseg * C::ROWS; q += 256) odd |= __float_as_uint(rsc[q]) & 0x7FFFFFu;
    if (__syncthreads_or(odd != 0u) != 0) poison = __uint_as_float(0x7FC00000u);   // also the barrier below
  } else {
    __syncthreads();                                   // all waves are done reading the stage buffers
  }
  float* epi = reinterpret_cast<float*>(smem + wave * C::EPI_WAVE);
  // the lane half, derived afresh: kept live from the prologue, the register
  // allocator of the 256 x 256 tile spills it and the epilogue then waits on
  // a scratch load
  const int he = (int)(__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) >> 5);
  const float* rse = rsc + (SEG ? (sg.nseg - 1) * C::ROWS : 0);   // the last segment's row scales
  constexpr int WN = BN / 2;                            // columns of this wave's tile
  constexpr int CHUNKS = WN / 8;                        // 8-column chunks per row
  const bool vec_ok = (p.ldo % 8) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15u) == 0);
  // The row scales a slab needs are read into registers before any of its
  // staging writes: the compiler keeps LDS reads in order behind LDS writes
  // to the same array, so a read per write would wait out the LDS latency
  // once per accumulator (this lane's rows of slab i are 8g + 4h + (0..3),
  // one aligned 16-byte read per g).
  float rbv[WTN];
#pragma unroll
  for (int j = 0; j < WTN; ++j) rbv[j] = rse[BM + wn * WN + j * 32 + li] * poison;
  // a tile inside the output with 16-byte aligned rows takes the unchecked
  // slab path
  const bool full = vec_ok && m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    uint16_t* const slab_out = p.out + (m0 + wm * (BM / 2) + i * 32) * p.ldo + n0 + wn * WN;
    float4 rav[4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
      rav[g] = *reinterpret_cast<const float4*>(rse + wm * (BM / 2) + i * 32 + 8 * g + 4 * he);
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = j * 32 + li;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * he + (rr & 3);
        const float4& q = rav[rr >> 2];
        const float ra = (rr & 3) == 0 ? q.x : (rr & 3) == 1 ? q.y : (rr & 3) == 2 ? q.z : q.w;
        epi[row * C::EPI_LD + col] = acc[i][j][rr] * (ra * rbv[j]);
      }
    }
    __builtin_amdgcn_wave_barrier();                    // the slab is this wave's: LDS order suffices
    if (full) {
      slab_store<WN, C::EPI_LD>(epi, slab_out, p.ldo, p.accumulate, lane);
      __builtin_amdgcn_wave_barrier();
      continue;
    }
    for (int q = lane; q < 32 * CHUNKS; q += 64) {
      const int row = q / CHUNKS, ch = q % CHUNKS;
      const int64_t m = m0 + wm * (BM / 2) + i * 32 + row;
      const int64_t n = n0 + wn * WN + ch * 8;
      if (m >= M || n >= N) continue;
      const float* src = epi + row * C::EPI_LD + ch * 8;
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = src[t];
      uint16_t* dst = p.out + m * p.ldo + n;
      if (vec_ok && n + 8 <= N) {
        if (p.accumulate) {
          const uint4 old = *reinterpret_cast<const uint4*>(dst);
          v[0] += bf16_lo(old.x); v[1] += bf16_hi(old.x); v[2] += bf16_lo(old.y); v[3] += bf16_hi(old.y);
          v[4] += bf16_lo(old.z); v[5] += bf16_hi(old.z); v[6] += bf16_lo(old.w); v[7] += bf16_hi(old.w);
        }
        uint4 o;
        o.x = pack_bf16x2(v[0], v[1]); o.y = pack_bf16x2(v[2], v[3]);
        o.z = pack_bf16x2(v[4], v[5]); o.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(dst) = o;
      } else {
        for (int t = 0; t < 8 && n + t < N; ++t) {
          float x = v[t];
          if (p.accumulate) x += __uint_as_float((uint32_t)dst[t] << 16);
          dst[t] = (uint16_t)f32_to_bf16_rne(x);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();                    // slab consumed before the next one is written
  }
}

void gemm_tile(int64_t M, int64_t N, int* bm, int* bn) {
  auto ntiles = [&](int64_t tm, int64_t tn) { return ((M + tm - 1) / tm) * ((N + tn - 1) / tn); };
  if (ntiles(256, 256) >= 384) { *bm = 256; *bn = 256; return; }
  if (ntiles(256, 192) >= 192) { *bm = 256; *bn = 192; return; }
  if (ntiles(256, 128) >= 256) { *bm = 256; *bn = 128; return; }
  *bm = 128; *bn = 128;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  int bm, bn;
  gemm_tile(a.M, a.N, &bm, &bn);
  const int tm = (int)((a.M + bm - 1) / bm), tn = (int)((a.N + bn - 1) / bn);
  // fast path: K a multiple of the stage length and every operand addressable
  // with 32-bit buffer offsets, unless the caller asks for the general one
  // (its LoRA term takes any row scale; the fast kernel's needs powers of two)
  const bool fast = !a.general && (a.K % KT2) == 0 &&
                    (uint64_t)(a.M > a.N ? a.M : a.N) * (uint64_t)(a.K / 2) < (1ull << 31);
  if (fast) {
    const SegArgs none{};
    if (bm == 256 && bn == 256) k_gemm_nvfp4_fast<4, 4><<<tm * tn, 256, 0, s>>>(a, tm, tn, none);
    else if (bn == 192) k_gemm_nvfp4_fast<4, 3><<<tm * tn, 256, 0, s>>>(a, tm, tn, none);
    else if (bm == 256) k_gemm_nvfp4_fast<4, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn, none);
    else k_gemm_nvfp4_fast<2, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn, none);
  } else {
    // generic contraction lengths: register-staged kernel (tile shapes 256x256, 256x128, 128x128)
    if (bm == 256 && bn == 256) k_gemm_nvfp4<4, 4><<<tm * tn, 256, 0, s>>>(a, tm, tn);
    else if (bm == 256) {
      const int tn2 = (int)((a.N + 127) / 128);
      k_gemm_nvfp4<4, 2><<<tm * tn2, 256, 0, s>>>(a, tm, tn2);
    } else k_gemm_nvfp4<2, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  }
  return hipGetLastError();
}

// Input gradient summed over segments (sg): a.M x a.N output, every segment's
// contraction a multiple of the stage and addressable with 32-bit buffer
// offsets (checked by the caller, gemm_multi_supported).
bool gemm_multi_supported(const GemmArgs& a, const SegArgs& sg) {
  if (sg.nseg < 1 || sg.nseg > kMaxSeg) return false;
  for (int i = 0; i < sg.nseg; ++i) {
    const int64_t Ks = sg.s[i].K;
    if (Ks <= 0 || Ks % KT2 != 0) return false;
    if ((uint64_t)(a.M > a.N ? a.M : a.N) * (uint64_t)(Ks / 2) >= (1ull << 31)) return false;
  }
  return true;
}

// The segmented kernel has no 256 x 256 instantiation: with the segment loop
// around the pipeline that tile's per-lane load offsets no longer fit in
// registers (hundreds of spilled values, reloaded before every segment's first
// loads), while 256 x 192 tiles stay spill-free at the same MFMA rate per tile
// column.
void gemm_multi_tile(int64_t M, int64_t N, int* bm, int* bn) {
  gemm_tile(M, N, bm, bn);
  if (*bm == 256 && *bn == 256) *bn = 192;
}

hipError_t launch_gemm_multi(const GemmArgs& a, const SegArgs& sg, hipStream_t s) {
  int bm, bn;
  gemm_multi_tile(a.M, a.N, &bm, &bn);
  const int tm = (int)((a.M + bm - 1) / bm), tn = (int)((a.N + bn - 1) / bn);
  if (bn == 192) k_gemm_nvfp4_fast<4, 3, true><<<tm * tn, 256, 0, s>>>(a, tm, tn, sg);
  else if (bm == 256) k_gemm_nvfp4_fast<4, 2, true><<<tm * tn, 256, 0, s>>>(a, tm, tn, sg);
  else k_gemm_nvfp4_fast<2, 2, true><<<tm * tn, 256, 0, s>>>(a, tm, tn, sg);
  return hipGetLastError();
}

}  // namespace pact
