// NVFP4 x NVFP4 -> BF16 GEMM for the frozen projections: C = A B^T with both
// operands row-blocked NVFP4 (PACT, Appendix Table 7 row "Frozen projections":
// NVFP4 GEMMs with FP32 accumulation and BF16 output, forward and input
// gradient over cached forward and backward weight layouts).  With
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
// (BM/2) x (BN/2) as WTM x WTN MFMA tiles of 32 x 32.  K advances in stages of
// 128 (8 NVFP4 blocks): packed codes (64 B per row) and the block scales
// (converted once to FP16 pairs) are staged in LDS, double buffered, with the
// next stage's global loads issued before the current stage's MFMAs.  Within a
// stage, lane half h of a wave owns K range [64h, 64h+64) of every row it
// touches, so each fragment is one 32-byte LDS read of codes plus one 16-byte
// read of scales; MFMA step s takes K = 64h + 8s + t (t = 0..7) from both
// operands, a consistent permutation of K.
#include "pact_internal.h"

namespace pact {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int KT = 128;            // K elements per stage
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

__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t sp) {
  const half2_t s = __builtin_bit_cast(half2_t, sp);
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ __bf16 bf16_of(uint16_t v) { return __builtin_bit_cast(__bf16, v); }

// 8 codes of one word times a broadcast FP16 scale (both halves equal).
__device__ __forceinline__ half8_t dequant8h(uint32_t w, half2_t s) {
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
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
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
        m = m < M ? m : M - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          tf[i][t] = bf16_of(j < r ? p.lora_t[m * r + j] : (uint16_t)0);
        }
      }
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
        n = n < N ? n : N - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          uf[i][t] = bf16_of(j < r ? p.lora_u[j * p.u_stride_j + n * p.u_stride_n] : (uint16_t)0);
        }
      }
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
      ga[it] = b < kb ? *reinterpret_cast<const uint2*>(p.a_codes + m * crow + b * 8) : make_uint2(0, 0);
    }
#pragma unroll
    for (int it = 0; it < C::NCODE_B; ++it) {
      const int q = tid + 256 * it;
      const int row = q >> 3, blk = q & 7;
      int64_t n = n0 + row;
      n = n < N ? n : N - 1;
      const int64_t b = (int64_t)kt * 8 + blk;
      gb[it] = b < kb ? *reinterpret_cast<const uint2*>(p.b_codes + n * crow + b * 8) : make_uint2(0, 0);
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
// Fast path (K % 128 == 0): global -> LDS direct loads, three LDS stages.
//
// Each K stage holds, for the BM + BN rows of the tile, 64 bytes of codes and
// 8 bytes of raw E4M3 scales per row.  Loads use global_load_lds (16 bytes
// per lane for codes, 4 for scales), which write 64 consecutive lane slots of
// LDS per instruction, so no registers stage the data.  Instead of padding, a
// row's four 16-byte code chunks are stored XOR-swizzled by (row >> 1) & 3,
// which makes the fragment reads (8 consecutive rows per 128-byte LDS cycle)
// bank-conflict free.  Scales are converted per fragment with
// v_cvt_scalef32_pk_f16_fp8 and applied with a broadcast v_pk_mul_f16.
// ===========================================================================
template <int WTM, int WTN>
struct FastCfg {
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 64 * WTN;
  static constexpr int ROWS = BM + BN;
  static constexpr int CODES = 0;                       // [ROWS][64] swizzled
  static constexpr int SCALES = ROWS * 64;              // [ROWS][8]
  static constexpr int NC = ROWS / 64;                  // 16-byte code load instructions per wave per stage
  static constexpr int NS_TOTAL = ROWS / 32;            // 4-byte scale load instructions per stage
  static constexpr int NS = (NS_TOTAL + 3) / 4;         // per wave (the surplus ones fill a pad region)
  static constexpr int PAD = SCALES + ROWS * 8;         // 256 bytes per surplus instruction
  static constexpr int STAGE = PAD + (NS * 4 - NS_TOTAL) * 256;
  static constexpr int NSTAGE = 3;
  static constexpr int LOADS = NC + NS;                 // vmcnt per stage per wave
  // epilogue: per wave, one 32-row slab of its (BN/2)-column tile as FP32
  static constexpr int EPI_LD = BN / 2 + 4;             // floats per staged row (pad breaks bank aliasing)
  static constexpr int EPI_WAVE = 32 * EPI_LD * 4;      // bytes per wave
  static constexpr int MAIN = NSTAGE * STAGE > 4 * EPI_WAVE ? NSTAGE * STAGE : 4 * EPI_WAVE;
  static constexpr int RSC = MAIN;                      // row scales of A (BM floats) then B (BN floats)
  static constexpr int TOTAL = RSC + ROWS * 4;
};

// Global -> LDS loads of 16 / 4 bytes per lane.  Issued through inline asm so
// that the compiler does not treat every later LDS read as a possible alias of
// the asynchronous write (it would then wait for all outstanding loads, which
// serializes the stage pipeline); the kernel waits for them explicitly with
// s_waitcnt vmcnt before the barrier that publishes a stage.  M0 holds the
// wave-uniform LDS destination; lane i writes bytes [16 i, 16 i + 16) (or
// [4 i, 4 i + 4)) after it.
__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gptr), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
#define PACT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

template <int WTM, int WTN>
__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4_fast(GemmArgs p, int tiles_m, int tiles_n) {
  using C = FastCfg<WTM, WTN>;
  constexpr int BM = C::BM, BN = C::BN;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::TOTAL];

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
  const int64_t crow = K >> 1, srow = K >> 4;
  const int nk = (int)(K / KT);

  // row scales of this tile's A rows and B rows, staged once (clamped at the edges)
  float* rsc = reinterpret_cast<float*>(smem + C::RSC);
  for (int q = tid; q < C::ROWS; q += 256) {
    if (q < BM) {
      const int64_t m = m0 + q;
      rsc[q] = p.a_rscale[m < M ? m : M - 1];
    } else {
      const int64_t n = n0 + (q - BM);
      rsc[q] = p.b_rscale[n < N ? n : N - 1];
    }
  }
  __syncthreads();

  floatx16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  if (p.lora_t != nullptr) {
    const int64_t r = p.lora_r;
    for (int64_t k0 = 0; k0 < r; k0 += 16) {
      bf16x8_t tf[WTM], uf[WTN];
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
        m = m < M ? m : M - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          tf[i][t] = bf16_of(j < r ? p.lora_t[m * r + j] : (uint16_t)0);
        }
      }
#pragma unroll
      for (int i = 0; i < WTN; ++i) {
        int64_t n = n0 + wn * (BN / 2) + i * 32 + li;
        n = n < N ? n : N - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = k0 + 8 * h + t;
          uf[i][t] = bf16_of(j < r ? p.lora_u[j * p.u_stride_j + n * p.u_stride_n] : (uint16_t)0);
        }
      }
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], uf[j], acc[i][j], 0, 0, 0);
    }
    // row scales are powers of two: 1/r is exact and computed on the exponent
    auto inv_pow2 = [](float r) { return __uint_as_float((254u << 23) - __float_as_uint(r)); };
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = wm * (BM / 2) + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        const float fa = p.lora_scale * inv_pow2(rsc[row]);
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
          const int col = wn * (BN / 2) + j * 32 + li;
          acc[i][j][rr] *= fa * inv_pow2(rsc[BM + col]);
        }
      }
  }

  // ---- per-lane global source addresses for this wave's load instructions ----
  // code instruction q (q = wave + 4 * c): rows 16q .. 16q+15, lane -> row 16q + lane/4, LDS slot lane%4
  const uint8_t* csrc[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    const int q = wave + 4 * c;
    const int row = 16 * q + (lane >> 2);
    const int slot = lane & 3;
    const int chunk = slot ^ ((row >> 1) & 3);
    if (row < BM) {
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      csrc[c] = p.a_codes + m * crow + chunk * 16;
    } else {
      int64_t n = n0 + (row - BM);
      n = n < N ? n : N - 1;
      csrc[c] = p.b_codes + n * crow + chunk * 16;
    }
  }
  // scale instruction q: rows 32q .. 32q+31, lane -> row 32q + lane/2, dword lane%2
  const uint8_t* ssrc[C::NS];
#pragma unroll
  for (int c = 0; c < C::NS; ++c) {
    const int q = wave + 4 * c;
    int row = 32 * q + (lane >> 1);
    if (q >= C::NS_TOTAL) row = 0;                    // surplus instruction: any valid address
    if (row < BM) {
      int64_t m = m0 + row;
      m = m < M ? m : M - 1;
      ssrc[c] = p.a_scales + m * srow + (lane & 1) * 4;
    } else {
      int64_t n = n0 + (row - BM);
      n = n < N ? n : N - 1;
      ssrc[c] = p.b_scales + n * srow + (lane & 1) * 4;
    }
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  auto issue_stage = [&](int kt, int buf) {
    const uint32_t st = lds0 + (uint32_t)(buf * C::STAGE);
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const int q = wave_s + 4 * c;
      lds_dma16(csrc[c] + (int64_t)kt * 64, st + C::CODES + q * 1024);
    }
#pragma unroll
    for (int c = 0; c < C::NS; ++c) {
      const int q = wave_s + 4 * c;
      const uint32_t dst = q < C::NS_TOTAL ? st + C::SCALES + q * 256 : st + C::PAD + (q - C::NS_TOTAL) * 256;
      lds_dma4(ssrc[c] + (int64_t)kt * 8, dst);
    }
  };

  issue_stage(0, 0);
  if (nk > 1) issue_stage(1, 1);

  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) PACT_WAIT_VMCNT(C::LOADS);
    else PACT_WAIT_VMCNT(0);
    __syncthreads();
    if (kt + 2 < nk) issue_stage(kt + 2, (kt + 2) % 3);
    const uint8_t* st = smem + (kt % 3) * C::STAGE;

    uint4 ca[WTM][2], cb[WTN][2];
    half2_t sa[WTM][2], sb[WTN][2];
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = wm * (BM / 2) + i * 32 + li;
      const int sw = (row >> 1) & 3;
      const uint8_t* rp = st + C::CODES + row * 64;
      ca[i][0] = *reinterpret_cast<const uint4*>(rp + (((2 * h) ^ sw) << 4));
      ca[i][1] = *reinterpret_cast<const uint4*>(rp + (((2 * h + 1) ^ sw) << 4));
      const uint32_t sraw = *reinterpret_cast<const uint32_t*>(st + C::SCALES + row * 8 + 4 * h);
      sa[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw, 1.0f, false);
      sa[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw, 1.0f, true);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int row = BM + wn * (BN / 2) + j * 32 + li;
      const int sw = (row >> 1) & 3;
      const uint8_t* rp = st + C::CODES + row * 64;
      cb[j][0] = *reinterpret_cast<const uint4*>(rp + (((2 * h) ^ sw) << 4));
      cb[j][1] = *reinterpret_cast<const uint4*>(rp + (((2 * h + 1) ^ sw) << 4));
      const uint32_t sraw = *reinterpret_cast<const uint32_t*>(st + C::SCALES + row * 8 + 4 * h);
      sb[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw, 1.0f, false);
      sb[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sraw, 1.0f, true);
    }
    // software pipeline over the 8 K16 steps: dequantize step s+1 while the
    // MFMAs of step s run, interleaved 1 MFMA : 4 VALU
    half8_t af[2][WTM], bf[2][WTN];
    auto deq_step = [&](int s, half8_t* a_out, half8_t* b_out) {
#pragma unroll
      for (int i = 0; i < WTM; ++i) {
        const uint4& c = ca[i][s >> 2];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        const half2_t sp = (s >> 1) & 1 ? sa[i][s >> 2].yy : sa[i][s >> 2].xx;
        a_out[i] = dequant8h(w, sp);
      }
#pragma unroll
      for (int j = 0; j < WTN; ++j) {
        const uint4& c = cb[j][s >> 2];
        const uint32_t w = (s & 3) == 0 ? c.x : (s & 3) == 1 ? c.y : (s & 3) == 2 ? c.z : c.w;
        const half2_t sp = (s >> 1) & 1 ? sb[j][s >> 2].yy : sb[j][s >> 2].xx;
        b_out[j] = dequant8h(w, sp);
      }
    };
    deq_step(0, af[0], bf[0]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      if (s < 7) deq_step(s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][i], bf[s & 1][j], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < WTM * WTN; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // four VALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- epilogue: row scales, optional accumulate, BF16 rounding ----
  // Each wave stages one 32-row slab of its tile at a time in LDS as FP32
  // (MFMA layout in, row-major out), then every lane writes 8 consecutive
  // columns of a row with one 16-byte store.
  __syncthreads();                                     // all waves are done reading the stage buffers
  float* epi = reinterpret_cast<float*>(smem + wave * C::EPI_WAVE);
  constexpr int WN = BN / 2;                            // columns of this wave's tile
  constexpr int CHUNKS = WN / 8;                        // 8-column chunks per row
  const bool vec_ok = (p.ldo % 8) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15u) == 0);
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = j * 32 + li;
      const float rb = rsc[BM + wn * WN + col];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * h + (rr & 3);
        epi[row * C::EPI_LD + col] = acc[i][j][rr] * (rsc[wm * (BM / 2) + i * 32 + row] * rb);
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                 // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();
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
  const bool fast = (a.K % KT) == 0;
  if (fast) {
    if (bm == 256 && bn == 256) k_gemm_nvfp4_fast<4, 4><<<tm * tn, 256, 0, s>>>(a, tm, tn);
    else if (bn == 192) k_gemm_nvfp4_fast<4, 3><<<tm * tn, 256, 0, s>>>(a, tm, tn);
    else if (bm == 256) k_gemm_nvfp4_fast<4, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
    else k_gemm_nvfp4_fast<2, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
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

}  // namespace pact
