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

void gemm_tile(int64_t M, int64_t N, int* bm, int* bn) {
  auto ntiles = [&](int64_t tm, int64_t tn) { return ((M + tm - 1) / tm) * ((N + tn - 1) / tn); };
  if (ntiles(256, 256) >= 256) { *bm = 256; *bn = 256; return; }
  if (ntiles(256, 128) >= 256) { *bm = 256; *bn = 128; return; }
  *bm = 128; *bn = 128;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s) {
  int bm, bn;
  gemm_tile(a.M, a.N, &bm, &bn);
  const int tm = (int)((a.M + bm - 1) / bm), tn = (int)((a.N + bn - 1) / bn);
  if (bm == 256 && bn == 256) k_gemm_nvfp4<4, 4><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  else if (bm == 256) k_gemm_nvfp4<4, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  else k_gemm_nvfp4<2, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  return hipGetLastError();
}

}  // namespace pact
