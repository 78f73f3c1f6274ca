// MXFP4 variant of the frozen-projection path: quantizers and the GEMM on
// gfx950's scaled FP4 matrix instructions.
//
// Format (PACT, Appendix Table 6, MXFP4 column): 32-element blocks, E2M1
// elements, one E8M0 scale per block, 4.25 bits per element, no other scale.
// Block scale (the OCP microscaling rule): shared exponent
// e = floor(log2(blockmax)) - 2 clamped to [-127, 127] (-127 for an all-zero
// block), stored as the byte e + 127; element code = RNE(|x| / 2^e) onto E2M1,
// ties to even, saturating at 6, sign kept.  |x| / 2^e is an exact power-of-
// two scaling (2^-e is a normal FP32 number for every e a finite FP32 block
// maximum can produce), and v_cvt_scalef32_pk_fp4_f32 with scale 1.0 performs
// the RNE, saturation and sign handling.
//
// GEMM.  v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4 takes, per
// lane (i = lane % 32, h = lane / 32), row i's 32 elements K = 32h .. 32h + 31
// (16 bytes) and one E8M0 scale byte for them (selected from a VGPR by
// op_sel): exactly one MX block per lane.  The hardware applies both scales,
// so the kernel does no dequantization; the accumulator layout is that of
// v_mfma_f32_32x32x16_f16.  Tiling follows the NVFP4 kernel (4 waves as 2 x 2,
// XCD-aware tile order, buffer loads straight into LDS with range-checked zero
// fill), with K stages of 128 and four LDS buffers: a stage takes a quarter of
// the MFMA time of an NVFP4 stage, so loads are issued three stages ahead.
#include <type_traits>

#include "lds_dma.h"
#include "pact_internal.h"

namespace pact {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kMxBlock = 32;

// floor(log2(amax)) - 2, clamped to [-127, 127]; -127 for amax == 0 (amax >= 0 finite).
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u == 0u) return -127;
  const int ef = (int)(u >> 23);
  const int fl = ef != 0 ? ef - 127 : (31 - __builtin_clz(u & 0x7FFFFFu)) - 149;   // subnormal amax
  const int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// 8 elements times 2^-e -> 8 packed E2M1 codes (element 0 in the low nibble).
__device__ __forceinline__ uint32_t mx_encode8(const float* x, float inv) {
  uint32_t w = 0u;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0] * inv, x[1] * inv, 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2] * inv, x[3] * inv, 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4] * inv, x[5] * inv, 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6] * inv, x[7] * inv, 1.0f, 3);
  return w;
}

// 2^-e as FP32 for e in [-127, 125] (a normal number)
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------------------
// Row quantizer: thread q handles chunk q (8 elements) of the [rows x cols]
// input; chunks 4p .. 4p + 3 are one block, held by four consecutive lanes.
// No row-level reduction is needed, so every block is independent.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_mx_quantize_rows(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t cpr = cols >> 3;                    // chunks per row (a multiple of 4)
  const int64_t total = rows * cpr;
  // q % 4 == lane % 4 and total % 4 == 0, so the four lanes of a block take
  // the same trip count and hold chunks 4p .. 4p + 3 of one row
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < total; q += (int64_t)gridDim.x * 256) {
    const int64_t row = q / cpr, c = q - row * cpr;
    float f[8];
    unpack_bf16x8(*reinterpret_cast<const uint4*>(x + row * ldx + 8 * c), f);
    float m = absmax8(f);
    m = fmaxf(m, __shfl_xor(m, 1, 64));
    m = fmaxf(m, __shfl_xor(m, 2, 64));
    const int e = mx_shared_exp(m);
    *reinterpret_cast<uint32_t*>(codes + row * (cols >> 1) + 4 * c) = mx_encode8(f, mx_inv_scale(e));
    if ((c & 3) == 0) scales[row * (cols >> 5) + (c >> 2)] = (uint8_t)(e + 127);
  }
}

// Transposed quantizer: output row i is column i of x [cols x rows] (the
// cached backward weight layout W_bwd = Q(W^T)).  A workgroup owns 64
// consecutive output rows (lane i of each wave reads x[j][i0 + i], so a wave's
// loads are 128 contiguous bytes per j); its 4 waves take interleaved blocks.
__global__ __launch_bounds__(256) void k_mx_quantize_cols(const uint16_t* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ldx, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int li = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + li;
  const bool ok = i < rows;
  const int64_t ic = ok ? i : rows - 1;
  const int64_t nblk = cols >> 5;
  for (int64_t b = g; b < nblk; b += 4) {
    float f[32];
    float m = 0.0f;
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      f[t] = bf16_lo(x[(32 * b + t) * ldx + ic]);
      m = fmaxf(m, fabsf(f[t]));
    }
    const int e = mx_shared_exp(m);
    const float inv = mx_inv_scale(e);
    if (ok) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(codes + i * (cols >> 1) + 16 * b);
#pragma unroll
      for (int w = 0; w < 4; ++w) dst[w] = mx_encode8(f + 8 * w, inv);
      scales[i * nblk + b] = (uint8_t)(e + 127);
    }
  }
}

// ---------------------------------------------------------------------------
// GEMM: C = A B^T, A = MXFP4 [M x K], B = MXFP4 [N x K], FP32 accumulation,
// BF16 output (optionally C = bf16(f32(C) + A B^T)).
// ---------------------------------------------------------------------------
template <int WTM, int WTN>
struct MxCfg {
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 64 * WTN;
  static constexpr int ROWS = BM + BN;
  static constexpr int KS = 128;                        // K elements per stage
  static constexpr int CODES = 0;                       // [ROWS][64] swizzled by (row >> 2) & 3
  static constexpr int SCALES = ROWS * 64;              // [ROWS][4] (4 blocks of 32 per stage)
  static constexpr int NC = ROWS / 64;                  // code load instructions per wave per stage (16 rows each)
  static constexpr int NS_TOTAL = ROWS / 64;            // scale load instructions per stage (64 rows each)
  static constexpr int NS = (NS_TOTAL + 3) / 4;         // per wave; surplus ones fill a pad region with zeros
  static constexpr int PAD = SCALES + ROWS * 4;
  static constexpr int STAGE = PAD + (NS * 4 - NS_TOTAL) * 256;
  static constexpr int NSTAGE = 4;
  static constexpr int LOADS = NC + NS;
  static constexpr int EPI_LD = BN / 2 + 4;
  static constexpr int EPI_WAVE = 32 * EPI_LD * 4;
  static constexpr int TOTAL = NSTAGE * STAGE > 4 * EPI_WAVE ? NSTAGE * STAGE : 4 * EPI_WAVE;
  static_assert(ROWS % 64 == 0 && BM % 64 == 0, "tile rows");
  static_assert(2 * LOADS <= 63 && 3 * LOADS <= 63, "vmcnt range");
};

struct MxGemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int64_t M, N, K;
  uint16_t* out;
  int64_t ldo;
  int accumulate;
};

__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) { return pack_bf16x2(lo, hi); }

template <int WTM, int WTN>
__global__ __launch_bounds__(256, 1) void k_gemm_mxfp4(MxGemmArgs p, int tiles_m, int tiles_n) {
  using C = MxCfg<WTM, WTN>;
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
  const uint32_t crow = (uint32_t)(K >> 1), srow = (uint32_t)(K >> 5);
  const int nk = (int)(K / C::KS);

  // ---- load addressing ----
  // Code instruction c of this wave covers tile rows 16 (wave + 4c) .. +15:
  // lane -> row 16 (wave + 4c) + lane / 4, LDS slot lane % 4, global chunk
  // slot ^ ((row >> 2) & 3) = slot ^ ((lane >> 4) & 3).
  const int4v_t ra_c = buffer_rsrc(p.a_codes, (uint32_t)(M * crow));
  const int4v_t rb_c = buffer_rsrc(p.b_codes, (uint32_t)(N * crow));
  const int4v_t ra_s = buffer_rsrc(p.a_scales, (uint32_t)(M * srow));
  const int4v_t rb_s = buffer_rsrc(p.b_scales, (uint32_t)(N * srow));
  const uint32_t cchunk = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  uint32_t cvo[C::NC];
#pragma unroll
  for (int c = 0; c < C::NC; ++c) {
    const int row = 16 * (wave + 4 * c) + (lane >> 2);
    uint32_t v = 0xfffffff0u;
    if (row < BM) {
      const int64_t m = m0 + row;
      if (m < M) v = (uint32_t)m * crow + cchunk;
    } else {
      const int64_t n = n0 + (row - BM);
      if (n < N) v = (uint32_t)n * crow + cchunk;
    }
    cvo[c] = v;
  }
  uint32_t svo[C::NS];
#pragma unroll
  for (int c = 0; c < C::NS; ++c) {
    const int q = wave + 4 * c;
    const int row = 64 * q + lane;
    uint32_t v = 0xfffffff0u;
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
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  auto issue_one = [&](int kt, int buf, int q) {
    const uint32_t st = lds0 + (uint32_t)(buf * C::STAGE);
    if (q < C::NC) {
      static_assert(BM % 64 == 0, "A/B split on an instruction boundary");
      const uint32_t dst = st + C::CODES + (uint32_t)(wave_s + 4 * q) * 1024u;
      const uint32_t soff = (uint32_t)kt * 64u;
      if (16 * (4 * q + 3) + 15 < BM) lds_dma_buf16(ra_c, cvo[q], soff, dst);
      else lds_dma_buf16(rb_c, cvo[q], soff, dst);
    } else {
      const int c = q - C::NC;
      const int qq = wave_s + 4 * c;
      const uint32_t dst = qq < C::NS_TOTAL ? st + C::SCALES + (uint32_t)qq * 256u
                                            : st + C::PAD + (uint32_t)(qq - C::NS_TOTAL) * 256u;
      const uint32_t soff = (uint32_t)kt * 4u;
      if (64 * (4 * c + 3) + 63 < BM) lds_dma_buf4(ra_s, svo[c], soff, dst);
      else if (256 * c >= BM) lds_dma_buf4(rb_s, svo[c], soff, dst);
      else if (qq * 64 < BM) lds_dma_buf4(ra_s, svo[c], soff, dst);   // split by wave: uniform branch
      else lds_dma_buf4(rb_s, svo[c], soff, dst);
    }
  };
  auto issue_stage = [&](int kt, int buf) {
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q) issue_one(kt, buf, q);
  };

  // ---- fragments ----
  // step s (0, 1) of a stage: lane (i, h) holds row i's K = 64 s + 32 h .. + 32
  // (16 bytes, chunk 2s + h of the row) and the scale of that block.
  uint4 fa[2][WTM], fb[2][WTN];
  uint32_t sa[WTM], sb[WTN], sa_n[WTM], sb_n[WTN];
  auto read_frags = [&](const uint8_t* st, int s, int slot) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = wm * (BM / 2) + i * 32 + li;
      fa[slot][i] = *reinterpret_cast<const uint4*>(st + C::CODES + row * 64 + (((2 * s + h) ^ ((row >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int row = BM + wn * (BN / 2) + j * 32 + li;
      fb[slot][j] = *reinterpret_cast<const uint4*>(st + C::CODES + row * 64 + (((2 * s + h) ^ ((row >> 2) & 3)) << 4));
    }
  };
  // scale dword of a row holds blocks 0..3 of the stage; lane half h needs
  // blocks h (step 0) and 2 + h (step 1): moved to bytes 0 and 1
  const uint32_t ssel = h ? 0x0c0c0301u : 0x0c0c0200u;
  auto read_scales = [&](const uint8_t* st, uint32_t* a_out, uint32_t* b_out) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(st + C::SCALES + (wm * (BM / 2) + i * 32 + li) * 4);
      a_out[i] = __builtin_amdgcn_perm(w, w, ssel);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(st + C::SCALES + (BM + wn * (BN / 2) + j * 32 + li) * 4);
      b_out[j] = __builtin_amdgcn_perm(w, w, ssel);
    }
  };

  floatx16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto v8 = [](const uint4& q) {
    v8i_t r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
    return r;
  };
  // MFMAs of step s (scale byte s), optionally with the loads of stage dma_kt
  // into buffer dma_buf spread one per MFMA
  auto mfma_step = [&](int s, int slot, bool dma, int dma_kt, int dma_buf) {
#pragma unroll
    for (int k = 0; k < WTM * WTN; ++k) {
      const int i = k / WTN, j = k % WTN;
      if (s == 0)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8(fa[slot][i]), v8(fb[slot][j]), acc[i][j], 4, 4,
                                                                    0, (int)sa[i], 0, (int)sb[j]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8(fa[slot][i]), v8(fb[slot][j]), acc[i][j], 4, 4,
                                                                    1, (int)sa[i], 1, (int)sb[j]);
      if (dma && k < C::LOADS) issue_one(dma_kt, dma_buf, k);
    }
    if (dma) {
#pragma unroll
      for (int q = WTM * WTN; q < C::LOADS; ++q) issue_one(dma_kt, dma_buf, q);   // small tiles: the rest
    }
  };

  // Stage kt lives in buffer kt % 4; its loads are issued during step 1 of
  // stage kt - 4 (stages 0..3 in the prologue) and published by the barrier
  // at step 1 of stage kt - 1, after which every wave has read stage kt - 1
  // completely (its step-1 fragments were read during step 0).
  auto wait_for_next = [&](int kt) {
    // loads in flight: stages kt+1 .. min(kt+3, nk-1); keep all but the oldest
    const int inflight = min(nk - 1, kt + 3) - kt;
    if (inflight >= 3) PACT_WAIT_VMCNT(2 * C::LOADS);
    else if (inflight == 2) PACT_WAIT_VMCNT(C::LOADS);
    else PACT_WAIT_VMCNT(0);
  };
  auto run_stage = [&](int kt, auto dma_tag) {
    constexpr bool DMA = decltype(dma_tag)::value;
    const uint8_t* st = smem + (kt & 3) * C::STAGE;
    // step 0
    read_frags(st, 1, 1);
    mfma_step(0, 0, false, 0, 0);
    // step 1: publish stage kt + 1, refill buffer kt % 4 with stage kt + 4
    __builtin_amdgcn_s_waitcnt(0xc07f);                    // lgkmcnt(0): this wave's reads of stage kt done
    wait_for_next(kt);
    __syncthreads();
    const uint8_t* stn = smem + ((kt + 1) & 3) * C::STAGE;   // stale (in-bounds) after the last stage
    read_frags(stn, 0, 0);
    read_scales(stn, sa_n, sb_n);
    mfma_step(1, 1, DMA, kt + 4, kt & 3);
#pragma unroll
    for (int i = 0; i < WTM; ++i) sa[i] = sa_n[i];
#pragma unroll
    for (int j = 0; j < WTN; ++j) sb[j] = sb_n[j];
  };

  // prologue: stages 0..3 in flight, wait for stage 0
  const int pre = nk < 4 ? nk : 4;
  for (int q = 0; q < pre; ++q) issue_stage(q, q);
  if (pre >= 4) PACT_WAIT_VMCNT(3 * C::LOADS);
  else if (pre == 3) PACT_WAIT_VMCNT(2 * C::LOADS);
  else if (pre == 2) PACT_WAIT_VMCNT(C::LOADS);
  else PACT_WAIT_VMCNT(0);
  __syncthreads();
  read_frags(smem, 0, 0);
  read_scales(smem, sa, sb);
  int kt = 0;
  for (; kt + 4 < nk; ++kt) run_stage(kt, std::true_type{});
  for (; kt < nk; ++kt) run_stage(kt, std::false_type{});
  PACT_WAIT_VMCNT(0);

  // ---- epilogue: optional accumulate, BF16 rounding, staged through LDS ----
  __syncthreads();
  float* epi = reinterpret_cast<float*>(smem + wave * C::EPI_WAVE);
  constexpr int WN = BN / 2;
  constexpr int CHUNKS = WN / 8;
  const bool vec_ok = (p.ldo % 8) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15u) == 0);
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = j * 32 + li;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * h + (rr & 3);
        epi[row * C::EPI_LD + col] = acc[i][j][rr];
      }
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);
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
        o.x = bf16_pack2(v[0], v[1]); o.y = bf16_pack2(v[2], v[3]);
        o.z = bf16_pack2(v[4], v[5]); o.w = bf16_pack2(v[6], v[7]);
        *reinterpret_cast<uint4*>(dst) = o;
      } else {
        for (int t = 0; t < 8 && n + t < N; ++t) {
          float xv = v[t];
          if (p.accumulate) xv += __uint_as_float((uint32_t)dst[t] << 16);
          dst[t] = (uint16_t)f32_to_bf16_rne(xv);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                              uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (transpose) {
    k_mx_quantize_cols<<<(unsigned)((rows + 63) / 64), 256, 0, s>>>(x, rows, cols, ldx, codes, scales);
    return hipGetLastError();
  }
  const int64_t total = rows * (cols >> 3);
  const int64_t blocks = (total + 255) / 256;
  k_mx_quantize_rows<<<(unsigned)(blocks < 8192 ? blocks : 8192), 256, 0, s>>>(x, rows, cols, ldx, codes, scales);
  return hipGetLastError();
}

bool mx_gemm_supported(int64_t M, int64_t N, int64_t K) {
  return K % 128 == 0 && (uint64_t)(M > N ? M : N) * (uint64_t)(K / 2) < (1ull << 31);
}

hipError_t launch_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t M, int64_t K, const uint8_t* bc,
                          const uint8_t* bs, int64_t N, uint16_t* out, int64_t ldo, int accumulate, hipStream_t s) {
  MxGemmArgs a{ac, as, bc, bs, M, N, K, out, ldo, accumulate};
  int bm, bn;
  gemm_tile(M, N, &bm, &bn);
  const int tm = (int)((M + bm - 1) / bm), tn = (int)((N + bn - 1) / bn);
  if (bm == 256 && bn == 256) k_gemm_mxfp4<4, 4><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  else if (bn == 192) k_gemm_mxfp4<4, 3><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  else if (bm == 256) k_gemm_mxfp4<4, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  else k_gemm_mxfp4<2, 2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  return hipGetLastError();
}

}  // namespace pact
