// MXFP4 variant of the frozen-projection path: quantizers and the GEMM on
// gfx950's scaled FP4 matrix instructions.
//
// Format and block rule: mxfp4_device.h (Appendix Table 6, MXFP4 column).
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
#include <utility>

#include "epilogue.h"
#include "lds_dma.h"
#include "mxfp4_device.h"
#include "pact_internal.h"

namespace pact {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef int v8i_t __attribute__((ext_vector_type(8)));

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
//
// K is processed in stages of 128 (64 code bytes per row) held in a ring of
// four LDS buffers; the loads of stage kt + 4 are issued while stage kt is
// multiplied.  Scales travel in groups of G = 4 stages (16 bytes per row: one
// memory request per row per group instead of one per stage; 8 stages measured
// no faster): the group for stages Gg .. Gg + G - 1 is loaded together with
// the codes of stage Gg into one of two scale buffers.
// Fragments are double-buffered in registers: after the barrier that
// publishes stage kt + 1, a wave reads stage kt + 1's fragments and scales
// while it multiplies stage kt, one LDS read after each MFMA (a burst of reads
// stalls the wave's in-order issue behind a full LDS queue and starves the
// matrix core), so LDS latency is hidden behind a whole stage of MFMAs.
// ---------------------------------------------------------------------------
template <int WTM, int WTN>
struct MxCfg {
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 64 * WTN;
  static constexpr int ROWS = BM + BN;
  static constexpr int KS = 128;                        // K elements per stage
  static constexpr int NCODE = 4;                       // code stage buffers
  static constexpr int CODE_STAGE = ROWS * 64;          // [ROWS][64] swizzled by (row >> 2) & 3
#ifndef PACT_MX_SCALE_GROUP
#define PACT_MX_SCALE_GROUP 4
#endif
  static constexpr int G = PACT_MX_SCALE_GROUP;         // stages per scale group
  static constexpr int SC_ROW = 4 * G;                  // scale bytes per row and group
  static constexpr int SC_BYTES = ROWS * SC_ROW;        // [ROWS][SC_ROW]: G stages x 4 blocks
  static constexpr int SC_OFF = NCODE * CODE_STAGE;
  static constexpr int NC = ROWS / 64;                  // code loads per wave per stage (16 rows each)
  static constexpr int SC_LANES = SC_ROW / 16;          // lanes per row in a scale load
  static constexpr int NSG_TOTAL = SC_BYTES / 1024;     // scale loads per group (1 KB each)
  static constexpr int NSG = (NSG_TOTAL + 3) / 4;       // per wave; surplus ones fill a pad region
  static constexpr int PAD_OFF = SC_OFF + 2 * SC_BYTES;
  static constexpr int MAIN = PAD_OFF + (NSG * 4 - NSG_TOTAL) * 1024;
  static constexpr int EPI_LD = BN / 2 + 4;
  static constexpr int EPI_WAVE = 32 * EPI_LD * 4;
  static constexpr int TOTAL = MAIN > 4 * EPI_WAVE ? MAIN : 4 * EPI_WAVE;
  static_assert(ROWS % 64 == 0 && BM % 64 == 0, "tile rows");
  static_assert(2 * NC + NSG <= 63 && 3 * NC + NSG <= 63, "vmcnt range");
  static_assert(NC + NSG <= 2 * WTM * WTN, "one load per MFMA");
  static_assert(TOTAL <= 160 * 1024, "LDS");
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
  constexpr int BM = C::BM, BN = C::BN, NC = C::NC, NSG = C::NSG;
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
  // Code load c of this wave covers tile rows 16 (wave + 4c) .. +15: lane ->
  // row 16 (wave + 4c) + lane / 4, LDS slot lane % 4, global chunk
  // slot ^ ((row >> 2) & 3) = slot ^ ((lane >> 4) & 3).  Scale load c covers
  // 1 KB of the [ROWS][SC_ROW] group buffer: lane -> row
  // (64 / SC_LANES) (wave + 4c) + lane / SC_LANES, 16-byte part lane % SC_LANES.
  // Rows outside the operands get an offset past the buffer end: the range
  // check returns zeros.
  const int4v_t ra_c = buffer_rsrc(p.a_codes, (uint32_t)(M * crow));
  const int4v_t rb_c = buffer_rsrc(p.b_codes, (uint32_t)(N * crow));
  const int4v_t ra_s = buffer_rsrc(p.a_scales, (uint32_t)(M * srow));
  const int4v_t rb_s = buffer_rsrc(p.b_scales, (uint32_t)(N * srow));
  const uint32_t cchunk = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  uint32_t cvo[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
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
  uint32_t svo[NSG];
#pragma unroll
  for (int c = 0; c < NSG; ++c) {
    const int q = wave + 4 * c;
    const int row = (64 / C::SC_LANES) * q + lane / C::SC_LANES;
    const uint32_t part = (uint32_t)(lane % C::SC_LANES) * 16u;
    uint32_t v = 0xfffffff0u;
    if (q < C::NSG_TOTAL) {
      if (row < BM) {
        const int64_t m = m0 + row;
        if (m < M) v = (uint32_t)m * srow + part;
      } else {
        const int64_t n = n0 + (row - BM);
        if (n < N) v = (uint32_t)n * srow + part;
      }
    }
    svo[c] = v;
  }
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  // load q of stage s: codes for q < NC, then (first stage of a group only) scales
  auto issue_one = [&](int s, int q) {
    if (q < NC) {
      const uint32_t dst = lds0 + (uint32_t)((s & 3) * C::CODE_STAGE) + (uint32_t)(wave_s + 4 * q) * 1024u;
      const uint32_t soff = (uint32_t)s * 64u;
      if (16 * (4 * q + 3) + 15 < BM) lds_dma_buf16(ra_c, cvo[q], soff, dst);
      else lds_dma_buf16(rb_c, cvo[q], soff, dst);
    } else {
      const int c = q - NC;
      const int qq = wave_s + 4 * c;
      const int g = s / C::G;
      const uint32_t dst = qq < C::NSG_TOTAL
                               ? lds0 + (uint32_t)(C::SC_OFF + (g & 1) * C::SC_BYTES) + (uint32_t)qq * 1024u
                               : lds0 + (uint32_t)C::PAD_OFF + (uint32_t)(qq - C::NSG_TOTAL) * 1024u;
      const uint32_t soff = (uint32_t)g * (uint32_t)C::SC_ROW;
      constexpr int RPL = 64 / C::SC_LANES;                    // rows per scale load
      if (RPL * (4 * c + 3) + RPL - 1 < BM) lds_dma_buf16(ra_s, svo[c], soff, dst);
      else if (RPL * 4 * c >= BM) lds_dma_buf16(rb_s, svo[c], soff, dst);
      else if (qq * RPL < BM) lds_dma_buf16(ra_s, svo[c], soff, dst);   // split by wave: uniform branch
      else lds_dma_buf16(rb_s, svo[c], soff, dst);
    }
  };
  // number of loads issued for stage s (0 past the end)
  auto loads_of = [&](int s) { return (s >= 0 && s < nk) ? NC + ((s % C::G) == 0 ? NSG : 0) : 0; };
  // wait until at most n loads are outstanding (n is one of a few per-tile constants)
  auto wait_outstanding = [&](int n) {
    if (n >= 2 * NC + NSG) PACT_WAIT_VMCNT(2 * NC + NSG);
    else if (n >= 2 * NC) PACT_WAIT_VMCNT(2 * NC);
    else if (n >= NC + NSG) PACT_WAIT_VMCNT(NC + NSG);
    else if (n >= NC) PACT_WAIT_VMCNT(NC);
    else PACT_WAIT_VMCNT(0);
  };

  // ---- fragments (two register sets) ----
  // step s (0, 1) of a stage: lane (i, h) holds row i's K = 64 s + 32 h .. + 32
  // (16 bytes, chunk 2s + h of the row) and the scale of that block; the scale
  // dword of a row holds blocks 0..3 of the stage and is permuted so that
  // byte 0 / 1 are the blocks of steps 0 / 1 (op_sel picks the byte).
  uint4 fa[2][2][WTM], fb[2][2][WTN];
  uint32_t wa[2][WTM], wb[2][WTN];          // raw scale dwords (permuted when used)
  const uint32_t ssel = h ? 0x0c0c0301u : 0x0c0c0200u;
  // read item q (0 .. NREAD-1) of stage s into register set R: per A row tile
  // i the two code fragments and the scale dword, then the same per B tile j
  constexpr int NREAD = 3 * (WTM + WTN);
  auto read_item = [&](int s, auto set_tag, auto item_tag) {
    constexpr int R = decltype(set_tag)::value;
    constexpr int Q = decltype(item_tag)::value;
    constexpr bool IS_A = Q < 3 * WTM;
    constexpr int T = IS_A ? Q / 3 : (Q - 3 * WTM) / 3;       // tile index i or j
    constexpr int PART = Q % 3;                                 // 0, 1: code fragment of step PART; 2: scale
    const int row = IS_A ? wm * (BM / 2) + T * 32 + li : BM + wn * (BN / 2) + T * 32 + li;
    if constexpr (PART < 2) {
      const uint8_t* st = smem + (s & 3) * C::CODE_STAGE;
      const uint4 v = *reinterpret_cast<const uint4*>(st + row * 64 + (((2 * PART + h) ^ ((row >> 2) & 3)) << 4));
      if constexpr (IS_A) fa[R][PART][T] = v; else fb[R][PART][T] = v;
    } else {
      const uint8_t* sc = smem + C::SC_OFF + ((s / C::G) & 1) * C::SC_BYTES + (s % C::G) * 4;
      const uint32_t v = *reinterpret_cast<const uint32_t*>(sc + row * C::SC_ROW);
      if constexpr (IS_A) wa[R][T] = v; else wb[R][T] = v;
    }
  };
  auto read_stage = [&](int s, auto set_tag) {
    [&]<int... Q>(std::integer_sequence<int, Q...>) {
      (read_item(s, set_tag, std::integral_constant<int, Q>{}), ...);
    }(std::make_integer_sequence<int, NREAD>{});
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

  // Stage kt: wait for stage kt + 1's loads (issued three stages earlier) and
  // for this wave's reads of stage kt, barrier (stage kt + 1 published, buffer
  // kt % 4 free), read stage kt + 1 into the other register set, multiply
  // stage kt, and issue stage kt + 4's loads into buffer kt % 4, one per MFMA.
  // MODE 0 .. G-1: steady state with kt % G == MODE (every count is a
  // constant); MODE G: the last stages, with counts from kt.
  auto run_stage = [&](int kt, auto set_tag, auto mode_tag) {
    constexpr int R = decltype(set_tag)::value;
    constexpr int MODE = decltype(mode_tag)::value;
    if constexpr (MODE < C::G) {
      constexpr int W = 2 * NC + (((MODE + 2) % C::G == 0 || (MODE + 3) % C::G == 0) ? NSG : 0);
      PACT_WAIT_VMCNT(W);
    } else {
      wait_outstanding(loads_of(kt + 2) + loads_of(kt + 3));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);                    // lgkmcnt(0)
    __syncthreads();
    uint32_t sa[WTM], sb[WTN];
#pragma unroll
    for (int i = 0; i < WTM; ++i) sa[i] = __builtin_amdgcn_perm(wa[R][i], wa[R][i], ssel);
#pragma unroll
    for (int j = 0; j < WTN; ++j) sb[j] = __builtin_amdgcn_perm(wb[R][j], wb[R][j], ssel);
    // Stage kt's MFMAs with stage kt + 1's reads (past the last stage: stale,
    // in-bounds, unused) and stage kt + 4's loads spread between them: a burst
    // of LDS reads would stall the wave's in-order issue and starve the MFMAs.
    const int nload = MODE < C::G ? NC + ((MODE + 4) % C::G == 0 ? NSG : 0) : (kt + 4 < nk ? loads_of(kt + 4) : 0);
    constexpr int NMFMA = 2 * WTM * WTN;
    [&]<int... K>(std::integer_sequence<int, K...>) {
      ([&] {
        constexpr int k = K % (WTM * WTN), st = K / (WTM * WTN);
        constexpr int i = k / WTN, j = k % WTN;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(v8(fa[R][st][i]), v8(fb[R][st][j]), acc[i][j], 4, 4,
                                                                    st, (int)sa[i], st, (int)sb[j]);
        // read items r with r * NMFMA / NREAD == K follow MFMA K
        constexpr int r0 = (K * NREAD + NMFMA - 1) / NMFMA, r1 = ((K + 1) * NREAD + NMFMA - 1) / NMFMA;
        [&]<int... Rr>(std::integer_sequence<int, Rr...>) {
          (read_item(kt + 1, std::integral_constant<int, R ^ 1>{}, std::integral_constant<int, r0 + Rr>{}), ...);
        }(std::make_integer_sequence<int, r1 - r0>{});
        // loads spread evenly: load q follows MFMA q * NMFMA / (NC + NSG)
        constexpr int NL = NC + NSG;
        constexpr int l0 = (K * NL + NMFMA - 1) / NMFMA, l1 = ((K + 1) * NL + NMFMA - 1) / NMFMA;
        [&]<int... Ll>(std::integer_sequence<int, Ll...>) {
          ((l0 + Ll < nload ? issue_one(kt + 4, l0 + Ll) : void()), ...);
        }(std::make_integer_sequence<int, l1 - l0>{});
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // this MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);  // then its reads
      }(), ...);
    }(std::make_integer_sequence<int, NMFMA>{});
    __builtin_amdgcn_sched_barrier(0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // prologue: stages 0..3 (and scale group 0) in flight; wait for stage 0
  const int pre = nk < 4 ? nk : 4;
  for (int s = 0; s < pre; ++s) {
    const int nl = loads_of(s);
#pragma unroll
    for (int q = 0; q < NC + NSG; ++q)
      if (q < nl) issue_one(s, q);
  }
  if (pre >= 4) PACT_WAIT_VMCNT(3 * NC);      // stages 1..3 carry no scale group
  else if (pre == 3) PACT_WAIT_VMCNT(2 * NC);
  else if (pre == 2) PACT_WAIT_VMCNT(NC);
  else PACT_WAIT_VMCNT(0);
  __syncthreads();
  read_stage(0, I0{});
  int kt = 0;
  for (; kt + C::G + 4 <= nk; kt += C::G) {  // stages kt .. kt + G - 1 all issue loads
    [&]<int... U>(std::integer_sequence<int, U...>) {
      (run_stage(kt + U, std::integral_constant<int, U & 1>{}, std::integral_constant<int, U>{}), ...);
    }(std::make_integer_sequence<int, C::G>{});
  }
  for (; kt < nk; kt += 2) {                 // kt is even here
    run_stage(kt, I0{}, std::integral_constant<int, C::G>{});
    if (kt + 1 < nk) run_stage(kt + 1, I1{}, std::integral_constant<int, C::G>{});
  }
  PACT_WAIT_VMCNT(0);

  // ---- epilogue: optional accumulate, BF16 rounding, staged through LDS ----
  __syncthreads();
  float* epi = reinterpret_cast<float*>(smem + wave * C::EPI_WAVE);
  constexpr int WN = BN / 2;
  constexpr int CHUNKS = WN / 8;
  const bool vec_ok = (p.ldo % 8) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15u) == 0);
  // unchecked slab path (not in the 256 x 256 tile: there the compiler holds
  // every accumulator in VGPRs after the loop and the path's registers spill)
  const bool full = WTM * WTN < 16 && vec_ok && m0 + BM <= M && n0 + BN <= N;
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    uint16_t* const slab_out = p.out + (m0 + wm * (BM / 2) + i * 32) * p.ldo + n0 + wn * WN;
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = j * 32 + li;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * h + (rr & 3);
        epi[row * C::EPI_LD + col] = acc[i][j][rr];
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
