// Input-gradient GEMM over the forward weight layout only (single-layout
// dgrad): dX = dY_q . deq(W_fwd), W_fwd = Q(W) [N x K] blocked along K, so the
// frozen weight needs one cached NVFP4 layout instead of two and the forward
// and input-gradient products use identical effective weights.  (PACT keeps
// two cached NVFP4 copies of each weight, one per direction, Appendix Table 7
// row "Frozen projections"; this variant instead reuses the W_fwd tiles
// through a transposed read, so each weight keeps one layout.)
//
// The contraction runs over N, the row axis of W_fwd.  Per stage of 256
// contraction rows the workgroup stages, for its 128 output columns, the
// W_fwd codes [256 n][64 B] (16-byte chunks XOR-swizzled by (n >> 2) & 3), the
// raw E4M3 block scales [256 n][8] and the row scales [256 n] straight into
// LDS.  ds_read_b64_tr_b4 transposes 16 rows x 16 nibbles per 16 lanes, so a
// lane receives, for one output column, 16 consecutive contraction elements:
// the MFMA B fragment for two K steps.  Every one of those elements has its
// own scale (its row's block scale times its row scale), so each stage also
// builds an FP16 table T[kb][n] = e4m3(s[n][kb]) * 2^(e_n - e_ref) in LDS, and
// the dequantization multiplies code pairs by table pairs (4 conversions and
// 4 packed multiplies per 8 elements, as for A).  e_ref is the largest row
// exponent over W_fwd's nonzero rows (a per-weight constant computed once);
// the epilogue multiplies by 2^e_ref.  A B element c * s * 2^(e_n - e_ref) is exact
// in FP16 while e_ref - e_n <= 14 (c s is a multiple of 2^-10 with at most 6
// significant bits).  A row with nonzero block scales outside that window
// (more than 2^14 below e_ref, or above it: an e_ref that is not this
// weight's), or whose row scale is not a power of two, would round or vanish
// in FP16; the table build flags it and the
// workgroup then writes NaN to every output it owns instead of a silently
// wrong gradient (pact_nvfp4_row_exp_max rejects such a weight up front).
//
// The A side (dY_q, blocked along N), the stage pipeline (two LDS stages of
// 256, loads issued one stage ahead, one barrier per stage plus one after the
// table build), the XCD-aware tile order and the epilogue follow the
// dual-layout kernel.
#include <type_traits>

#include "epilogue.h"
#include "lds_dma.h"
#include "mfma_fp16.h"
#include "pact_internal.h"

namespace pact {

constexpr int FL_KT = 256;                         // contraction elements per stage

template <int WTM>
struct FlCfg {
  static constexpr int WTN = 2;                    // 128 output columns
  static constexpr int BM = 64 * WTM;
  static constexpr int BN = 128;
  static constexpr int A_CODES = 0;                // [BM][128] swizzled by (row >> 1) & 7
  static constexpr int A_SC = BM * 128;            // [BM][16] raw E4M3 (room for 256 rows: surplus
                                                   // loads of a 128-row tile write zeros there)
  static constexpr int B_CODES = A_SC + (BM > 256 ? BM : 256) * 16;   // [256][64] swizzled by (n >> 2) & 3
  static constexpr int B_SC = B_CODES + 256 * 64;  // [256][8] raw E4M3
  static constexpr int B_R = B_SC + 256 * 8;       // [256] f32 row scales
  static constexpr int STAGE = B_R + 256 * 4;
  static constexpr int TAB = 2 * STAGE;            // 2 x [8 kb][256 n] FP16
  static constexpr int TAB_BYTES = 8 * 256 * 2;
  static constexpr int RSC = TAB + 2 * TAB_BYTES;  // A row scales [BM] f32
  static constexpr int EPI_LD = BN / 2 + 4;
  static constexpr int EPI_WAVE = 32 * EPI_LD * 4;
  static constexpr int MAIN = RSC + BM * 4;
  static constexpr int TOTAL = MAIN > 4 * EPI_WAVE ? MAIN : 4 * EPI_WAVE;
  static constexpr int NCA = BM / 32;              // A code loads per wave per stage (8 rows x 128 B each)
  static constexpr int NSA = BM / 256 > 0 ? BM / 256 : 1;   // A scale loads per wave (64 rows x 16 B each)
  static constexpr int NSA_TOTAL = BM / 64;
  static constexpr int NCB = 4;                    // B code loads per wave (16 rows x 64 B each)
  static constexpr int NSB = 2;                    // B scale loads per wave (32 rows x 8 B, 4 B per lane)
  static constexpr int NRB = 1;                    // B row-scale loads per wave (64 rows)
  static constexpr int LOADS = NCA + NSA + NCB + NSB + NRB;
  static_assert(TOTAL <= 160 * 1024, "LDS");
  static_assert(NSA * 4 >= NSA_TOTAL, "A scale loads");
};

struct FlArgs {
  const uint8_t* a_codes;       // dY_q [M x N]
  const uint8_t* a_scales;
  const float* a_rscale;
  const uint8_t* b_codes;       // W_fwd [N x K]
  const uint8_t* b_scales;
  const float* b_rscale;
  const int* b_exp_ref;         // largest row exponent of W_fwd (device)
  int64_t M, N, K;              // output [M x K], contraction over N
  uint16_t* out;
  int64_t ldo;
  int accumulate;
  const uint16_t* lora_t;       // optional dT [M x r]
  const uint16_t* lora_a;       // A [r x K]
  int64_t lora_r;
};

template <int WTM>
__global__ __launch_bounds__(256, 1) void k_gemm_dgrad_fwdlayout(FlArgs p, int tiles_m, int tiles_n) {
  using C = FlCfg<WTM>;
  constexpr int BM = C::BM, BN = C::BN, WTN = C::WTN;
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
  const int64_t m0 = (int64_t)tile_m * BM, k0 = (int64_t)tile_n * BN;

  const int64_t M = p.M, N = p.N, K = p.K;
  const uint32_t arow = (uint32_t)(N >> 1), asrow = (uint32_t)(N >> 4);     // dY_q row strides (bytes)
  const uint32_t brow = (uint32_t)(K >> 1), bsrow = (uint32_t)(K >> 4);     // W_fwd row strides (bytes)
  const int nk = (int)(N / FL_KT);
  const int e_ref = *p.b_exp_ref;

  // ---- load addressing (rows past an operand end read zeros) ----
  const int4v_t ra_c = buffer_rsrc(p.a_codes, (uint32_t)(M * arow));
  const int4v_t ra_s = buffer_rsrc(p.a_scales, (uint32_t)(M * asrow));
  const int4v_t rb_c = buffer_rsrc(p.b_codes, (uint32_t)(N * brow));
  const int4v_t rb_s = buffer_rsrc(p.b_scales, (uint32_t)(N * bsrow));
  const int4v_t rb_r = buffer_rsrc(p.b_rscale, (uint32_t)(N * 4));
  // A codes: load c of this wave covers tile rows 8 (wave + 4c) + lane / 8, LDS slot lane % 8
  const int arow0 = 8 * wave + (lane >> 3);
  const uint32_t achunk = (uint32_t)(((lane & 7) ^ ((arow0 >> 1) & 7)) << 4);
  uint32_t avo[C::NCA];
#pragma unroll
  for (int c = 0; c < C::NCA; ++c) {
    const int64_t m = m0 + arow0 + 32 * c;
    avo[c] = m < M ? (uint32_t)m * arow + achunk : 0xfffffff0u;
  }
  uint32_t asvo[C::NSA];
#pragma unroll
  for (int c = 0; c < C::NSA; ++c) {
    const int q = wave + 4 * c;
    const int64_t m = m0 + 64 * q + lane;
    asvo[c] = (q < C::NSA_TOTAL && m < M) ? (uint32_t)m * asrow : 0xfffffff0u;
  }
  // B codes: load c covers stage rows 16 (wave + 4c) + lane / 4, LDS slot lane % 4 <- chunk
  // slot ^ ((n >> 2) & 3) = slot ^ ((lane >> 4) & 3); 64 bytes of columns k0 .. k0 + 127
  const uint32_t bchunk = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  // per-stage offsets are n * brow: the row term is added per stage (rows past N fail the range check)
  auto b_code_voff = [&](int kt, int c) -> uint32_t {
    const int64_t n = (int64_t)kt * FL_KT + 16 * (wave + 4 * c) + (lane >> 2);
    return n < N ? (uint32_t)n * brow + (uint32_t)(k0 >> 1) + bchunk : 0xfffffff0u;
  };
  auto b_sc_voff = [&](int kt, int c) -> uint32_t {
    const int64_t n = (int64_t)kt * FL_KT + 32 * (wave + 4 * c) + (lane >> 1);
    return n < N ? (uint32_t)n * bsrow + (uint32_t)(k0 >> 4) + 4u * (uint32_t)(lane & 1) : 0xfffffff0u;
  };
  auto b_r_voff = [&](int kt) -> uint32_t {
    const int64_t n = (int64_t)kt * FL_KT + 64 * wave + lane;
    return n < N ? (uint32_t)n * 4u : 0xfffffff0u;
  };
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t lds0 = lds_addr(smem);
  auto issue_one = [&](int kt, int buf, int q) {
    const uint32_t st = lds0 + (uint32_t)(buf * C::STAGE);
    if (q < C::NCA) {
      lds_dma_buf16(ra_c, avo[q], (uint32_t)kt * 128u, st + C::A_CODES + (uint32_t)(wave_s + 4 * q) * 1024u);
    } else if (q < C::NCA + C::NSA) {
      const int c = q - C::NCA;
      const int qq = wave_s + 4 * c;                   // qq >= NSA_TOTAL: zeros into unused rows (uniform count)
      lds_dma_buf16(ra_s, asvo[c], (uint32_t)kt * 16u, st + C::A_SC + (uint32_t)qq * 1024u);
    } else if (q < C::NCA + C::NSA + C::NCB) {
      const int c = q - C::NCA - C::NSA;
      lds_dma_buf16(rb_c, b_code_voff(kt, c), 0u, st + C::B_CODES + (uint32_t)(wave_s + 4 * c) * 1024u);
    } else if (q < C::NCA + C::NSA + C::NCB + C::NSB) {
      const int c = q - C::NCA - C::NSA - C::NCB;
      lds_dma_buf4(rb_s, b_sc_voff(kt, c), 0u, st + C::B_SC + (uint32_t)(wave_s + 4 * c) * 256u);
    } else {
      lds_dma_buf4(rb_r, b_r_voff(kt), 0u, st + C::B_R + (uint32_t)wave_s * 256u);
    }
  };
  auto issue_stage = [&](int kt, int buf) {
#pragma unroll
    for (int q = 0; q < C::LOADS; ++q) issue_one(kt, buf, q);
  };

  // ---- FP16 scale table of a stage: thread t handles contraction row t ----
  uint32_t inexact_row = 0;                              // a nonzero row outside the exact FP16 window
  auto build_table = [&](int buf, bool real_stage) {
    const uint8_t* st = smem + buf * C::STAGE;
    const uint2 raw = *reinterpret_cast<const uint2*>(st + C::B_SC + tid * 8);
    const uint32_t rb = __float_as_uint(*reinterpret_cast<const float*>(st + C::B_R + tid * 4));
    const int e_n = (int)((rb >> 23) & 0xFFu) - 127;     // r is a power of two (0 for rows past N)
    const int d = e_ref - e_n;
    // 2^-d in FP16, exact for 0 <= d <= 24; d > 24: below FP16 (0); d < 0 only
    // for all-zero rows (excluded from e_ref), whose block scales are 0 anyway.
    // Exactness of every c s 2^-d needs 0 <= d <= 14 on rows with a nonzero scale.
    // (only for a real stage: past the last one the buffer holds stale bytes)
    // A row scale that is not a power of two (the FP32 tensor-scale recipe)
    // cannot be folded into the table exactly at all.
    inexact_row |= (real_stage && (d > 14 || d < 0 || (rb & 0x7FFFFFu) != 0u) && (raw.x | raw.y) != 0u) ? 1u : 0u;
    const _Float16 mult = (d >= 0 && d <= 24) ? (_Float16)__uint_as_float((uint32_t)(127 - d) << 23)
                                               : (_Float16)0.0f;
    const half2_t m2 = {mult, mult};
    _Float16* tab = reinterpret_cast<_Float16*>(smem + C::TAB + buf * C::TAB_BYTES);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const uint32_t word = w ? raw.y : raw.x;
      const half2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false) * m2;
      const half2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true) * m2;
      tab[(4 * w + 0) * 256 + tid] = lo[0];
      tab[(4 * w + 1) * 256 + tid] = lo[1];
      tab[(4 * w + 2) * 256 + tid] = hi[0];
      tab[(4 * w + 3) * 256 + tid] = hi[1];
    }
  };

  // ---- fragments ----
  uint4 ca[WTM][2], cb[WTN][2];
  uint2 sra[WTM], sra_n[WTM];
  half2_t sa[WTM][2];
  uint4 tb[WTN][2][4];                              // B scale table pairs per chunk (4 steps x 8 FP16)
  // A: codes chunk c (K steps 4c .. 4c + 3) into slot c & 1 (as the dual-layout kernel)
  auto read_a = [&](const uint8_t* st, int c) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int row = wm * (BM / 2) + i * 32 + li;
      ca[i][c & 1] = *reinterpret_cast<const uint4*>(st + C::A_CODES + row * 128 + (((4 * h + c) ^ ((row >> 1) & 7)) << 4));
    }
  };
  auto read_a_scales = [&](const uint8_t* st, uint2* out) {
#pragma unroll
    for (int i = 0; i < WTM; ++i)
      out[i] = *reinterpret_cast<const uint2*>(st + C::A_SC + (wm * (BM / 2) + i * 32 + li) * 16 + 8 * h);
  };
  // B: chunk c = transposed reads q = 2c, 2c + 1.  Lane (g = lane / 16, i = lane % 16) points at
  // contraction row 128 (g / 2) + 16 q + i, byte (k0' + 16 (g % 2)) / 2 of its 64-byte row.
  const int g16 = lane >> 4, i16 = lane & 15;
  auto read_b = [&](const uint8_t* st, int c) {
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int kcol = wn * (BN / 2) + j * 32 + 16 * (g16 & 1);     // first column of the 16-lane group
      const int lb = kcol >> 1;                                     // logical byte in the row
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int q = 2 * c + t;
        const int n = 128 * (g16 >> 1) + 16 * q + i16;
        const int phys = n * 64 + ((((lb >> 4) ^ ((n >> 2) & 3))) << 4) + (lb & 15);
        typedef int v2i_t __attribute__((ext_vector_type(2)));
        const v2i_t v = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
            (__attribute__((address_space(3))) v2i_t*)(lds0 + (uint32_t)(st - smem) + (uint32_t)(C::B_CODES + phys)));
        w[2 * t] = (uint32_t)v.x;
        w[2 * t + 1] = (uint32_t)v.y;
      }
      cb[j][c & 1] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  };
  // B scales for chunk c: table[kb][128 h + 8 s .. + 8] for s = 4c .. 4c + 3
  auto read_b_scales = [&](int tbuf, int c) {
    const uint8_t* tab = smem + C::TAB + tbuf * C::TAB_BYTES;
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int kb = (wn * (BN / 2) + j * 32 + li) >> 4;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        tb[j][c & 1][u] = *reinterpret_cast<const uint4*>(tab + (kb * 256 + 128 * h + 8 * (4 * c + u)) * 2);
    }
  };
  auto pair = [](uint32_t w, bool hi) {
    return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true)
              : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  };
  auto cvt_a_scales = [&](int c) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) sa[i][c & 1] = pair((c >> 1) ? sra[i].y : sra[i].x, (c & 1) != 0);
  };
  half8_t af[2][WTM], bfr[2][WTN];
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
      const uint4 sp = tb[j][c & 1][s & 3];
      const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * __builtin_bit_cast(half2_t, sp.x);
      const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * __builtin_bit_cast(half2_t, sp.y);
      const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * __builtin_bit_cast(half2_t, sp.z);
      const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * __builtin_bit_cast(half2_t, sp.w);
      half8_t r;
      r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
      r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
      b_out[j] = r;
    }
  };

  floatx16 acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  constexpr int DMA_SP = (3 * WTM * WTN) / C::LOADS > 0 ? (3 * WTM * WTN) / C::LOADS : 1;
  auto mfma_step = [&](int s, int dma_kt, int dma_buf, bool dma) {
#pragma unroll
    for (int k = 0; k < WTM * WTN; ++k) {
      const int i = k / WTN, j = k % WTN;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[s & 1][i], bfr[s & 1][j], acc[i][j], 0, 0, 0);
      const int g = (s - 12) * WTM * WTN + k;
      if (dma && s >= 12 && g % DMA_SP == 0 && g / DMA_SP < C::LOADS) issue_one(dma_kt, dma_buf, g / DMA_SP);
    }
    if (dma && s == 14) {
#pragma unroll
      for (int q = (3 * WTM * WTN + DMA_SP - 1) / DMA_SP; q < C::LOADS; ++q) issue_one(dma_kt, dma_buf, q);
    }
  };

  // Stage kt lives in LDS buffer kt % 2 (table buffer kt % 2).  Its loads are
  // issued during steps 12-14 of stage kt - 2 and published by the barrier at
  // step 12 of stage kt - 1; the table of stage kt + 1 is built right after
  // that barrier and published by a second one at step 14, before step 15
  // dequantizes stage kt + 1's first step.
  auto run_stage = [&](int kt, auto dma_tag) {
    constexpr bool DMA = decltype(dma_tag)::value;
    const uint8_t* st = smem + (kt & 1) * C::STAGE;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      __builtin_amdgcn_sched_barrier(0);
      if (c < 3) {
        read_a(st, c + 1);
        read_b(st, c + 1);
        read_b_scales(kt & 1, c + 1);
      } else {
        PACT_WAIT_VMCNT(0);
        __syncthreads();                                // stage kt + 1 published (stale past the end)
        const uint8_t* stn = smem + ((kt + 1) & 1) * C::STAGE;
        build_table((kt + 1) & 1, kt + 1 < nk);
        read_a(stn, 0);
        read_b(stn, 0);
        read_a_scales(stn, sra_n);
      }
#pragma unroll
      for (int s = 4 * c; s < 4 * c + 4; ++s) {
        __builtin_amdgcn_sched_barrier(0);
        if (s == 14) {
          __syncthreads();                              // table of stage kt + 1 complete
          read_b_scales((kt + 1) & 1, 0);
        }
        if (s == 15) {
#pragma unroll
          for (int i = 0; i < WTM; ++i) sra[i] = sra_n[i];
          cvt_a_scales(0);
          deq_step(0, af[0], bfr[0]);
        } else {
          if (((s + 1) & 3) == 0) cvt_a_scales((s + 1) >> 2);
          deq_step(s + 1, af[(s + 1) & 1], bfr[(s + 1) & 1]);
        }
        mfma_step(s, kt + 2, kt & 1, DMA);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- prologue: A row scales into LDS, stages 0 and 1 in flight ----
  float* rsc = reinterpret_cast<float*>(smem + C::RSC);
  {
    const int4v_t ra_r = buffer_rsrc(p.a_rscale, (uint32_t)(M * 4));
    for (int q = wave_s; q < BM / 64; q += 4) {
      const int64_t m = m0 + 64 * q + lane;
      lds_dma_buf4(ra_r, m < M ? (uint32_t)m * 4u : 0xfffffff0u, 0u, lds0 + (uint32_t)C::RSC + (uint32_t)q * 256u);
    }
  }
  issue_stage(0, 0);
  if (nk > 1) issue_stage(1, 1);

  // LoRA input-gradient term dT . A, formed into the accumulators and
  // prescaled by 1 / (r_A 2^e_ref) so that the epilogue's scaling restores it
  if (p.lora_t != nullptr) {
    const int64_t r = p.lora_r;
    // dT rows as 16-byte runs of 8 ranks where aligned; otherwise (and for A,
    // whose 8 ranks of one column are K apart) every element is loaded from a
    // clamped, valid index and selected afterwards.  A conditional load
    // compiles to a branch, and the wait after each one serialized them
    // (12 us of prologue per tile).
    const bool t_vec = (r & 15) == 0 && (reinterpret_cast<uintptr_t>(p.lora_t) & 15u) == 0;
    for (int64_t j0 = 0; j0 < r; j0 += 16) {
      bf16x8_t tf[WTM], uf[WTN];
      if (t_vec) {
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
          int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
          m = m < M ? m : M - 1;
          tf[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(p.lora_t + m * r + j0 + 8 * h));
        }
      } else {
        uint16_t e[WTM][8];
#pragma unroll
        for (int i = 0; i < WTM; ++i) {
          int64_t m = m0 + wm * (BM / 2) + i * 32 + li;
          m = m < M ? m : M - 1;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int64_t j = j0 + 8 * h + t;
            e[i][t] = p.lora_t[m * r + (j < r ? j : r - 1)];
          }
        }
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
          for (int t = 0; t < 8; ++t) tf[i][t] = bf16_of(j0 + 8 * h + t < r ? e[i][t] : (uint16_t)0);
      }
      uint16_t ea[WTN][8];
#pragma unroll
      for (int jj = 0; jj < WTN; ++jj) {
        int64_t k = k0 + wn * (BN / 2) + jj * 32 + li;
        k = k < K ? k : K - 1;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t j = j0 + 8 * h + t;
          ea[jj][t] = p.lora_a[(j < r ? j : r - 1) * K + k];
        }
      }
#pragma unroll
      for (int jj = 0; jj < WTN; ++jj)
#pragma unroll
        for (int t = 0; t < 8; ++t) uf[jj][t] = bf16_of(j0 + 8 * h + t < r ? ea[jj][t] : (uint16_t)0);
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int jj = 0; jj < WTN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf[i], uf[jj], acc[i][jj], 0, 0, 0);
    }
  }
  // stage 0 (and the row scales) complete and visible
  if (nk > 1) PACT_WAIT_VMCNT(C::LOADS);
  else PACT_WAIT_VMCNT(0);
  __syncthreads();
  const float inv_ref = __uint_as_float((uint32_t)(127 - e_ref) << 23);   // 2^-e_ref (e_ref in [-126, 127])
  if (p.lora_t != nullptr) {
    // 1/r_A: exact on the exponent for a power of two, else a rounded quotient
    // (one FP32 rounding of the term, which the epilogue's r_A multiply undoes
    // up to that rounding)
    auto inv_r = [](float v) {
      return (__float_as_uint(v) & 0x7FFFFFu) == 0u ? __uint_as_float((254u << 23) - __float_as_uint(v)) : 1.0f / v;
    };
#pragma unroll
    for (int i = 0; i < WTM; ++i)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = wm * (BM / 2) + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3);
        const float fa = inv_r(rsc[row]) * inv_ref;
#pragma unroll
        for (int j = 0; j < WTN; ++j) acc[i][j][rr] *= fa;
      }
  }
  build_table(0, true);
  read_a(smem, 0);
  read_b(smem, 0);
  read_a_scales(smem, sra);
  __syncthreads();                                       // table of stage 0 complete
  read_b_scales(0, 0);
  cvt_a_scales(0);
  deq_step(0, af[0], bfr[0]);
  int kt = 0;
  for (; kt + 2 < nk; ++kt) run_stage(kt, std::true_type{});
  for (; kt < nk; ++kt) run_stage(kt, std::false_type{});
  PACT_WAIT_VMCNT(0);

  // ---- epilogue: r_A[m] 2^e_ref, optional accumulate, BF16 rounding ----
  // the threads together saw every stage's table rows: OR the flag over the
  // workgroup (a ballot per wave, one LDS word per wave)
  __shared__ uint32_t inexact_wave[4];
  const bool wave_inexact = __ballot(inexact_row != 0u) != 0ull;
  if (lane == 0) inexact_wave[wave] = wave_inexact ? 1u : 0u;
  __syncthreads();
  const bool poison = (inexact_wave[0] | inexact_wave[1] | inexact_wave[2] | inexact_wave[3]) != 0u;
  const float ref = poison ? __uint_as_float(0x7FC00000u) : __uint_as_float((uint32_t)(e_ref + 127) << 23);
  float* epi = reinterpret_cast<float*>(smem + wave * C::EPI_WAVE);
  constexpr int WN = BN / 2;
  constexpr int CHUNKS = WN / 8;
  const bool vec_ok = (p.ldo % 8) == 0 && ((reinterpret_cast<uintptr_t>(p.out) & 15u) == 0);
  float ra_row[WTM][4][4];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr)
      ra_row[i][rr >> 2][rr & 3] = rsc[wm * (BM / 2) + i * 32 + 8 * (rr >> 2) + 4 * h + (rr & 3)] * ref;
  __syncthreads();                                       // row scales read before the slabs overwrite them
  const bool full = vec_ok && m0 + BM <= M && k0 + BN <= K;   // unchecked slab path
#pragma unroll
  for (int i = 0; i < WTM; ++i) {
    uint16_t* const slab_out = p.out + (m0 + wm * (BM / 2) + i * 32) * p.ldo + k0 + wn * WN;
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = j * 32 + li;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int row = 8 * (rr >> 2) + 4 * h + (rr & 3);
        epi[row * C::EPI_LD + col] = acc[i][j][rr] * ra_row[i][rr >> 2][rr & 3];
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
      const int64_t k = k0 + wn * WN + ch * 8;
      if (m >= M || k >= K) continue;
      const float* src = epi + row * C::EPI_LD + ch * 8;
      float v[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) v[t] = src[t];
      uint16_t* dst = p.out + m * p.ldo + k;
      if (vec_ok && k + 8 <= K) {
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
        for (int t = 0; t < 8 && k + t < K; ++t) {
          float x = v[t];
          if (p.accumulate) x += __uint_as_float((uint32_t)dst[t] << 16);
          dst[t] = (uint16_t)f32_to_bf16_rne(x);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Largest and smallest row exponent over the rows of an NVFP4 tensor that are
// not all zero (an all-zero row has row scale 1 by the row rule, which must
// not set the reference).  Each wave tests one row at a time (any nonzero block
// scale); one atomic pair per workgroup combines the extremes (initial values
// -126 and 127).
__global__ void k_init_exp(int* out) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    out[0] = -126;
    out[1] = 127;
  }
}
__global__ __launch_bounds__(256) void k_row_exp_range(const float* __restrict__ rscale,
                                                       const uint8_t* __restrict__ scales, int64_t rows,
                                                       int64_t nblk, int* __restrict__ out) {
  __shared__ int red[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int hi = -126, lo = 127;
  for (int64_t i = (int64_t)blockIdx.x * 4 + wave; i < rows; i += (int64_t)gridDim.x * 4) {
    uint32_t any = 0;
    for (int64_t b = lane; b < nblk; b += 64) any |= scales[i * nblk + b];
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) any |= (uint32_t)__shfl_xor((int)any, o, 64);
    if (any != 0) {
      const uint32_t u = __float_as_uint(rscale[i]);
      // a row scale that is not a power of two reports the out-of-range
      // exponent 255, which fails the caller's window check
      const int e = (u & 0x7FFFFFu) != 0u ? 255 : (int)((u >> 23) & 0xFFu) - 127;
      hi = e > hi ? e : hi;
      lo = e < lo ? e : lo;
    }
  }
  if (lane == 0) {
    red[0][wave] = hi;
    red[1][wave] = lo;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int h = red[0][0], l = red[1][0];
    for (int k = 1; k < 4; ++k) {
      h = red[0][k] > h ? red[0][k] : h;
      l = red[1][k] < l ? red[1][k] : l;
    }
    atomicMax(out, h);
    atomicMin(out + 1, l);
  }
}

hipError_t launch_row_exp_max(const float* rscale, const uint8_t* scales, int64_t rows, int64_t cols, int* out,
                              hipStream_t s) {
  k_init_exp<<<1, 64, 0, s>>>(out);
  int64_t grid = (rows + 3) / 4;
  if (grid > 256) grid = 256;
  k_row_exp_range<<<(unsigned)grid, 256, 0, s>>>(rscale, scales, rows, cols / 16, out);
  return hipGetLastError();
}

bool dgrad_fwdlayout_supported(int64_t M, int64_t N, int64_t K) {
  return N % FL_KT == 0 && K % 64 == 0 && (uint64_t)N * (uint64_t)(K / 2) < (1ull << 31) &&
         (uint64_t)M * (uint64_t)(N / 2) < (1ull << 31);
}

hipError_t launch_dgrad_fwdlayout(const uint8_t* ac, const uint8_t* as, const float* ar, int64_t M, int64_t N,
                                  const uint8_t* bc, const uint8_t* bs, const float* br, const int* bexp, int64_t K,
                                  uint16_t* out, int64_t ldo, int accumulate, const uint16_t* lora_dt,
                                  const uint16_t* lora_a, int64_t r, hipStream_t s) {
  FlArgs a{ac, as, ar, bc, bs, br, bexp, M, N, K, out, ldo, accumulate, lora_dt, lora_a, r};
  const int tn = (int)((K + 127) / 128);
  const int tm256 = (int)((M + 255) / 256);
  if ((int64_t)tm256 * tn >= 256) {
    k_gemm_dgrad_fwdlayout<4><<<tm256 * tn, 256, 0, s>>>(a, tm256, tn);
  } else {
    const int tm = (int)((M + 127) / 128);
    k_gemm_dgrad_fwdlayout<2><<<tm * tn, 256, 0, s>>>(a, tm, tn);
  }
  return hipGetLastError();
}

}  // namespace pact
