/*
 * pact_nvfp4.h -- C ABI of the NVFP4 frozen-projection library for MI355X (gfx950).
 *
 * The operations are those of PACT's LoRA linear layer and decoder MLP as its
 * precision-allocation table describes them ("PACT: NVFP4 Data-Flow LoRA
 * Fine-Tuning on Consumer GPUs", Appendix Table 7): frozen projections run as
 * NVFP4 GEMMs that sum in FP32 and write BF16, each direction over its own
 * cached NVFP4 copy of the weight; RMSNorm and SiLU-multiply are fused with
 * NVFP4 quantization and rebuild their inputs in FP32 for backward; the LoRA
 * branch runs in BF16 on the dequantized input.
 *
 * NVFP4 tensor (Appendix Table 6: 16-element blocks, E2M1 elements, E4M3
 * block scales, 4.50 bits/element).  A tensor of logical shape [rows x cols],
 * cols % 16 == 0, is three buffers, all row-major:
 *   codes  uint8 [rows][cols/2]   E2M1 codes, element 2j in the low nibble of byte j
 *   scales uint8 [rows][cols/16]  E4M3FN block scales (bias 7, max 448)
 *   rscale float [rows]           power-of-two FP32 row scale r = 2^e
 * Element (i, j) is  E2M1(code) * E4M3(scale[i][j/16]) * rscale[i].
 * Quantization rules: e is the smallest integer with rowmax <= 6*448*2^e,
 * clamped to [-126, 127] (0 for an all-zero row); block scale
 * s = RNE_E4M3(blockmax / (6 r)) saturating at 448; element code =
 * RNE(|x| / (s r)) onto {0,.5,1,1.5,2,3,4,6}, ties to the even code,
 * saturating at 6, sign bit of x kept, magnitude 0 when s == 0.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates, frees and synchronizes nothing; it launches asynchronously on
 *     `stream` (a hipStream_t; NULL is the default stream).
 *   - BF16 tensors are uint16_t bit patterns.
 *   - Arguments are validated on the host before any HIP call; a negative
 *     status is returned and pact_last_error() describes it.  Launch failures
 *     return PACT_EHIP.  Faults inside kernels surface at the caller's next
 *     synchronization.  No C++ exception crosses this interface.
 *   - rows == 0 (or M == 0) is a valid no-op.  Column counts that carry NVFP4
 *     blocks must be multiples of 16.  Every pointer that is dereferenced must
 *     be non-NULL and 16-byte aligned; leading dimensions are in elements.
 *   - NaN and Inf inputs are outside the contract.
 */
#ifndef PACT_NVFP4_H
#define PACT_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PACT_OK = 0,
  PACT_EINVAL = -1,      /* NULL pointer, negative size, bad flag */
  PACT_ESHAPE = -2,      /* cols % 16 != 0, ld < cols, rank out of range */
  PACT_EALIGN = -3,      /* pointer not 16-byte aligned */
  PACT_EHIP = -4,        /* a HIP launch failed */
  PACT_EUNSUPPORTED = -5 /* valid but unsupported by this library */
};

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *pact_last_error(void);

/* Interface version (incremented on any change of signature or semantics). */
int pact_abi_version(void);

/*
 * pact_selftest_arith -- device self-test of the arithmetic shortcuts inside
 * the kernels, each checked against the IEEE operation it stands for over
 * every input bit pattern of its range.  counts: device array of 5 unsigned
 * 64-bit integers (caller-owned), set to the number of disagreements of
 *   [0] the correctly rounded reciprocal (hardware estimate + one FMA
 *       correction), d in [2^-126, 2^126);
 *   [1] the correctly rounded division by 6 (reciprocal product + one FMA
 *       correction), every x in [6 * 2^-126, FLT_MAX] (a normal quotient;
 *       below it the block-scale code is 0 whatever the quotient's low bits);
 *   [2] the SiLU sigmoid 1/(1 + E(-a)) with that reciprocal (IEEE division
 *       past 1 + E >= 2^126), every non-NaN a;
 *   [3] the hardware float -> BF16 conversion against integer round to
 *       nearest even on the bit pattern, every non-NaN x;
 *   [4] the hardware FP8 conversions used for block scales in the row
 *       kernels against the software E4M3FN encoder (round to nearest even,
 *       every t in [0, 448]) and decoder (every code 0 .. 0x7E).
 * All five are 0 on a conforming device.  Asynchronous on `stream`; about
 * 1.4e10 evaluations (well under a second on one GPU).
 */
int pact_selftest_arith(unsigned long long *counts, void *stream);

/*
 * pact_mfma_probe -- measured MFMA-loop peak (a diagnostic beside the
 * published dense peaks; no part of the method).  Launches 512 workgroups of
 * 256 threads; every wave runs `iters` (1 .. 2^20) iterations of 16
 * independent accumulation chains of
 *   kind 0: v_mfma_f32_32x32x16_f16           (32768 FLOP each), or
 *   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands and unit
 *           scales (131072 FLOP each),
 * so one launch performs 512 * 4 * iters * 16 MFMAs.  sink: device float
 * array of at least 512 * 256 (written, to keep the work); clocks: device
 * array of at least 2 * 512 unsigned 64-bit values, set per workgroup to the
 * shader-clock cycles (s_memtime) and the 100 MHz constant-clock ticks
 * (s_memrealtime) between its start and end.  The caller times the launch
 * (e.g. with events on `stream`).  Errors: PACT_EINVAL for a bad kind, iters or
 * NULL pointer, PACT_ESHAPE for short buffers.
 */
int pact_mfma_probe(int kind, int iters, float *sink, int64_t sink_len, unsigned long long *clocks,
                    int64_t clocks_len, void *stream);

/* Host-only size query: bytes of the three buffers of an NVFP4 [rows x cols]. */
int pact_nvfp4_sizes(int64_t rows, int64_t cols, size_t *codes_bytes, size_t *scales_bytes,
                     size_t *rscale_bytes);

/*
 * nvfp4_quantize -- BF16 -> NVFP4 (Appendix Table 6 format; the abstract's
 * quantization step, Table 11 "Quantization / fused kernels").
 *   transpose == 0: x is [rows x cols] with leading dimension ldx >= cols; the
 *                   result is Q(x), blocks along cols.
 *   transpose == 1: x is [cols x rows] with leading dimension ldx >= rows; the
 *                   result is Q(x^T) of shape [rows x cols] (row i of the result
 *                   is column i of x).  This builds the cached backward weight
 *                   layout W_bwd = Q(W^T) from W [N x K] (rows = K, cols = N).
 *   Outputs: codes [rows][cols/2], scales [rows][cols/16], rscale [rows].
 */
int nvfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                   uint8_t *codes, uint8_t *scales, float *rscale, void *stream);

/*
 * nvfp4_quantize_ex -- nvfp4_quantize with the recipe variants (what the
 * tables leave open; the default, flags == 0, is nvfp4_quantize exactly):
 *   PACT_QUANT_ROUND_UP_SCALES: each block scale is the smallest E4M3 value
 *       >= blockmax / (6 r) instead of the nearest, so no element saturates
 *       (every |x| / (s r) <= 6).
 *   PACT_QUANT_TENSOR_SCALE: one power-of-two scale for the whole tensor, the
 *       row-scale rule applied to the tensor maximum *amax (every row's rscale
 *       is that value; rows with smaller maxima keep it).  amax: device float,
 *       4-byte aligned.  Without PACT_QUANT_COMPUTE_AMAX the caller supplies
 *       *amax (for example from the epilogue of the kernel that produced x); it
 *       must be >= max |x| or elements saturate.
 *   PACT_QUANT_COMPUTE_AMAX (with PACT_QUANT_TENSOR_SCALE): a first pass over x
 *       writes max |x| to *amax (two passes over x in all).
 *   PACT_QUANT_TENSOR_SCALE_FP32 (with PACT_QUANT_TENSOR_SCALE): the tensor
 *       scale is the conventional FP32 one instead of a power of two: every
 *       rscale is S = RN32(*amax / 2688) (at least 2^-126; 1 if *amax == 0),
 *       and each element is scaled by the FP32 product u = RN32(|x| * R),
 *       R = RN32(1 / S), before the block rules (s = RNE_E4M3(max u / 6),
 *       code = RNE_E2M1(u / s)).  *amax must be finite.  nvfp4_gemm_fwd
 *       and nvfp4_gemm_dgrad accept such tensors (results within the GEMM
 *       bound), with a fused LoRA term only through their _ex forms with
 *       PACT_GEMM_ANY_ROW_SCALES; nvfp4_gemm_dgrad_multi with two or more
 *       segments and nvfp4_gemm_dgrad_fwd_layout need power-of-two row scales
 *       (NaN output, and PACT_EUNSUPPORTED from pact_nvfp4_row_exp_max).
 * Other arguments and layouts as nvfp4_quantize.  Unknown flags: PACT_EINVAL.
 */
#define PACT_QUANT_ROUND_UP_SCALES 1
#define PACT_QUANT_TENSOR_SCALE 2
#define PACT_QUANT_COMPUTE_AMAX 4
#define PACT_QUANT_TENSOR_SCALE_FP32 8
int nvfp4_quantize_ex(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int transpose, int flags,
                      float *amax, uint8_t *codes, uint8_t *scales, float *rscale, void *stream);

/*
 * nvfp4_quantize_batch -- n (1..8) independent row-wise quantizations, as
 * nvfp4_quantize with transpose == 0, in one launch: the several output
 * gradients that one backward step quantizes at the same point for their
 * NVFP4 input-gradient GEMMs (Appendix Table 7 row "Frozen projections":
 * gradients quantized on the fly; in a decoder layer the attention gradients
 * of q, k and v).  Problem i: x[i] [rows[i] x cols[i]] with leading dimension
 * ldx[i] into codes[i], scales[i], rscale[i]; its outputs are bit-identical to
 * nvfp4_quantize of that problem alone.  The pointer and size arrays are host
 * arrays of n entries; every problem is validated as nvfp4_quantize (first
 * failure reported, nothing launched).  Problems of at most 3072 columns share
 * one launch; wider ones get launches of their own on the same stream.
 * Outputs must not overlap one another or any input.
 */
int nvfp4_quantize_batch(int n, const uint16_t *const *x, const int64_t *rows, const int64_t *cols,
                         const int64_t *ldx, uint8_t *const *codes, uint8_t *const *scales,
                         float *const *rscale, void *stream);

/*
 * rmsnorm_quant -- RMSNorm forward fused with NVFP4 quantization (Appendix
 * Table 7 row "RMSNorm": a BF16 row normalized in FP32; the NVFP4 result and
 * one FP32 statistic per token are saved for backward).  For each row of x [M x H] (leading dim ldx):
 *   S = sum x^2 (float64), ms = fp32(S/H), v = ms + eps, rstd = 1/sqrt(v),
 *   y = (x * rstd) * gain  (FP32, round-to-nearest, no contraction),
 * writes Q(y) (the projection input) and rstd [M].  gain is BF16 [H].
 * H % 16 == 0.
 */
int rmsnorm_quant(const uint16_t *x, const uint16_t *gain, float eps, int64_t M, int64_t H,
                  int64_t ldx, uint8_t *y_codes, uint8_t *y_scales, float *y_rscale, float *rstd,
                  void *stream);

/*
 * rmsnorm_quant_ex -- rmsnorm_quant with flags (0: rmsnorm_quant exactly).
 *   PACT_RMSNORM_EXACT_SUM: every row's sum of squares takes the double-double
 *   path.  rmsnorm_quant already switches a row to that path whenever its
 *   float64 sum lies within the sum's error bound of a float32 rounding
 *   boundary, so the results are identical; the flag exists so that tests can
 *   check the double-double path on every row.  Unknown flags: PACT_EINVAL.
 */
#define PACT_RMSNORM_EXACT_SUM 1
int rmsnorm_quant_ex(const uint16_t *x, const uint16_t *gain, float eps, int64_t M, int64_t H,
                     int64_t ldx, int flags, uint8_t *y_codes, uint8_t *y_scales, float *y_rscale,
                     float *rstd, void *stream);

/*
 * silu_mul_quant -- SiLU-multiply forward fused with NVFP4 quantization
 * (Appendix Table 7 row "SiLU-multiply": FP32 arithmetic on the BF16 gate and
 * up values; an NVFP4 copy of each of the two is saved for backward).  Elementwise on gate a, up b [M x I]
 * (shared leading dim ld):
 *   sigma = 1/(1 + E(-a)), h = (a * sigma) * b   (FP32; E is the library's
 *   Cody-Waite + degree-7 Taylor exponential, each reduction and Horner step
 *   one fused multiply-add),
 * writes Q(h) (the down-projection input), Q(a) and Q(b).  I % 16 == 0.
 */
int silu_mul_quant(const uint16_t *gate, const uint16_t *up, int64_t M, int64_t I, int64_t ld,
                   uint8_t *h_codes, uint8_t *h_scales, float *h_rscale,
                   uint8_t *g_codes, uint8_t *g_scales, float *g_rscale,
                   uint8_t *u_codes, uint8_t *u_scales, float *u_rscale, void *stream);

/*
 * pact_gemm_tile -- host-only query: the workgroup tile (bm x bn output
 * elements) that nvfp4_gemm_fwd / nvfp4_gemm_dgrad launch for an output of
 * M x Nout with contraction length Kr.  Lets callers attribute kernel times.
 */
int pact_gemm_tile(int64_t M, int64_t Nout, int64_t Kr, int *bm, int *bn);

/*
 * pact_gemm_multi_tile -- host-only query: the workgroup tile that
 * nvfp4_gemm_dgrad_multi launches for an output of M x Nout (the tile of
 * pact_gemm_tile, except that a 256 x 256 tile becomes 256 x 192: the
 * segmented kernel has no 256 x 256 instantiation).
 */
int pact_gemm_multi_tile(int64_t M, int64_t Nout, int *bm, int *bn);

/*
 * nvfp4_gemm_fwd -- frozen-projection forward Y = X W^T (Appendix Table 7 row
 * "Frozen projections": NVFP4 GEMM, FP32 accumulation, BF16 output).
 *   X_q: NVFP4 [M x K]; W_fwd: NVFP4 [N x K] (= Q(W), the cached forward layout).
 *   Y: BF16 [M x N], leading dim ldy >= N.
 *   Optional LoRA term (Table 7 row "LoRA branch"): if lora_t != NULL,
 *     Y = bf16( deq(X_q) deq(W_fwd)^T + lora_scale * T B^T )
 *   with T BF16 [M x r] (row-major, from lora_down) and B BF16 [N x r]
 *   (row-major), 1 <= r <= 128.  The sum is formed in FP32; one BF16 rounding.
 * K % 16 == 0.
 */
int nvfp4_gemm_fwd(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale,
                   int64_t M, int64_t K,
                   const uint8_t *w_codes, const uint8_t *w_scales, const float *w_rscale, int64_t N,
                   uint16_t *y, int64_t ldy,
                   const uint16_t *lora_t, const uint16_t *lora_b, int64_t lora_r, float lora_scale,
                   void *stream);

/*
 * nvfp4_gemm_fwd_ex / nvfp4_gemm_dgrad_ex -- nvfp4_gemm_fwd / nvfp4_gemm_dgrad
 * with flags (0: exactly the plain call).
 *   PACT_GEMM_ANY_ROW_SCALES: the operands' row scales may be any positive
 *     FP32 values, as the FP32 tensor-scale recipe (PACT_QUANT_TENSOR_SCALE_FP32)
 *     writes; the launch takes the register-staged kernel, whose LoRA term is
 *     scaled in FP32 after its BF16 MFMAs.  Without the flag the plain calls
 *     handle such operands too unless a LoRA term is fused: the
 *     direct-to-LDS kernel folds 1/r into the term's BF16 operands, which is
 *     exact only for powers of two, and writes NaN (at least to every output
 *     whose row or column scale is not a power of two) rather than a
 *     silently rounded result.
 * Unknown flags: PACT_EINVAL.
 */
#define PACT_GEMM_ANY_ROW_SCALES 1
int nvfp4_gemm_fwd_ex(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale,
                      int64_t M, int64_t K,
                      const uint8_t *w_codes, const uint8_t *w_scales, const float *w_rscale, int64_t N,
                      uint16_t *y, int64_t ldy,
                      const uint16_t *lora_t, const uint16_t *lora_b, int64_t lora_r, float lora_scale,
                      int flags, void *stream);
int nvfp4_gemm_dgrad_ex(const uint8_t *dy_codes, const uint8_t *dy_scales, const float *dy_rscale,
                        int64_t M, int64_t N,
                        const uint8_t *w_codes, const uint8_t *w_scales, const float *w_rscale, int64_t K,
                        uint16_t *dx, int64_t lddx, int accumulate,
                        const uint16_t *lora_dt, const uint16_t *lora_a, int64_t lora_r, int flags, void *stream);

/*
 * nvfp4_gemm_dgrad -- frozen-projection input gradient dX = dY W (Appendix
 * Table 7 row "Frozen projections": the input gradient is an NVFP4 GEMM over
 * the weight's cached backward copy).
 *   dY_q: NVFP4 [M x N]; W_bwd: NVFP4 [K x N] (= Q(W^T), blocks along N).
 *   dX: BF16 [M x K], leading dim lddx >= K.
 *   accumulate != 0: dX = bf16( f32(dX) + result )  (sums several consumers).
 *   Optional LoRA input-gradient term: if lora_dt != NULL,
 *     result += dT A  with dT BF16 [M x r] and A BF16 [r x K] (row-major),
 *   formed in FP32 before the one BF16 rounding.  1 <= r <= 128.
 * N % 16 == 0.
 */
int nvfp4_gemm_dgrad(const uint8_t *dy_codes, const uint8_t *dy_scales, const float *dy_rscale,
                     int64_t M, int64_t N,
                     const uint8_t *w_codes, const uint8_t *w_scales, const float *w_rscale, int64_t K,
                     uint16_t *dx, int64_t lddx, int accumulate,
                     const uint16_t *lora_dt, const uint16_t *lora_a, int64_t lora_r,
                     void *stream);

/*
 * nvfp4_gemm_dgrad_fwd_layout -- single-layout input gradient: dX = dY W over
 * the forward layout W_fwd = Q(W) [N x K] only (blocks along K), so a frozen
 * weight keeps one cached NVFP4 layout instead of two and the forward and
 * input-gradient products use identical effective weights.  (The pages keep
 * both layouts, Appendix Table 7 row "Frozen projections"; this is the
 * alternative that reuses W_fwd tiles through a transposed read.)
 *   dX = bf16( [f32(dX) +] deq(dY_q) deq(W_fwd) [+ dT A] ),
 *   dY_q NVFP4 [M x N]; W_fwd NVFP4 [N x K]; dX BF16 [M x K], ldx >= K;
 *   LoRA term and accumulate as nvfp4_gemm_dgrad.
 *   w_exp_max: device int, the largest row-scale exponent over W_fwd's
 *   nonzero rows (out[0] of pact_nvfp4_row_exp_max, once per weight).  Each B
 *   element is formed in FP16 as code * block scale * 2^(e_row - w_exp_max),
 *   exact while every nonzero row's exponent lies in [w_exp_max - 14,
 *   w_exp_max] (the weights pact_nvfp4_row_exp_max accepts).  If a nonzero row
 *   falls outside that window, or its row scale is not a power of two (the
 *   FP32 tensor-scale recipe), the launch cannot be exact: every output the
 *   affected workgroups own is written as NaN (in practice all of dX, since
 *   every workgroup contracts over all rows) rather than a rounded gradient.
 *   N % 256 == 0 and K % 64 == 0 (else PACT_EUNSUPPORTED), operands below
 *   2^31 bytes of codes.
 */
int nvfp4_gemm_dgrad_fwd_layout(const uint8_t *dy_codes, const uint8_t *dy_scales, const float *dy_rscale,
                                int64_t M, int64_t N,
                                const uint8_t *w_codes, const uint8_t *w_scales, const float *w_rscale,
                                const int *w_exp_max, int64_t K, uint16_t *dx, int64_t ldx, int accumulate,
                                const uint16_t *lora_dt, const uint16_t *lora_a, int64_t lora_r, void *stream);

/*
 * nvfp4_gemm_dgrad_multi -- input gradient summed over the projections that
 * read one input (Appendix Table 7 row "Frozen projections": q, k and v, or
 * gate and up, each contribute dY_i W_i to the same dX): one launch whose
 * contraction runs over nseg (1..4) segments,
 *   dX = bf16( [f32(dX) +] sum_i ( deq(dY_i) deq(W_bwd,i) + dT_i A_i ) ),
 * formed in FP32 with one BF16 rounding.  Segment i: dY_i NVFP4 [M x N_i]
 * (dy_codes[i], dy_scales[i], dy_rscale[i]), W_bwd,i NVFP4 [K x N_i], N_i =
 * seg_n[i] a positive multiple of 256 (else PACT_EUNSUPPORTED); optional LoRA
 * term dT_i BF16 [M x r_i] and A_i BF16 [r_i x K] (lora_dt may be NULL, or
 * lora_dt[i] NULL for a segment without one; 1 <= r_i <= 128).  The segment
 * arrays are host arrays of device pointers.  dX BF16 [M x K], lddx >= K.
 * Each segment keeps its own row scales: the partial sum is carried from one
 * segment's row-scale units to the next by an exact power-of-two rescale
 * (exact unless two segments' row exponents differ by more than about 90,
 * where the smaller contribution can leave the FP32 range).  With nseg >= 2
 * every row scale must be a power of two: operands from the FP32
 * tensor-scale recipe (PACT_QUANT_TENSOR_SCALE_FP32) make the launch write
 * NaN to the output tiles whose row scales it meets (use one nvfp4_gemm_dgrad
 * per segment with accumulate for them).  With nseg == 1 the result equals
 * nvfp4_gemm_dgrad's bit for bit.
 */
int nvfp4_gemm_dgrad_multi(int nseg, const uint8_t *const *dy_codes, const uint8_t *const *dy_scales,
                           const float *const *dy_rscale, const int64_t *seg_n,
                           const uint8_t *const *w_codes, const uint8_t *const *w_scales,
                           const float *const *w_rscale, int64_t M, int64_t K, uint16_t *dx, int64_t lddx,
                           int accumulate, const uint16_t *const *lora_dt, const uint16_t *const *lora_a,
                           const int64_t *lora_r, void *stream);

/*
 * pact_nvfp4_row_exp_max -- set-up of a weight for nvfp4_gemm_dgrad_fwd_layout,
 * once per weight.  Over the rows of an NVFP4 tensor [rows x cols] that are not
 * all zero, writes the largest exponent e of the power-of-two row scales 2^e to
 * out[0] and the smallest to out[1] (out: device array of 2 ints; -126 and 127
 * if every row is zero).  codes is validated but not read.  rows > 0,
 * cols % 16 == 0.  Unlike the other entry points this call synchronizes
 * `stream` (it reads the two exponents back) and returns PACT_EUNSUPPORTED when
 * out[0] - out[1] > 14: the single-layout dgrad forms each weight element in
 * FP16 relative to 2^out[0], which is exact only within that window (the
 * exponents are still written).  A nonzero row whose row scale is not a power
 * of two counts as exponent 255 (out[0] = 255) and also gives
 * PACT_EUNSUPPORTED.
 */
int pact_nvfp4_row_exp_max(const uint8_t *codes, const uint8_t *scales, const float *rscale, int64_t rows,
                           int64_t cols, int *out, void *stream);

/*
 * lora_down -- LoRA forward down-projection on the reconstructed input
 * (Appendix Table 7 row "LoRA branch": a BF16 product on the dequantized input).
 *   T = bf16( deq(X_q) A^T ),  X_q NVFP4 [M x K], A BF16 [r x K] row-major,
 *   T BF16 [M x r] row-major.  FP32 accumulation.  1 <= r <= 128, K % 16 == 0.
 */
int lora_down(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale,
              int64_t M, int64_t K, const uint16_t *A, int64_t r, uint16_t *T, void *stream);

/*
 * lora_bwd -- LoRA adapter gradients (Appendix Table 7 row "LoRA branch": BF16
 * adapter gradients and input gradients; saved state is the shared NVFP4 input
 * and the BF16 adapters, so T is recomputed).  With X~ = deq(X_q) [M x K],
 * A [r x K], B [N x r], the BF16 output gradient dY [M x N] (row-major) and
 * scale s:
 *   T  = bf16(X~ A^T)          (recomputed into the workspace)
 *   dT = bf16(s dY B)          [M x r]   (feeds nvfp4_gemm_dgrad's LoRA term)
 *   dB = bf16(s dY^T T)        [N x r]
 *   dA = bf16(dT^T X~)         [r x K]
 * The reductions over M are split across workgroups into FP32 partials in
 * `workspace` (device memory owned by the caller, at least
 * pact_lora_bwd_workspace_size() bytes, 256-byte aligned) and summed in a fixed
 * order, so results are deterministic.  Calls that share a workspace must not
 * overlap.  1 <= r <= 128; K % 16 == 0; N % 16 == 0.
 */
int pact_lora_bwd_workspace_size(int64_t M, int64_t K, int64_t N, int64_t r, size_t *bytes);

int lora_bwd(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale,
             int64_t M, int64_t K, const uint16_t *A, const uint16_t *B, int64_t r, float scale,
             const uint16_t *dy, int64_t N, uint16_t *dT, uint16_t *dA, uint16_t *dB,
             void *workspace, size_t workspace_bytes, void *stream);

/*
 * lora_bwd_dt / lora_bwd_ab -- lora_bwd in two calls, so that the input
 * gradient (which needs only dT, through nvfp4_gemm_dgrad's LoRA term) does
 * not wait for the adapter gradients (which nothing in the step reads before
 * the optimizer):
 *   lora_bwd_dt: dT = bf16(s dY B) [M x r] from dY [M x N] and B [N x r];
 *     no workspace.
 *   lora_bwd_ab: dB and dA as lora_bwd, given that dT (T recomputed from X_q
 *     and A); workspace as for lora_bwd (pact_lora_bwd_workspace_size).
 * Together they write exactly lora_bwd's dT, dA and dB, bit for bit.
 * Arguments and requirements as lora_bwd.
 */
int lora_bwd_dt(const uint16_t *dy, int64_t M, int64_t N, const uint16_t *B, int64_t r, float scale,
                uint16_t *dT, void *stream);
int lora_bwd_ab(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale, int64_t M, int64_t K,
                const uint16_t *A, int64_t r, float scale, const uint16_t *dy, int64_t N, const uint16_t *dT,
                uint16_t *dA, uint16_t *dB, void *workspace, size_t workspace_bytes, void *stream);

/*
 * lora_bwd_ab_batch -- the adapter gradients dA and dB of n (1..8) projections
 * in three launches (for example the projections of a decoder layer once
 * their dT is done), given T = X~ A^T (the LoRA branch of Appendix Table 7:
 * dB = s dY^T T, dA = dT^T X~).  T is lora_down's output: the branch keeps
 * only the shared NVFP4 input and the adapters for the backward, so a caller
 * recomputes it there, and one stacked lora_down serves every projection that
 * reads the same input.  Problem i
 * has X_q (x_codes[i], x_scales[i], x_rscale[i]) [M x K[i]], T[i] [M x r[i]]
 * with leading dimension ldT[i] >= r[i] (lora_down's output for the
 * projection's adapter: a column slice of a stacked lora_down's output is
 * fine), dY dy[i] [M x N[i]], dT[i] [M x r[i]] (lora_bwd_dt's output),
 * outputs dA[i] [r[i] x K[i]] and dB[i] [N[i] x r[i]], and its own workspace
 * (workspace[i], workspace_bytes[i] >= pact_lora_bwd_workspace_size(M, K[i],
 * N[i], r[i]), 256-byte aligned).  One token count M and one scale for all.
 * Every r[i] must be in the rank class of r[0] (1-16, 17-32, 33-64 or
 * 65-128), else PACT_EINVAL.  With T[i] = lora_down(X_q, A[i]) each
 * problem's dA and dB equal lora_bwd's bit for bit.  The arrays are host
 * arrays of device pointers (sizes on the host).
 */
int lora_bwd_ab_batch(int n, const uint8_t *const *x_codes, const uint8_t *const *x_scales,
                      const float *const *x_rscale, int64_t M, const int64_t *K, const uint16_t *const *T,
                      const int64_t *ldT, const int64_t *r, float scale, const uint16_t *const *dy,
                      const int64_t *N, const uint16_t *const *dT, uint16_t *const *dA, uint16_t *const *dB,
                      void *const *workspace, const size_t *workspace_bytes, void *stream);

/*
 * lora_bwd_noalloc -- lora_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same operation, arguments and results as lora_bwd (bit for
 * bit), without the workspace.  The library's own fixed scratch array of
 * 32 MiB per device (allocated when the library is loaded onto that device,
 * held until the process ends) takes its place; no call allocates or frees
 * memory.  PACT_EUNSUPPORTED when pact_lora_bwd_workspace_size(M, K, N, r)
 * exceeds 32 MiB (never for r <= 128 with M <= 16384 and K, N <= 16384).
 * Every call on a device shares that device's array: calls that overlap on one
 * GPU (other streams, other threads) race and must be serialized by the caller.
 */
int lora_bwd_noalloc(const uint8_t *x_codes, const uint8_t *x_scales, const float *x_rscale,
                     int64_t M, int64_t K, const uint16_t *A, const uint16_t *B, int64_t r, float scale,
                     const uint16_t *dy, int64_t N, uint16_t *dT, uint16_t *dA, uint16_t *dB, void *stream);

/*
 * silu_mul_bwd -- SiLU-multiply backward from the NVFP4 state (Appendix Table 7
 * row "SiLU-multiply", backward column: inputs rebuilt from the NVFP4 copies,
 * derivatives in FP32, BF16 results).
 *   a^ = deq(gate_q), b^ = deq(up_q), sigma = 1/(1 + E(-a^)) with E the
 *   pinned FP32 exponential of silu_mul_quant:
 *   dgate = bf16( ((dh b^) sigma) (1 + a^ (1 - sigma)) ),  dup = bf16( (dh a^) sigma ),
 *   every FP32 operation rounded to nearest in the order written (so the
 *   result is reproducible bit for bit).
 *   gate_q, up_q NVFP4 [M x I]; dh, dgate, dup BF16 [M x I] (dense rows).
 */
int silu_mul_bwd(const uint8_t *g_codes, const uint8_t *g_scales, const float *g_rscale,
                 const uint8_t *u_codes, const uint8_t *u_scales, const float *u_rscale,
                 const uint16_t *dh, int64_t M, int64_t I, uint16_t *dgate, uint16_t *dup,
                 void *stream);

/*
 * silu_mul_bwd_quant -- silu_mul_bwd that also emits the NVFP4 copies
 * dgate_q = Q(dgate), dup_q = Q(dup) of the BF16 gradients it stores (the
 * inputs of the gate and up input-gradient GEMMs; the BF16 gradients still
 * feed the LoRA backward).  Same results as silu_mul_bwd followed by two
 * nvfp4_quantize calls, with one pass over the data (quantize-on-emit).
 * dgate_q, dup_q NVFP4 [M x I] (caller buffers).  I % 16 == 0, I <= 16384.
 */
int silu_mul_bwd_quant(const uint8_t *g_codes, const uint8_t *g_scales, const float *g_rscale,
                       const uint8_t *u_codes, const uint8_t *u_scales, const float *u_rscale,
                       const uint16_t *dh, int64_t M, int64_t I, uint16_t *dgate, uint16_t *dup,
                       uint8_t *dg_codes, uint8_t *dg_scales, float *dg_rscale,
                       uint8_t *du_codes, uint8_t *du_scales, float *du_rscale, void *stream);

/*
 * rmsnorm_bwd -- RMSNorm backward from the NVFP4 state (Appendix Table 7 row
 * "RMSNorm", backward column: input rebuilt from the NVFP4 copy, FP32 row
 * reduction, BF16 result).
 *   y^ = deq(y_q) [M x H], rstd f32 [M], gain BF16 [H], dy BF16 [M x H]:
 *   S = sum_j dy_j y^_j exactly, rounded once to float64; mean = fp32(S / H)
 *   (float64 division);
 *   dx_i = bf16( rstd ((g_i dy_i) - ((y^_i / g_i) mean)) ), each FP32 operation
 *   rounded to nearest in the order written.
 *   dx BF16 [M x H] (dense rows).  The gain is frozen (no gain gradient).
 *   H % 16 == 0, H <= 16384.
 */
int rmsnorm_bwd(const uint8_t *y_codes, const uint8_t *y_scales, const float *y_rscale,
                const float *rstd, const uint16_t *gain, const uint16_t *dy, int64_t M, int64_t H,
                uint16_t *dx, void *stream);

/*
 * rmsnorm_bwd_residual -- rmsnorm_bwd fused with the residual-gradient
 * accumulation (Appendix Table 7 row "Residuals": residual gradients summed in BF16)
 * and, optionally, the NVFP4 quantization of the sum (quantize-on-emit: the
 * result is the output gradient of the projection that produced the residual
 * stream's previous value).
 *   out = bf16( fp32(bf16(dx)) + resid )   with dx as in rmsnorm_bwd;
 *   resid BF16 [M x H] or NULL (then out = bf16(dx));
 *   out_q = Q(out) NVFP4 [M x H] when q_codes, q_scales, q_rscale are all given
 *   (all NULL: no NVFP4 output).  out BF16 [M x H] must not alias dy or resid.
 */
int rmsnorm_bwd_residual(const uint8_t *y_codes, const uint8_t *y_scales, const float *y_rscale,
                         const float *rstd, const uint16_t *gain, const uint16_t *dy,
                         const uint16_t *resid, int64_t M, int64_t H, uint16_t *dx,
                         uint8_t *q_codes, uint8_t *q_scales, float *q_rscale, void *stream);

/* ---------------------------------------------------------------------------
 * MXFP4 variant (Appendix Table 6, MXFP4 column: 32-element blocks, E2M1
 * elements, E8M0 block scales, 4.25 bits/element, no other scale).  A tensor
 * of logical shape [rows x cols], cols % 32 == 0, is two row-major buffers:
 *   codes  uint8 [rows][cols/2]   E2M1 codes, element 2j in the low nibble of byte j
 *   scales uint8 [rows][cols/32]  E8M0 block scales: byte b is 2^(b - 127)
 * Element (i, j) is  E2M1(code) * 2^(scale[i][j/32] - 127).
 * Block scale (the tables give none; the OCP microscaling rule): shared
 * exponent e = floor(log2(blockmax)) - 2, clamped to [-127, 127], -127 for an
 * all-zero block, stored as e + 127; element code = RNE(|x| / 2^e) onto
 * {0,.5,1,1.5,2,3,4,6}, ties to the even code, saturating at 6, sign kept.
 * ------------------------------------------------------------------------- */

/* Host-only size query: bytes of the two buffers of an MXFP4 [rows x cols]. */
int pact_mxfp4_sizes(int64_t rows, int64_t cols, size_t *codes_bytes, size_t *scales_bytes);

/*
 * mxfp4_quantize -- BF16 -> MXFP4.
 *   transpose == 0: x is [rows x cols] with leading dimension ldx >= cols
 *                   (a multiple of 8); the result is Q(x), blocks along cols.
 *   transpose == 1: x is [cols x rows] with leading dimension ldx >= rows; the
 *                   result is Q(x^T) [rows x cols] (the backward weight layout
 *                   W_bwd = Q(W^T) from W [N x K] with rows = K, cols = N).
 *   cols % 32 == 0.  Outputs: codes [rows][cols/2], scales [rows][cols/32].
 */
int mxfp4_quantize(const uint16_t *x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                   uint8_t *codes, uint8_t *scales, void *stream);

/*
 * mxfp4_rmsnorm_quant -- rmsnorm_quant with an MXFP4 output (Appendix Table 7
 * row "RMSNorm" with the Table 6 MXFP4 format): the same FP32 sequence
 *   S = sum x^2 (float64), ms = fp32(S/H), v = ms + eps, rstd = 1/sqrt(v),
 *   y = (x * rstd) * gain,
 * then y_q = MXFP4(y) [M x H] (codes, E8M0 scales) and rstd [M].  H % 32 == 0,
 * H <= 16384; ldx >= H, a multiple of 8.
 */
int mxfp4_rmsnorm_quant(const uint16_t *x, const uint16_t *gain, float eps, int64_t M, int64_t H, int64_t ldx,
                        uint8_t *y_codes, uint8_t *y_scales, float *rstd, void *stream);

/*
 * mxfp4_silu_mul_quant -- silu_mul_quant with MXFP4 outputs (Appendix Table 7
 * row "SiLU-multiply" with the Table 6 MXFP4 format): h = (a * sigma) * b in
 * the same FP32 sequence, outputs MXFP4(h), MXFP4(a), MXFP4(b) [M x I].
 * I % 32 == 0, I <= 16384; gate and up share the leading dimension ld.
 */
int mxfp4_silu_mul_quant(const uint16_t *gate, const uint16_t *up, int64_t M, int64_t I, int64_t ld,
                         uint8_t *h_codes, uint8_t *h_scales, uint8_t *g_codes, uint8_t *g_scales,
                         uint8_t *u_codes, uint8_t *u_scales, void *stream);

/*
 * mxfp4_silu_mul_bwd_quant -- silu_mul_bwd_quant from an MXFP4 state with
 * MXFP4 copies (Appendix Table 7 row "SiLU-multiply", backward column, with
 * the Table 6 MXFP4 format): a^ = deq(gate_q), b^ = deq(up_q) (MXFP4
 * [M x I]), the same pinned FP32 sequence as silu_mul_bwd for the BF16 dgate,
 * dup [M x I] (dense rows), and dgate_q = MXFP4(dgate), dup_q = MXFP4(dup).
 * I % 32 == 0, I <= 16384.
 */
int mxfp4_silu_mul_bwd_quant(const uint8_t *g_codes, const uint8_t *g_scales, const uint8_t *u_codes,
                             const uint8_t *u_scales, const uint16_t *dh, int64_t M, int64_t I, uint16_t *dgate,
                             uint16_t *dup, uint8_t *dg_codes, uint8_t *dg_scales, uint8_t *du_codes,
                             uint8_t *du_scales, void *stream);

/*
 * mxfp4_rmsnorm_bwd_residual -- rmsnorm_bwd_residual from an MXFP4 state
 * (Appendix Table 7 rows "RMSNorm" and "Residuals", backward column, with the
 * Table 6 MXFP4 format): y^ = deq(y_q) (MXFP4 [M x H]), the same FP32 sequence
 * as rmsnorm_bwd, out = bf16(fp32(bf16(dx)) + resid) (resid may be NULL),
 * and, when q_codes and q_scales are given, out_q = MXFP4(out).
 * H % 32 == 0, H <= 16384.
 */
int mxfp4_rmsnorm_bwd_residual(const uint8_t *y_codes, const uint8_t *y_scales, const float *rstd,
                               const uint16_t *gain, const uint16_t *dy, const uint16_t *resid, int64_t M, int64_t H,
                               uint16_t *dx, uint8_t *q_codes, uint8_t *q_scales, void *stream);

/*
 * mxfp4_gemm -- C = A B^T for MXFP4 A [M x K] and B [N x K] (forward: X_q and
 * W_fwd = Q(W); input gradient: dY_q [M x N] and W_bwd = Q(W^T) [K x N]), on
 * the scaled FP4 matrix instructions with FP32 accumulation (Appendix Table 7
 * row "Frozen projections", with the Table 6 MXFP4 format in place of NVFP4).
 *   C BF16 [M x N], leading dim ldc >= N; accumulate != 0: C = bf16(f32(C) + A B^T).
 *   K % 128 == 0; A and B hold fewer than 2^31 bytes of codes each.
 */
int mxfp4_gemm(const uint8_t *a_codes, const uint8_t *a_scales, int64_t M, int64_t K,
               const uint8_t *b_codes, const uint8_t *b_scales, int64_t N, uint16_t *c, int64_t ldc,
               int accumulate, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PACT_NVFP4_H */
