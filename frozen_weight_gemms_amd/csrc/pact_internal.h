// Internal launch interface between the C ABI layer (abi.hip) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4_device.h"

namespace pact {

hipError_t launch_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                           uint8_t* codes, uint8_t* scales, float* rscale, hipStream_t s);

// n <= kQuantBatch row-wise quantizations (default recipe) in one launch;
// problems wider than 3072 columns get launches of their own
constexpr int kQuantBatch = 8;
struct QuantBatch {
  const uint16_t* x[kQuantBatch];
  int64_t rows[kQuantBatch], cols[kQuantBatch], ldx[kQuantBatch];
  uint8_t* codes[kQuantBatch];
  uint8_t* scales[kQuantBatch];
  float* rscale[kQuantBatch];
  int64_t wg_end[kQuantBatch];   // workgroups of problems 0 .. i
  int nb[kQuantBatch];           // 16-element blocks per lane (1..3)
  int n;
};
hipError_t launch_quantize_batch(int n, const uint16_t* const* x, const int64_t* rows, const int64_t* cols,
                                 const int64_t* ldx, uint8_t* const* codes, uint8_t* const* scales,
                                 float* const* rscale, hipStream_t s);

// round_up: block scales rounded up (non-saturating); tensor_amax (device, may be
// null): one power-of-two scale for the whole tensor from that maximum
hipError_t launch_quantize_ex(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                              int qmode, const float* tensor_amax, uint8_t* codes, uint8_t* scales,
                              float* rscale, hipStream_t s);   // qmode: bit 0 round-up scales, bit 1 FP32 tensor scale
// *amax = max |x| over x [rows x cols] (row stride ldx)
hipError_t launch_selftest_arith(unsigned long long* counts, hipStream_t s);
constexpr int kMfmaProbeGroups = 512;      // workgroups of the MFMA-rate probe
hipError_t launch_mfma_probe(int kind, int iters, float* sink, unsigned long long* clocks, hipStream_t s);
hipError_t launch_tensor_absmax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, float* amax,
                                hipStream_t s);

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t H,
                                int64_t ldx, uint8_t* codes, uint8_t* scales, float* rscale, float* rstd,
                                int force_exact, int mx, hipStream_t s);   // mx: MXFP4 output (rscale unused)

hipError_t launch_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t I, int64_t ld,
                                 uint8_t* hc, uint8_t* hs, float* hr, uint8_t* gc, uint8_t* gs, float* gr,
                                 uint8_t* uc, uint8_t* us, float* ur, int mx, hipStream_t s);

// C[M x N] = A[M x K] B[N x K]^T for row-blocked NVFP4 A and B, BF16 output.
struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_rscale;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_rscale;
  int64_t M, N, K;
  uint16_t* out;
  int64_t ldo;
  int accumulate;
  // optional rank-r term: acc += lora_scale * sum_j T[m][j] * U(j, n)
  const uint16_t* lora_t;   // [M x r], leading dim lora_r
  const uint16_t* lora_u;   // U(j, n) = lora_u[j * u_stride_j + n * u_stride_n]
  int64_t u_stride_j, u_stride_n;
  int64_t lora_r;
  float lora_scale;
  int general;              // 1: row scales may be any positive FP32 (register-staged kernel)
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// Contraction over up to kMaxSeg segments (see launch_gemm_multi): segment i
// has its own operands [M x K_i] and [N x K_i] with row scales and its own
// optional rank-r term (lora_t [M x lora_r], lora_u with GemmArgs' strides).
constexpr int kMaxSeg = 4;
struct SegOperand {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const float* a_rscale;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* b_rscale;
  int64_t K;
  const uint16_t* lora_t;
  const uint16_t* lora_u;
  int64_t lora_r;
};
struct SegArgs {
  int nseg;
  SegOperand s[kMaxSeg];
};
bool gemm_multi_supported(const GemmArgs& a, const SegArgs& sg);
hipError_t launch_gemm_multi(const GemmArgs& a, const SegArgs& sg, hipStream_t s);
void gemm_tile(int64_t M, int64_t N, int* bm, int* bn);
void gemm_multi_tile(int64_t M, int64_t N, int* bm, int* bn);

// Single-layout input gradient: dX [M x K] = deq(dY_q [M x N]) deq(W_fwd [N x K]);
// bexp = largest row exponent over W_fwd's nonzero rows (device int, from launch_row_exp_max)
bool dgrad_fwdlayout_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_dgrad_fwdlayout(const uint8_t* ac, const uint8_t* as, const float* ar, int64_t M, int64_t N,
                                  const uint8_t* bc, const uint8_t* bs, const float* br, const int* bexp, int64_t K,
                                  uint16_t* out, int64_t ldo, int accumulate, const uint16_t* lora_dt,
                                  const uint16_t* lora_a, int64_t r, hipStream_t s);
hipError_t launch_row_exp_max(const float* rscale, const uint8_t* scales, int64_t rows, int64_t cols, int* out,
                              hipStream_t s);

hipError_t launch_lora_down(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                            const uint16_t* A, int64_t r, uint16_t* T, hipStream_t s);

size_t lora_bwd_workspace(int64_t M, int64_t K, int64_t N, int64_t r);

// fixed per-device scratch of lora_bwd_noalloc (a device array; its address on
// the current device is looked up once per device)
constexpr size_t kLoraScratchBytes = (size_t)32 << 20;
// problems per batched adapter-gradient launch (lora_bwd_ab_batch)
constexpr int kLoraBatch = 8;
// dA and dB of n <= kLoraBatch problems given T and dT; problem i: X_q
// (xc[i], xs[i], xr[i]) [M x K[i]], T[i] [M x r[i]] with leading dimension
// ldT[i], dY dy[i] [M x N[i]], dT[i] [M x r[i]], outputs dA[i], dB[i], its own
// workspace ws[i] (at least lora_bwd_workspace(M, K[i], N[i], r[i]) bytes).
// Every r[i] in one rank class.
hipError_t launch_lora_bwd_ab_batch(int n, const uint8_t* const* xc, const uint8_t* const* xs,
                                    const float* const* xr, int64_t M, const int64_t* K,
                                    const uint16_t* const* T, const int64_t* ldT, const int64_t* r, float scale,
                                    const uint16_t* const* dy, const int64_t* N, const uint16_t* const* dT,
                                    uint16_t* const* dA, uint16_t* const* dB, void* const* ws, hipStream_t s);
bool lora_same_rank_class(int64_t r0, int64_t r1);
hipError_t lora_scratch_address(void** out);

hipError_t launch_lora_bwd(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                           const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                           int64_t N, uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, hipStream_t s);
// dT = bf16(scale dY B) alone (the row kernel's dT part)
hipError_t launch_lora_bwd_dt(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* B, int64_t r, float scale,
                              uint16_t* dT, hipStream_t s);
// dA and dB given dT (lora_bwd_dt's output): the rest of launch_lora_bwd
hipError_t launch_lora_bwd_ab(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                              const uint16_t* A, int64_t r, float scale, const uint16_t* dy, int64_t N,
                              const uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, hipStream_t s);
hipError_t launch_lora_bwd_impl(const uint8_t* xc, const uint8_t* xs, const float* xr, int64_t M, int64_t K,
                                const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy,
                                int64_t N, uint16_t* dT, const uint16_t* dT_in, uint16_t* dA, uint16_t* dB,
                                void* workspace, hipStream_t s);

hipError_t launch_silu_mul_bwd(const uint8_t* gc, const uint8_t* gs, const float* gr, const uint8_t* uc,
                               const uint8_t* us, const float* ur, const uint16_t* dh, int64_t M, int64_t I,
                               uint16_t* dgate, uint16_t* dup, hipStream_t s);

hipError_t launch_silu_mul_bwd_quant(const uint8_t* gc, const uint8_t* gs, const float* gr, const uint8_t* uc,
                                     const uint8_t* us, const float* ur, const uint16_t* dh, int64_t M, int64_t I,
                                     uint16_t* dgate, uint16_t* dup, uint8_t* qgc, uint8_t* qgs, float* qgr,
                                     uint8_t* quc, uint8_t* qus, float* qur, int mx, hipStream_t s);

// dx = bf16(rmsnorm backward) [+ resid, rounded again to BF16]; qc == nullptr: no copy.
// mx: y_q and the copy are MXFP4 (yr, qr unused)
hipError_t launch_rmsnorm_bwd(const uint8_t* yc, const uint8_t* ys, const float* yr, const float* rstd,
                              const uint16_t* gain, const uint16_t* dy, int64_t M, int64_t H,
                              const uint16_t* resid, uint16_t* dx, uint8_t* qc, uint8_t* qs, float* qr, int mx,
                              hipStream_t s);

hipError_t launch_mx_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
bool mx_gemm_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_mx_gemm(const uint8_t* ac, const uint8_t* as, int64_t M, int64_t K, const uint8_t* bc,
                          const uint8_t* bs, int64_t N, uint16_t* out, int64_t ldo, int accumulate, hipStream_t s);

}  // namespace pact
