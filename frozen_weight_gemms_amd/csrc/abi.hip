// C ABI of the NVFP4 frozen-projection library: argument validation (on the
// host, before any HIP call) and dispatch to the kernel launchers.  The
// contract of every entry point is stated in include/pact_nvfp4.h.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "pact_internal.h"
#include "pact_nvfp4.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return PACT_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PACT_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, code, ...) \
  do {                           \
    if (!(cond)) return fail(code, __VA_ARGS__); \
  } while (0)

#define REQUIRE_PTR(p, name)                                                   \
  do {                                                                         \
    if ((p) == nullptr) return fail(PACT_EINVAL, "%s is NULL", name);          \
    if (!aligned16(p)) return fail(PACT_EALIGN, "%s is not 16-byte aligned", name); \
  } while (0)

constexpr int64_t kMaxFusedCols = 16384;
constexpr int64_t kMaxRank = 128;

int check_nvfp4(const uint8_t* c, const uint8_t* s, const float* r, const char* name) {
  char buf[64];
  snprintf(buf, sizeof(buf), "%s codes", name);
  if (c == nullptr) return fail(PACT_EINVAL, "%s is NULL", buf);
  if (!aligned16(c)) return fail(PACT_EALIGN, "%s is not 16-byte aligned", buf);
  snprintf(buf, sizeof(buf), "%s scales", name);
  if (s == nullptr) return fail(PACT_EINVAL, "%s is NULL", buf);
  if (!aligned16(s)) return fail(PACT_EALIGN, "%s is not 16-byte aligned", buf);
  snprintf(buf, sizeof(buf), "%s rscale", name);
  if (r == nullptr) return fail(PACT_EINVAL, "%s is NULL", buf);
  if (!aligned16(r)) return fail(PACT_EALIGN, "%s is not 16-byte aligned", buf);
  return PACT_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

const char* pact_last_error(void) { return g_err; }

int pact_abi_version(void) { return 15; }

int pact_nvfp4_sizes(int64_t rows, int64_t cols, size_t* codes_bytes, size_t* scales_bytes, size_t* rscale_bytes) {
  REQUIRE(rows >= 0 && cols >= 0, PACT_EINVAL, "negative size (rows=%lld, cols=%lld)", (long long)rows,
          (long long)cols);
  REQUIRE(cols % 16 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  REQUIRE(codes_bytes && scales_bytes && rscale_bytes, PACT_EINVAL, "NULL output pointer");
  *codes_bytes = (size_t)(rows * (cols / 2));
  *scales_bytes = (size_t)(rows * (cols / 16));
  *rscale_bytes = (size_t)rows * sizeof(float);
  return ok();
}

int pact_gemm_tile(int64_t M, int64_t Nout, int64_t Kr, int* bm, int* bn) {
  REQUIRE(M >= 0 && Nout >= 0 && Kr >= 0, PACT_EINVAL, "negative size");
  REQUIRE(bm != nullptr && bn != nullptr, PACT_EINVAL, "NULL output pointer");
  pact::gemm_tile(M, Nout, bm, bn);
  return ok();
}

int pact_gemm_multi_tile(int64_t M, int64_t Nout, int* bm, int* bn) {
  REQUIRE(M >= 0 && Nout >= 0, PACT_EINVAL, "negative size");
  REQUIRE(bm != nullptr && bn != nullptr, PACT_EINVAL, "NULL output pointer");
  pact::gemm_multi_tile(M, Nout, bm, bn);
  return ok();
}

int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose, uint8_t* codes,
                   uint8_t* scales, float* rscale, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, PACT_EINVAL, "negative size (rows=%lld, cols=%lld)", (long long)rows,
          (long long)cols);
  REQUIRE(transpose == 0 || transpose == 1, PACT_EINVAL, "transpose must be 0 or 1 (got %d)", transpose);
  REQUIRE(cols % 16 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  if (rows == 0) return ok();
  REQUIRE_PTR(x, "x");
  int st = check_nvfp4(codes, scales, rscale, "out");
  if (st != PACT_OK) return st;
  if (transpose == 0) {
    REQUIRE(ldx >= cols, PACT_ESHAPE, "ldx=%lld < cols=%lld", (long long)ldx, (long long)cols);
    REQUIRE(ldx % 8 == 0, PACT_EALIGN, "ldx=%lld is not a multiple of 8 elements", (long long)ldx);
  } else {
    REQUIRE(ldx >= rows, PACT_ESHAPE, "ldx=%lld < rows=%lld (transposed input is [cols x rows])", (long long)ldx,
            (long long)rows);
  }
  REQUIRE(rows <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "rows=%lld exceeds the grid limit", (long long)rows);
  return hip_status(pact::launch_quantize(x, rows, cols, ldx, transpose, codes, scales, rscale, as_stream(stream)),
                    "nvfp4_quantize launch");
}

int nvfp4_quantize_batch(int n, const uint16_t* const* x, const int64_t* rows, const int64_t* cols,
                         const int64_t* ldx, uint8_t* const* codes, uint8_t* const* scales, float* const* rscale,
                         void* stream) {
  REQUIRE(n >= 1 && n <= pact::kQuantBatch, PACT_EINVAL, "n=%d outside [1, %d]", n, pact::kQuantBatch);
  REQUIRE(x && rows && cols && ldx && codes && scales && rscale, PACT_EINVAL, "a problem array is NULL");
  for (int i = 0; i < n; ++i) {
    REQUIRE(rows[i] >= 0 && cols[i] >= 0, PACT_EINVAL, "problem %d: negative size (rows=%lld, cols=%lld)", i,
            (long long)rows[i], (long long)cols[i]);
    REQUIRE(cols[i] % 16 == 0, PACT_ESHAPE, "problem %d: cols=%lld is not a multiple of 16", i,
            (long long)cols[i]);
    if (rows[i] == 0) continue;
    if (x[i] == nullptr) return fail(PACT_EINVAL, "problem %d: x is NULL", i);
    if (!aligned16(x[i])) return fail(PACT_EALIGN, "problem %d: x is not 16-byte aligned", i);
    int st = check_nvfp4(codes[i], scales[i], rscale[i], "out");
    if (st != PACT_OK) return st;
    REQUIRE(ldx[i] >= cols[i], PACT_ESHAPE, "problem %d: ldx=%lld < cols=%lld", i, (long long)ldx[i],
            (long long)cols[i]);
    REQUIRE(ldx[i] % 8 == 0, PACT_EALIGN, "problem %d: ldx=%lld is not a multiple of 8 elements", i,
            (long long)ldx[i]);
    REQUIRE(rows[i] <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "problem %d: rows=%lld exceeds the grid limit", i,
            (long long)rows[i]);
  }
  int64_t wgs = 0;
  for (int i = 0; i < n; ++i) wgs += (rows[i] + 3) / 4;
  REQUIRE(wgs <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "%lld workgroups exceed the grid limit", (long long)wgs);
  return hip_status(pact::launch_quantize_batch(n, x, rows, cols, ldx, codes, scales, rscale, as_stream(stream)),
                    "nvfp4_quantize_batch launch");
}

int nvfp4_quantize_ex(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose, int flags,
                      float* amax, uint8_t* codes, uint8_t* scales, float* rscale, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, PACT_EINVAL, "negative size (rows=%lld, cols=%lld)", (long long)rows,
          (long long)cols);
  REQUIRE(transpose == 0 || transpose == 1, PACT_EINVAL, "transpose must be 0 or 1 (got %d)", transpose);
  REQUIRE((flags & ~(PACT_QUANT_ROUND_UP_SCALES | PACT_QUANT_TENSOR_SCALE | PACT_QUANT_COMPUTE_AMAX |
                     PACT_QUANT_TENSOR_SCALE_FP32)) == 0,
          PACT_EINVAL, "unknown flags 0x%x", flags);
  REQUIRE(!(flags & PACT_QUANT_COMPUTE_AMAX) || (flags & PACT_QUANT_TENSOR_SCALE), PACT_EINVAL,
          "PACT_QUANT_COMPUTE_AMAX needs PACT_QUANT_TENSOR_SCALE");
  REQUIRE(!(flags & PACT_QUANT_TENSOR_SCALE_FP32) || (flags & PACT_QUANT_TENSOR_SCALE), PACT_EINVAL,
          "PACT_QUANT_TENSOR_SCALE_FP32 needs PACT_QUANT_TENSOR_SCALE");
  REQUIRE(cols % 16 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  const bool tensor = (flags & PACT_QUANT_TENSOR_SCALE) != 0;
  if (tensor) {
    REQUIRE(amax != nullptr, PACT_EINVAL, "amax is NULL (required by PACT_QUANT_TENSOR_SCALE)");
    REQUIRE((reinterpret_cast<uintptr_t>(amax) & 3u) == 0, PACT_EALIGN, "amax is not 4-byte aligned");
  }
  if (rows == 0 || cols == 0) return ok();
  REQUIRE_PTR(x, "x");
  int st = check_nvfp4(codes, scales, rscale, "out");
  if (st != PACT_OK) return st;
  if (transpose == 0) {
    REQUIRE(ldx >= cols, PACT_ESHAPE, "ldx=%lld < cols=%lld", (long long)ldx, (long long)cols);
    REQUIRE(ldx % 8 == 0, PACT_EALIGN, "ldx=%lld is not a multiple of 8 elements", (long long)ldx);
  } else {
    REQUIRE(ldx >= rows, PACT_ESHAPE, "ldx=%lld < rows=%lld (transposed input is [cols x rows])", (long long)ldx,
            (long long)rows);
  }
  REQUIRE(rows <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "rows=%lld exceeds the grid limit", (long long)rows);
  hipStream_t s = as_stream(stream);
  if (flags & PACT_QUANT_COMPUTE_AMAX) {
    // the input buffer is [rows x cols] (transpose 0) or [cols x rows] (transpose 1)
    const int64_t xr = transpose ? cols : rows, xc = transpose ? rows : cols;
    st = hip_status(pact::launch_tensor_absmax(x, xr, xc, ldx, amax, s), "tensor amax launch");
    if (st != PACT_OK) return st;
  }
  return hip_status(pact::launch_quantize_ex(x, rows, cols, ldx, transpose,
                                             ((flags & PACT_QUANT_ROUND_UP_SCALES) ? 1 : 0) |
                                                 ((flags & PACT_QUANT_TENSOR_SCALE_FP32) ? 2 : 0),
                                             tensor ? amax : nullptr,
                                             codes, scales, rscale, s),
                    "nvfp4_quantize_ex launch");
}

int rmsnorm_quant_ex(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t H, int64_t ldx,
                     int flags, uint8_t* y_codes, uint8_t* y_scales, float* y_rscale, float* rstd, void* stream) {
  REQUIRE((flags & ~PACT_RMSNORM_EXACT_SUM) == 0, PACT_EINVAL, "unknown flags 0x%x", flags);
  REQUIRE(M >= 0 && H >= 0, PACT_EINVAL, "negative size (M=%lld, H=%lld)", (long long)M, (long long)H);
  REQUIRE(H % 16 == 0, PACT_ESHAPE, "H=%lld is not a multiple of 16", (long long)H);
  REQUIRE(H <= kMaxFusedCols, PACT_EUNSUPPORTED, "H=%lld exceeds %lld", (long long)H, (long long)kMaxFusedCols);
  REQUIRE(eps >= 0.0f, PACT_EINVAL, "eps must be non-negative");
  if (M == 0) return ok();
  REQUIRE(H > 0, PACT_ESHAPE, "H must be positive");
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(gain, "gain");
  REQUIRE_PTR(rstd, "rstd");
  int st = check_nvfp4(y_codes, y_scales, y_rscale, "y");
  if (st != PACT_OK) return st;
  REQUIRE(ldx >= H && ldx % 8 == 0, PACT_ESHAPE, "ldx=%lld must be >= H and a multiple of 8", (long long)ldx);
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M=%lld exceeds the grid limit", (long long)M);
  const int force_exact = (flags & PACT_RMSNORM_EXACT_SUM) ? 1 : 0;
  return hip_status(pact::launch_rmsnorm_quant(x, gain, eps, M, H, ldx, y_codes, y_scales, y_rscale, rstd,
                                               force_exact, 0, as_stream(stream)),
                    "rmsnorm_quant launch");
}

int rmsnorm_quant(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t H, int64_t ldx,
                  uint8_t* y_codes, uint8_t* y_scales, float* y_rscale, float* rstd, void* stream) {
  return rmsnorm_quant_ex(x, gain, eps, M, H, ldx, 0, y_codes, y_scales, y_rscale, rstd, stream);
}

int silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t I, int64_t ld, uint8_t* h_codes,
                   uint8_t* h_scales, float* h_rscale, uint8_t* g_codes, uint8_t* g_scales, float* g_rscale,
                   uint8_t* u_codes, uint8_t* u_scales, float* u_rscale, void* stream) {
  REQUIRE(M >= 0 && I >= 0, PACT_EINVAL, "negative size (M=%lld, I=%lld)", (long long)M, (long long)I);
  REQUIRE(I % 16 == 0, PACT_ESHAPE, "I=%lld is not a multiple of 16", (long long)I);
  REQUIRE(I <= kMaxFusedCols, PACT_EUNSUPPORTED, "I=%lld exceeds %lld", (long long)I, (long long)kMaxFusedCols);
  if (M == 0) return ok();
  REQUIRE_PTR(gate, "gate");
  REQUIRE_PTR(up, "up");
  int st = check_nvfp4(h_codes, h_scales, h_rscale, "h");
  if (st == PACT_OK) st = check_nvfp4(g_codes, g_scales, g_rscale, "gate_q");
  if (st == PACT_OK) st = check_nvfp4(u_codes, u_scales, u_rscale, "up_q");
  if (st != PACT_OK) return st;
  REQUIRE(ld >= I && ld % 8 == 0, PACT_ESHAPE, "ld=%lld must be >= I and a multiple of 8", (long long)ld);
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M=%lld exceeds the grid limit", (long long)M);
  return hip_status(pact::launch_silu_mul_quant(gate, up, M, I, ld, h_codes, h_scales, h_rscale, g_codes, g_scales,
                                                g_rscale, u_codes, u_scales, u_rscale, 0, as_stream(stream)),
                    "silu_mul_quant launch");
}

static int gemm_common(pact::GemmArgs& a, const char* name, void* stream) {
  REQUIRE(a.M >= 0 && a.N >= 0 && a.K >= 0, PACT_EINVAL, "%s: negative size", name);
  REQUIRE(a.K % 16 == 0, PACT_ESHAPE, "%s: contraction length %lld is not a multiple of 16", name,
          (long long)a.K);
  if (a.M == 0 || a.N == 0) return ok();
  int st = check_nvfp4(a.a_codes, a.a_scales, a.a_rscale, "A");
  if (st == PACT_OK) st = check_nvfp4(a.b_codes, a.b_scales, a.b_rscale, "B");
  if (st != PACT_OK) return st;
  REQUIRE(a.out != nullptr, PACT_EINVAL, "%s: output is NULL", name);
  REQUIRE((reinterpret_cast<uintptr_t>(a.out) & 1u) == 0, PACT_EALIGN, "%s: output is not 2-byte aligned", name);
  REQUIRE(a.ldo >= a.N, PACT_ESHAPE, "%s: leading dimension %lld < %lld", name, (long long)a.ldo, (long long)a.N);
  if (a.lora_t != nullptr) {
    REQUIRE(a.lora_u != nullptr, PACT_EINVAL, "%s: LoRA T given without its second factor", name);
    REQUIRE(a.lora_r >= 1 && a.lora_r <= kMaxRank, PACT_ESHAPE, "%s: LoRA rank %lld outside [1, %lld]", name,
            (long long)a.lora_r, (long long)kMaxRank);
  }
  REQUIRE((a.M + 127) / 128 * ((a.N + 127) / 128) < 0x7FFFFFFF, PACT_EUNSUPPORTED, "%s: too many tiles", name);
  return hip_status(pact::launch_gemm(a, as_stream(stream)), name);
}

int nvfp4_gemm_fwd(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
                   const uint8_t* w_codes, const uint8_t* w_scales, const float* w_rscale, int64_t N, uint16_t* y,
                   int64_t ldy, const uint16_t* lora_t, const uint16_t* lora_b, int64_t lora_r, float lora_scale,
                   void* stream) {
  return nvfp4_gemm_fwd_ex(x_codes, x_scales, x_rscale, M, K, w_codes, w_scales, w_rscale, N, y, ldy, lora_t, lora_b,
                           lora_r, lora_scale, 0, stream);
}

int nvfp4_gemm_fwd_ex(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
                      const uint8_t* w_codes, const uint8_t* w_scales, const float* w_rscale, int64_t N, uint16_t* y,
                      int64_t ldy, const uint16_t* lora_t, const uint16_t* lora_b, int64_t lora_r, float lora_scale,
                      int flags, void* stream) {
  REQUIRE((flags & ~PACT_GEMM_ANY_ROW_SCALES) == 0, PACT_EINVAL, "unknown flags 0x%x", flags);
  pact::GemmArgs a{};
  a.general = (flags & PACT_GEMM_ANY_ROW_SCALES) ? 1 : 0;
  a.a_codes = x_codes; a.a_scales = x_scales; a.a_rscale = x_rscale;
  a.b_codes = w_codes; a.b_scales = w_scales; a.b_rscale = w_rscale;
  a.M = M; a.N = N; a.K = K;
  a.out = y; a.ldo = ldy; a.accumulate = 0;
  a.lora_t = lora_t; a.lora_u = lora_b;
  a.u_stride_j = 1; a.u_stride_n = lora_r;   // U(j, n) = B[n][j], B is [N x r]
  a.lora_r = lora_r; a.lora_scale = lora_scale;
  return gemm_common(a, "nvfp4_gemm_fwd", stream);
}

int nvfp4_gemm_dgrad(const uint8_t* dy_codes, const uint8_t* dy_scales, const float* dy_rscale, int64_t M, int64_t N,
                     const uint8_t* w_codes, const uint8_t* w_scales, const float* w_rscale, int64_t K, uint16_t* dx,
                     int64_t lddx, int accumulate, const uint16_t* lora_dt, const uint16_t* lora_a, int64_t lora_r,
                     void* stream) {
  return nvfp4_gemm_dgrad_ex(dy_codes, dy_scales, dy_rscale, M, N, w_codes, w_scales, w_rscale, K, dx, lddx,
                             accumulate, lora_dt, lora_a, lora_r, 0, stream);
}

int nvfp4_gemm_dgrad_ex(const uint8_t* dy_codes, const uint8_t* dy_scales, const float* dy_rscale, int64_t M,
                        int64_t N, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_rscale, int64_t K,
                        uint16_t* dx, int64_t lddx, int accumulate, const uint16_t* lora_dt, const uint16_t* lora_a,
                        int64_t lora_r, int flags, void* stream) {
  REQUIRE(accumulate == 0 || accumulate == 1, PACT_EINVAL, "accumulate must be 0 or 1 (got %d)", accumulate);
  REQUIRE((flags & ~PACT_GEMM_ANY_ROW_SCALES) == 0, PACT_EINVAL, "unknown flags 0x%x", flags);
  pact::GemmArgs a{};
  a.general = (flags & PACT_GEMM_ANY_ROW_SCALES) ? 1 : 0;
  a.a_codes = dy_codes; a.a_scales = dy_scales; a.a_rscale = dy_rscale;
  a.b_codes = w_codes; a.b_scales = w_scales; a.b_rscale = w_rscale;
  a.M = M; a.N = K; a.K = N;                 // output [M x K], contraction over N
  a.out = dx; a.ldo = lddx; a.accumulate = accumulate;
  a.lora_t = lora_dt; a.lora_u = lora_a;
  a.u_stride_j = K; a.u_stride_n = 1;        // U(j, k) = A[j][k], A is [r x K]
  a.lora_r = lora_r; a.lora_scale = 1.0f;
  return gemm_common(a, "nvfp4_gemm_dgrad", stream);
}

int nvfp4_gemm_dgrad_multi(int nseg, const uint8_t* const* dy_codes, const uint8_t* const* dy_scales,
                           const float* const* dy_rscale, const int64_t* seg_n, const uint8_t* const* w_codes,
                           const uint8_t* const* w_scales, const float* const* w_rscale, int64_t M, int64_t K,
                           uint16_t* dx, int64_t lddx, int accumulate, const uint16_t* const* lora_dt,
                           const uint16_t* const* lora_a, const int64_t* lora_r, void* stream) {
  REQUIRE(nseg >= 1 && nseg <= pact::kMaxSeg, PACT_EINVAL, "nseg=%d outside [1, %d]", nseg, pact::kMaxSeg);
  REQUIRE(dy_codes && dy_scales && dy_rscale && seg_n && w_codes && w_scales && w_rscale, PACT_EINVAL,
          "NULL segment array");
  REQUIRE(accumulate == 0 || accumulate == 1, PACT_EINVAL, "accumulate must be 0 or 1 (got %d)", accumulate);
  REQUIRE(M >= 0 && K >= 0, PACT_EINVAL, "negative size");
  REQUIRE(lora_dt == nullptr || (lora_a != nullptr && lora_r != nullptr), PACT_EINVAL,
          "LoRA dT array given without the A and rank arrays");
  pact::GemmArgs a{};
  pact::SegArgs sg{};
  sg.nseg = nseg;
  for (int i = 0; i < nseg; ++i) {
    REQUIRE(seg_n[i] > 0 && seg_n[i] % 256 == 0, PACT_EUNSUPPORTED,
            "segment %d: contraction length %lld is not a positive multiple of 256", i, (long long)seg_n[i]);
    pact::SegOperand& o = sg.s[i];
    o.a_codes = dy_codes[i]; o.a_scales = dy_scales[i]; o.a_rscale = dy_rscale[i];
    o.b_codes = w_codes[i]; o.b_scales = w_scales[i]; o.b_rscale = w_rscale[i];
    o.K = seg_n[i];
    if (M > 0 && K > 0) {
      int st = check_nvfp4(o.a_codes, o.a_scales, o.a_rscale, "dY segment");
      if (st == PACT_OK) st = check_nvfp4(o.b_codes, o.b_scales, o.b_rscale, "W_bwd segment");
      if (st != PACT_OK) return st;
    }
    if (lora_dt != nullptr && lora_dt[i] != nullptr) {
      REQUIRE(lora_a[i] != nullptr, PACT_EINVAL, "segment %d: LoRA dT given without A", i);
      REQUIRE(lora_r[i] >= 1 && lora_r[i] <= kMaxRank, PACT_ESHAPE, "segment %d: LoRA rank %lld outside [1, %lld]",
              i, (long long)lora_r[i], (long long)kMaxRank);
      o.lora_t = lora_dt[i]; o.lora_u = lora_a[i]; o.lora_r = lora_r[i];
    }
  }
  if (M == 0 || K == 0) return ok();
  REQUIRE(dx != nullptr, PACT_EINVAL, "dx is NULL");
  REQUIRE((reinterpret_cast<uintptr_t>(dx) & 1u) == 0, PACT_EALIGN, "dx is not 2-byte aligned");
  REQUIRE(lddx >= K, PACT_ESHAPE, "leading dimension %lld < %lld", (long long)lddx, (long long)K);
  // segment 0 fills the plain fields (the kernel's first descriptors)
  a.a_codes = sg.s[0].a_codes; a.a_scales = sg.s[0].a_scales; a.a_rscale = sg.s[0].a_rscale;
  a.b_codes = sg.s[0].b_codes; a.b_scales = sg.s[0].b_scales; a.b_rscale = sg.s[0].b_rscale;
  a.M = M; a.N = K; a.K = sg.s[0].K;
  a.out = dx; a.ldo = lddx; a.accumulate = accumulate;
  a.u_stride_j = K; a.u_stride_n = 1;        // U(j, k) = A[j][k], A is [r x K]
  a.lora_scale = 1.0f;
  REQUIRE(pact::gemm_multi_supported(a, sg), PACT_EUNSUPPORTED,
          "operands too large for 32-bit buffer offsets (M=%lld, K=%lld)", (long long)M, (long long)K);
  REQUIRE((M + 127) / 128 * ((K + 127) / 128) < 0x7FFFFFFF, PACT_EUNSUPPORTED, "too many tiles");
  return hip_status(pact::launch_gemm_multi(a, sg, as_stream(stream)), "nvfp4_gemm_dgrad_multi launch");
}

int lora_down(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
              const uint16_t* A, int64_t r, uint16_t* T, void* stream) {
  REQUIRE(M >= 0 && K >= 0, PACT_EINVAL, "negative size");
  REQUIRE(K % 16 == 0, PACT_ESHAPE, "K=%lld is not a multiple of 16", (long long)K);
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  if (M == 0) return ok();
  int st = check_nvfp4(x_codes, x_scales, x_rscale, "x");
  if (st != PACT_OK) return st;
  REQUIRE_PTR(A, "A");
  REQUIRE_PTR(T, "T");
  REQUIRE((M + 15) / 16 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_lora_down(x_codes, x_scales, x_rscale, M, K, A, r, T, as_stream(stream)),
                    "lora_down launch");
}

int pact_lora_bwd_workspace_size(int64_t M, int64_t K, int64_t N, int64_t r, size_t* bytes) {
  REQUIRE(M >= 0 && K >= 0 && N >= 0, PACT_EINVAL, "negative size");
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  REQUIRE(bytes != nullptr, PACT_EINVAL, "NULL output pointer");
  *bytes = pact::lora_bwd_workspace(M, K, N, r);
  return ok();
}

int lora_bwd(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
             const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy, int64_t N,
             uint16_t* dT, uint16_t* dA, uint16_t* dB, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(M >= 0 && K >= 0 && N >= 0, PACT_EINVAL, "negative size");
  REQUIRE(K % 16 == 0 && N % 16 == 0, PACT_ESHAPE, "K=%lld and N=%lld must be multiples of 16", (long long)K,
          (long long)N);
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  if (M > 0) {
    int st = check_nvfp4(x_codes, x_scales, x_rscale, "x");
    if (st != PACT_OK) return st;
    REQUIRE_PTR(dy, "dy");
    REQUIRE_PTR(dT, "dT");
  }
  REQUIRE_PTR(A, "A");
  REQUIRE_PTR(B, "B");
  REQUIRE_PTR(dA, "dA");
  REQUIRE_PTR(dB, "dB");
  const size_t need = pact::lora_bwd_workspace(M, K, N, r);
  REQUIRE(workspace != nullptr, PACT_EINVAL, "workspace is NULL (needs %zu bytes)", need);
  REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PACT_EALIGN, "workspace is not 256-byte aligned");
  REQUIRE(workspace_bytes >= need, PACT_EINVAL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  REQUIRE((M + 15) / 16 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_lora_bwd(x_codes, x_scales, x_rscale, M, K, A, B, r, scale, dy, N, dT, dA, dB,
                                          workspace, as_stream(stream)),
                    "lora_bwd launch");
}

int lora_bwd_dt(const uint16_t* dy, int64_t M, int64_t N, const uint16_t* B, int64_t r, float scale, uint16_t* dT,
                void* stream) {
  REQUIRE(M >= 0 && N >= 0, PACT_EINVAL, "negative size");
  REQUIRE(N % 16 == 0, PACT_ESHAPE, "N=%lld must be a multiple of 16", (long long)N);
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  if (M == 0) return ok();
  REQUIRE_PTR(dy, "dy");
  REQUIRE_PTR(B, "B");
  REQUIRE_PTR(dT, "dT");
  REQUIRE((M + 15) / 16 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_lora_bwd_dt(dy, M, N, B, r, scale, dT, as_stream(stream)), "lora_bwd_dt launch");
}

int lora_bwd_ab(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
                const uint16_t* A, int64_t r, float scale, const uint16_t* dy, int64_t N, const uint16_t* dT,
                uint16_t* dA, uint16_t* dB, void* workspace, size_t workspace_bytes, void* stream) {
  REQUIRE(M >= 0 && K >= 0 && N >= 0, PACT_EINVAL, "negative size");
  REQUIRE(K % 16 == 0 && N % 16 == 0, PACT_ESHAPE, "K=%lld and N=%lld must be multiples of 16", (long long)K,
          (long long)N);
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  if (M > 0) {
    int st = check_nvfp4(x_codes, x_scales, x_rscale, "x");
    if (st != PACT_OK) return st;
    REQUIRE_PTR(dy, "dy");
    REQUIRE_PTR(dT, "dT");
  }
  REQUIRE_PTR(A, "A");
  REQUIRE_PTR(dA, "dA");
  REQUIRE_PTR(dB, "dB");
  const size_t need = pact::lora_bwd_workspace(M, K, N, r);
  REQUIRE(workspace != nullptr, PACT_EINVAL, "workspace is NULL (needs %zu bytes)", need);
  REQUIRE((reinterpret_cast<uintptr_t>(workspace) & 255u) == 0, PACT_EALIGN, "workspace is not 256-byte aligned");
  REQUIRE(workspace_bytes >= need, PACT_EINVAL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  REQUIRE((M + 15) / 16 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_lora_bwd_ab(x_codes, x_scales, x_rscale, M, K, A, r, scale, dy, N, dT, dA, dB,
                                             workspace, as_stream(stream)),
                    "lora_bwd_ab launch");
}

int lora_bwd_ab_batch(int n, const uint8_t* const* x_codes, const uint8_t* const* x_scales,
                      const float* const* x_rscale, int64_t M, const int64_t* K, const uint16_t* const* T,
                      const int64_t* ldT, const int64_t* r, float scale, const uint16_t* const* dy,
                      const int64_t* N, const uint16_t* const* dT, uint16_t* const* dA, uint16_t* const* dB,
                      void* const* workspace, const size_t* workspace_bytes, void* stream) {
  REQUIRE(n >= 1 && n <= pact::kLoraBatch, PACT_EINVAL, "n=%d outside [1, %d]", n, pact::kLoraBatch);
  REQUIRE(x_codes && x_scales && x_rscale && K && T && ldT && r && dy && N && dT && dA && dB && workspace &&
              workspace_bytes,
          PACT_EINVAL, "a problem array is NULL");
  REQUIRE(M >= 0, PACT_EINVAL, "negative size");
  REQUIRE((M + 63) / 64 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  for (int i = 0; i < n; ++i) {
    REQUIRE(K[i] >= 0 && N[i] >= 0, PACT_EINVAL, "problem %d: negative size", i);
    REQUIRE(K[i] % 16 == 0 && N[i] % 16 == 0, PACT_ESHAPE, "problem %d: K=%lld and N=%lld must be multiples of 16",
            i, (long long)K[i], (long long)N[i]);
    REQUIRE(r[i] >= 1 && r[i] <= kMaxRank, PACT_ESHAPE, "problem %d: rank %lld outside [1, %lld]", i,
            (long long)r[i], (long long)kMaxRank);
    REQUIRE(pact::lora_same_rank_class(r[0], r[i]), PACT_EINVAL,
            "problem %d: rank %lld is not in the rank class of problem 0's rank %lld", i, (long long)r[i],
            (long long)r[0]);
    REQUIRE(ldT[i] >= r[i], PACT_ESHAPE, "problem %d: ldT=%lld is below the rank %lld", i, (long long)ldT[i],
            (long long)r[i]);
    if (M > 0) {
      int st = check_nvfp4(x_codes[i], x_scales[i], x_rscale[i], "x");
      if (st != PACT_OK) return st;
      REQUIRE(T[i] != nullptr && dy[i] != nullptr && dT[i] != nullptr, PACT_EINVAL,
              "problem %d: T, dy or dT is NULL", i);
    }
    REQUIRE(dA[i] != nullptr && dB[i] != nullptr, PACT_EINVAL, "problem %d: dA or dB is NULL", i);
    const size_t need = pact::lora_bwd_workspace(M, K[i], N[i], r[i]);
    REQUIRE(workspace[i] != nullptr, PACT_EINVAL, "problem %d: workspace is NULL (needs %zu bytes)", i, need);
    REQUIRE((reinterpret_cast<uintptr_t>(workspace[i]) & 255u) == 0, PACT_EALIGN,
            "problem %d: workspace is not 256-byte aligned", i);
    REQUIRE(workspace_bytes[i] >= need, PACT_EINVAL, "problem %d: workspace has %zu bytes, needs %zu", i,
            workspace_bytes[i], need);
  }
  return hip_status(pact::launch_lora_bwd_ab_batch(n, x_codes, x_scales, x_rscale, M, K, T, ldT, r, scale, dy, N, dT,
                                                   dA, dB, workspace, as_stream(stream)),
                    "lora_bwd_ab_batch launch");
}

int lora_bwd_noalloc(const uint8_t* x_codes, const uint8_t* x_scales, const float* x_rscale, int64_t M, int64_t K,
                     const uint16_t* A, const uint16_t* B, int64_t r, float scale, const uint16_t* dy, int64_t N,
                     uint16_t* dT, uint16_t* dA, uint16_t* dB, void* stream) {
  REQUIRE(M >= 0 && K >= 0 && N >= 0, PACT_EINVAL, "negative size");
  REQUIRE(K % 16 == 0 && N % 16 == 0, PACT_ESHAPE, "K=%lld and N=%lld must be multiples of 16", (long long)K,
          (long long)N);
  REQUIRE(r >= 1 && r <= kMaxRank, PACT_ESHAPE, "rank %lld outside [1, %lld]", (long long)r, (long long)kMaxRank);
  if (M > 0) {
    int st = check_nvfp4(x_codes, x_scales, x_rscale, "x");
    if (st != PACT_OK) return st;
    REQUIRE_PTR(dy, "dy");
    REQUIRE_PTR(dT, "dT");
  }
  REQUIRE_PTR(A, "A");
  REQUIRE_PTR(B, "B");
  REQUIRE_PTR(dA, "dA");
  REQUIRE_PTR(dB, "dB");
  const size_t need = pact::lora_bwd_workspace(M, K, N, r);
  REQUIRE(need <= pact::kLoraScratchBytes, PACT_EUNSUPPORTED,
          "lora_bwd_noalloc: M=%lld K=%lld N=%lld r=%lld needs %zu bytes of scratch, more than the fixed %zu "
          "(use lora_bwd with a workspace)",
          (long long)M, (long long)K, (long long)N, (long long)r, need, pact::kLoraScratchBytes);
  REQUIRE((M + 15) / 16 < 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  void* ws = nullptr;
  int st = hip_status(pact::lora_scratch_address(&ws), "lora_bwd_noalloc scratch lookup");
  if (st != PACT_OK) return st;
  return hip_status(pact::launch_lora_bwd(x_codes, x_scales, x_rscale, M, K, A, B, r, scale, dy, N, dT, dA, dB, ws,
                                          as_stream(stream)),
                    "lora_bwd_noalloc launch");
}

int silu_mul_bwd(const uint8_t* g_codes, const uint8_t* g_scales, const float* g_rscale, const uint8_t* u_codes,
                 const uint8_t* u_scales, const float* u_rscale, const uint16_t* dh, int64_t M, int64_t I,
                 uint16_t* dgate, uint16_t* dup, void* stream) {
  REQUIRE(M >= 0 && I >= 0, PACT_EINVAL, "negative size");
  REQUIRE(I % 16 == 0, PACT_ESHAPE, "I=%lld is not a multiple of 16", (long long)I);
  if (M == 0 || I == 0) return ok();
  int st = check_nvfp4(g_codes, g_scales, g_rscale, "gate_q");
  if (st == PACT_OK) st = check_nvfp4(u_codes, u_scales, u_rscale, "up_q");
  if (st != PACT_OK) return st;
  REQUIRE_PTR(dh, "dh");
  REQUIRE_PTR(dgate, "dgate");
  REQUIRE_PTR(dup, "dup");
  return hip_status(pact::launch_silu_mul_bwd(g_codes, g_scales, g_rscale, u_codes, u_scales, u_rscale, dh, M, I,
                                              dgate, dup, as_stream(stream)),
                    "silu_mul_bwd launch");
}

int rmsnorm_bwd(const uint8_t* y_codes, const uint8_t* y_scales, const float* y_rscale, const float* rstd,
                const uint16_t* gain, const uint16_t* dy, int64_t M, int64_t H, uint16_t* dx, void* stream) {
  REQUIRE(M >= 0 && H >= 0, PACT_EINVAL, "negative size");
  REQUIRE(H % 16 == 0, PACT_ESHAPE, "H=%lld is not a multiple of 16", (long long)H);
  REQUIRE(H <= kMaxFusedCols, PACT_EUNSUPPORTED, "H=%lld exceeds %lld", (long long)H, (long long)kMaxFusedCols);
  if (M == 0 || H == 0) return ok();
  int st = check_nvfp4(y_codes, y_scales, y_rscale, "y");
  if (st != PACT_OK) return st;
  REQUIRE_PTR(rstd, "rstd");
  REQUIRE_PTR(gain, "gain");
  REQUIRE_PTR(dy, "dy");
  REQUIRE_PTR(dx, "dx");
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_rmsnorm_bwd(y_codes, y_scales, y_rscale, rstd, gain, dy, M, H, nullptr, dx,
                                             nullptr, nullptr, nullptr, 0, as_stream(stream)),
                    "rmsnorm_bwd launch");
}

int pact_selftest_arith(unsigned long long* counts, void* stream) {
  REQUIRE(counts != nullptr, PACT_EINVAL, "NULL counts");
  return hip_status(pact::launch_selftest_arith(counts, as_stream(stream)), "selftest launch");
}

int pact_mfma_probe(int kind, int iters, float* sink, int64_t sink_len, unsigned long long* clocks,
                    int64_t clocks_len, void* stream) {
  REQUIRE(kind == 0 || kind == 1, PACT_EINVAL, "kind must be 0 (FP16) or 1 (scaled FP4), got %d", kind);
  REQUIRE(iters >= 1 && iters <= (1 << 20), PACT_EINVAL, "iters=%d outside 1 .. 2^20", iters);
  REQUIRE(sink != nullptr && clocks != nullptr, PACT_EINVAL, "NULL sink or clocks");
  REQUIRE(sink_len >= (int64_t)pact::kMfmaProbeGroups * 256, PACT_ESHAPE, "sink holds %lld floats, needs %d",
          (long long)sink_len, pact::kMfmaProbeGroups * 256);
  REQUIRE(clocks_len >= (int64_t)pact::kMfmaProbeGroups * 2, PACT_ESHAPE, "clocks holds %lld values, needs %d",
          (long long)clocks_len, pact::kMfmaProbeGroups * 2);
  return hip_status(pact::launch_mfma_probe(kind, iters, sink, clocks, as_stream(stream)), "mfma probe launch");
}

int pact_nvfp4_row_exp_max(const uint8_t* codes, const uint8_t* scales, const float* rscale, int64_t rows,
                           int64_t cols, int* out, void* stream) {
  REQUIRE(rows > 0 && cols > 0, PACT_EINVAL, "rows=%lld and cols=%lld must be positive", (long long)rows,
          (long long)cols);
  REQUIRE(cols % 16 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 16", (long long)cols);
  int st = check_nvfp4(codes, scales, rscale, "x");
  if (st != PACT_OK) return st;
  REQUIRE(out != nullptr, PACT_EINVAL, "out is NULL");
  REQUIRE((reinterpret_cast<uintptr_t>(out) & 3u) == 0, PACT_EALIGN, "out is not 4-byte aligned");
  hipStream_t s = as_stream(stream);
  st = hip_status(pact::launch_row_exp_max(rscale, scales, rows, cols, out, s), "row exponent range launch");
  if (st != PACT_OK) return st;
  // a once-per-weight set-up call: wait for the two exponents and check the
  // window in which the single-layout dgrad's FP16 operand is exact
  int host[2] = {0, 0};
  st = hip_status(hipMemcpyAsync(host, out, sizeof(host), hipMemcpyDeviceToHost, s), "row exponent read-back");
  if (st != PACT_OK) return st;
  st = hip_status(hipStreamSynchronize(s), "row exponent read-back");
  if (st != PACT_OK) return st;
  REQUIRE(host[0] <= 127, PACT_EUNSUPPORTED,
          "a nonzero row has a row scale that is not a power of two: the single-layout dgrad cannot fold it into "
          "its FP16 operand exactly");
  REQUIRE(host[0] - host[1] <= 14, PACT_EUNSUPPORTED,
          "nonzero rows span row exponents %d .. %d (more than 14 apart): the single-layout dgrad would not be "
          "exact for this weight",
          host[1], host[0]);
  return ok();
}

int nvfp4_gemm_dgrad_fwd_layout(const uint8_t* dy_codes, const uint8_t* dy_scales, const float* dy_rscale, int64_t M,
                                int64_t N, const uint8_t* w_codes, const uint8_t* w_scales, const float* w_rscale,
                                const int* w_exp_max, int64_t K, uint16_t* dx, int64_t ldx, int accumulate,
                                const uint16_t* lora_dt, const uint16_t* lora_a, int64_t r, void* stream) {
  REQUIRE(M >= 0 && N >= 0 && K >= 0, PACT_EINVAL, "negative size");
  REQUIRE(accumulate == 0 || accumulate == 1, PACT_EINVAL, "accumulate must be 0 or 1");
  REQUIRE(N % 16 == 0 && K % 16 == 0, PACT_ESHAPE, "N=%lld and K=%lld must be multiples of 16", (long long)N,
          (long long)K);
  if (M == 0 || K == 0) return ok();
  REQUIRE(N > 0, PACT_ESHAPE, "N must be positive");
  int st = check_nvfp4(dy_codes, dy_scales, dy_rscale, "dy_q");
  if (st == PACT_OK) st = check_nvfp4(w_codes, w_scales, w_rscale, "w_fwd");
  if (st != PACT_OK) return st;
  REQUIRE(w_exp_max != nullptr, PACT_EINVAL, "w_exp_max is NULL");
  REQUIRE((reinterpret_cast<uintptr_t>(w_exp_max) & 3u) == 0, PACT_EALIGN, "w_exp_max is not 4-byte aligned");
  REQUIRE_PTR(dx, "dx");
  REQUIRE(ldx >= K, PACT_ESHAPE, "ldx=%lld < K=%lld", (long long)ldx, (long long)K);
  REQUIRE(lora_dt == nullptr || (lora_a != nullptr && r >= 1 && r <= 128), PACT_EINVAL,
          "LoRA term needs lora_a and 1 <= r <= 128");
  REQUIRE(pact::dgrad_fwdlayout_supported(M, N, K), PACT_EUNSUPPORTED,
          "single-layout dgrad needs N %% 256 == 0, K %% 64 == 0 and operands below 2^31 bytes (N=%lld, K=%lld)",
          (long long)N, (long long)K);
  return hip_status(pact::launch_dgrad_fwdlayout(dy_codes, dy_scales, dy_rscale, M, N, w_codes, w_scales, w_rscale,
                                                 w_exp_max, K, dx, ldx, accumulate, lora_dt, lora_a,
                                                 lora_dt != nullptr ? r : 0, as_stream(stream)),
                    "nvfp4_gemm_dgrad_fwd_layout launch");
}

int silu_mul_bwd_quant(const uint8_t* g_codes, const uint8_t* g_scales, const float* g_rscale,
                       const uint8_t* u_codes, const uint8_t* u_scales, const float* u_rscale, const uint16_t* dh,
                       int64_t M, int64_t I, uint16_t* dgate, uint16_t* dup, uint8_t* dg_codes, uint8_t* dg_scales,
                       float* dg_rscale, uint8_t* du_codes, uint8_t* du_scales, float* du_rscale, void* stream) {
  REQUIRE(M >= 0 && I >= 0, PACT_EINVAL, "negative size");
  REQUIRE(I % 16 == 0, PACT_ESHAPE, "I=%lld is not a multiple of 16", (long long)I);
  REQUIRE(I <= kMaxFusedCols, PACT_EUNSUPPORTED, "I=%lld exceeds %lld", (long long)I, (long long)kMaxFusedCols);
  if (M == 0 || I == 0) return ok();
  int st = check_nvfp4(g_codes, g_scales, g_rscale, "gate_q");
  if (st == PACT_OK) st = check_nvfp4(u_codes, u_scales, u_rscale, "up_q");
  if (st == PACT_OK) st = check_nvfp4(dg_codes, dg_scales, dg_rscale, "dgate_q");
  if (st == PACT_OK) st = check_nvfp4(du_codes, du_scales, du_rscale, "dup_q");
  if (st != PACT_OK) return st;
  REQUIRE_PTR(dh, "dh");
  REQUIRE_PTR(dgate, "dgate");
  REQUIRE_PTR(dup, "dup");
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_silu_mul_bwd_quant(g_codes, g_scales, g_rscale, u_codes, u_scales, u_rscale, dh, M,
                                                    I, dgate, dup, dg_codes, dg_scales, dg_rscale, du_codes,
                                                    du_scales, du_rscale, 0, as_stream(stream)),
                    "silu_mul_bwd_quant launch");
}

int rmsnorm_bwd_residual(const uint8_t* y_codes, const uint8_t* y_scales, const float* y_rscale, const float* rstd,
                         const uint16_t* gain, const uint16_t* dy, const uint16_t* resid, int64_t M, int64_t H,
                         uint16_t* dx, uint8_t* q_codes, uint8_t* q_scales, float* q_rscale, void* stream) {
  REQUIRE(M >= 0 && H >= 0, PACT_EINVAL, "negative size");
  REQUIRE(H % 16 == 0, PACT_ESHAPE, "H=%lld is not a multiple of 16", (long long)H);
  REQUIRE(H <= kMaxFusedCols, PACT_EUNSUPPORTED, "H=%lld exceeds %lld", (long long)H, (long long)kMaxFusedCols);
  const bool want_q = q_codes != nullptr || q_scales != nullptr || q_rscale != nullptr;
  if (M == 0 || H == 0) return ok();
  int st = check_nvfp4(y_codes, y_scales, y_rscale, "y");
  if (st == PACT_OK && want_q) st = check_nvfp4(q_codes, q_scales, q_rscale, "out_q");
  if (st != PACT_OK) return st;
  REQUIRE_PTR(rstd, "rstd");
  REQUIRE_PTR(gain, "gain");
  REQUIRE_PTR(dy, "dy");
  REQUIRE_PTR(dx, "dx");
  if (resid != nullptr) REQUIRE_PTR(resid, "resid");
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_rmsnorm_bwd(y_codes, y_scales, y_rscale, rstd, gain, dy, M, H, resid, dx,
                                             want_q ? q_codes : nullptr, q_scales, q_rscale, 0, as_stream(stream)),
                    "rmsnorm_bwd_residual launch");
}

int mxfp4_silu_mul_bwd_quant(const uint8_t* g_codes, const uint8_t* g_scales, const uint8_t* u_codes,
                             const uint8_t* u_scales, const uint16_t* dh, int64_t M, int64_t I, uint16_t* dgate,
                             uint16_t* dup, uint8_t* dg_codes, uint8_t* dg_scales, uint8_t* du_codes,
                             uint8_t* du_scales, void* stream) {
  REQUIRE(M >= 0 && I >= 0, PACT_EINVAL, "negative size");
  REQUIRE(I % 32 == 0, PACT_ESHAPE, "I=%lld is not a multiple of 32", (long long)I);
  REQUIRE(I <= kMaxFusedCols, PACT_EUNSUPPORTED, "I=%lld exceeds %lld", (long long)I, (long long)kMaxFusedCols);
  if (M == 0 || I == 0) return ok();
  REQUIRE_PTR(g_codes, "gate_q codes");
  REQUIRE_PTR(g_scales, "gate_q scales");
  REQUIRE_PTR(u_codes, "up_q codes");
  REQUIRE_PTR(u_scales, "up_q scales");
  REQUIRE_PTR(dg_codes, "dgate_q codes");
  REQUIRE_PTR(dg_scales, "dgate_q scales");
  REQUIRE_PTR(du_codes, "dup_q codes");
  REQUIRE_PTR(du_scales, "dup_q scales");
  REQUIRE_PTR(dh, "dh");
  REQUIRE_PTR(dgate, "dgate");
  REQUIRE_PTR(dup, "dup");
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_silu_mul_bwd_quant(g_codes, g_scales, nullptr, u_codes, u_scales, nullptr, dh, M, I,
                                                    dgate, dup, dg_codes, dg_scales, nullptr, du_codes, du_scales,
                                                    nullptr, 1, as_stream(stream)),
                    "mxfp4_silu_mul_bwd_quant launch");
}

int mxfp4_rmsnorm_bwd_residual(const uint8_t* y_codes, const uint8_t* y_scales, const float* rstd,
                               const uint16_t* gain, const uint16_t* dy, const uint16_t* resid, int64_t M, int64_t H,
                               uint16_t* dx, uint8_t* q_codes, uint8_t* q_scales, void* stream) {
  REQUIRE(M >= 0 && H >= 0, PACT_EINVAL, "negative size");
  REQUIRE(H % 32 == 0, PACT_ESHAPE, "H=%lld is not a multiple of 32", (long long)H);
  REQUIRE(H <= kMaxFusedCols, PACT_EUNSUPPORTED, "H=%lld exceeds %lld", (long long)H, (long long)kMaxFusedCols);
  REQUIRE((q_codes == nullptr) == (q_scales == nullptr), PACT_EINVAL, "q_codes and q_scales: both or neither");
  if (M == 0 || H == 0) return ok();
  REQUIRE_PTR(y_codes, "y codes");
  REQUIRE_PTR(y_scales, "y scales");
  if (q_codes != nullptr) {
    REQUIRE_PTR(q_codes, "out_q codes");
    REQUIRE_PTR(q_scales, "out_q scales");
  }
  REQUIRE_PTR(rstd, "rstd");
  REQUIRE_PTR(gain, "gain");
  REQUIRE_PTR(dy, "dy");
  REQUIRE_PTR(dx, "dx");
  if (resid != nullptr) REQUIRE_PTR(resid, "resid");
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M too large");
  return hip_status(pact::launch_rmsnorm_bwd(y_codes, y_scales, nullptr, rstd, gain, dy, M, H, resid, dx, q_codes,
                                             q_scales, nullptr, 1, as_stream(stream)),
                    "mxfp4_rmsnorm_bwd_residual launch");
}


int pact_mxfp4_sizes(int64_t rows, int64_t cols, size_t* codes_bytes, size_t* scales_bytes) {
  REQUIRE(rows >= 0 && cols >= 0, PACT_EINVAL, "negative size (rows=%lld, cols=%lld)", (long long)rows,
          (long long)cols);
  REQUIRE(cols % 32 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 32", (long long)cols);
  REQUIRE(codes_bytes && scales_bytes, PACT_EINVAL, "NULL output pointer");
  *codes_bytes = (size_t)(rows * (cols / 2));
  *scales_bytes = (size_t)(rows * (cols / 32));
  return ok();
}

int mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldx, int transpose, uint8_t* codes,
                   uint8_t* scales, void* stream) {
  REQUIRE(rows >= 0 && cols >= 0, PACT_EINVAL, "negative size (rows=%lld, cols=%lld)", (long long)rows,
          (long long)cols);
  REQUIRE(transpose == 0 || transpose == 1, PACT_EINVAL, "transpose must be 0 or 1 (got %d)", transpose);
  REQUIRE(cols % 32 == 0, PACT_ESHAPE, "cols=%lld is not a multiple of 32", (long long)cols);
  if (rows == 0 || cols == 0) return ok();
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(codes, "out codes");
  REQUIRE_PTR(scales, "out scales");
  if (transpose == 0) {
    REQUIRE(ldx >= cols, PACT_ESHAPE, "ldx=%lld < cols=%lld", (long long)ldx, (long long)cols);
    REQUIRE(ldx % 8 == 0, PACT_EALIGN, "ldx=%lld is not a multiple of 8 elements", (long long)ldx);
  } else {
    REQUIRE(ldx >= rows, PACT_ESHAPE, "ldx=%lld < rows=%lld (transposed input is [cols x rows])", (long long)ldx,
            (long long)rows);
  }
  REQUIRE(rows <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "rows=%lld exceeds the grid limit", (long long)rows);
  return hip_status(pact::launch_mx_quantize(x, rows, cols, ldx, transpose, codes, scales, as_stream(stream)),
                    "mxfp4_quantize launch");
}

int mxfp4_rmsnorm_quant(const uint16_t* x, const uint16_t* gain, float eps, int64_t M, int64_t H, int64_t ldx,
                        uint8_t* y_codes, uint8_t* y_scales, float* rstd, void* stream) {
  REQUIRE(M >= 0 && H >= 0, PACT_EINVAL, "negative size (M=%lld, H=%lld)", (long long)M, (long long)H);
  REQUIRE(H % 32 == 0, PACT_ESHAPE, "H=%lld is not a multiple of 32", (long long)H);
  REQUIRE(H <= kMaxFusedCols, PACT_EUNSUPPORTED, "H=%lld exceeds %lld", (long long)H, (long long)kMaxFusedCols);
  REQUIRE(eps >= 0.0f, PACT_EINVAL, "eps must be non-negative");
  if (M == 0) return ok();
  REQUIRE(H > 0, PACT_ESHAPE, "H must be positive");
  REQUIRE_PTR(x, "x");
  REQUIRE_PTR(gain, "gain");
  REQUIRE_PTR(rstd, "rstd");
  REQUIRE_PTR(y_codes, "y codes");
  REQUIRE_PTR(y_scales, "y scales");
  REQUIRE(ldx >= H && ldx % 8 == 0, PACT_ESHAPE, "ldx=%lld must be >= H and a multiple of 8", (long long)ldx);
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M=%lld exceeds the grid limit", (long long)M);
  return hip_status(pact::launch_rmsnorm_quant(x, gain, eps, M, H, ldx, y_codes, y_scales, nullptr, rstd, 0, 1,
                                               as_stream(stream)),
                    "mxfp4_rmsnorm_quant launch");
}

int mxfp4_silu_mul_quant(const uint16_t* gate, const uint16_t* up, int64_t M, int64_t I, int64_t ld,
                         uint8_t* h_codes, uint8_t* h_scales, uint8_t* g_codes, uint8_t* g_scales, uint8_t* u_codes,
                         uint8_t* u_scales, void* stream) {
  REQUIRE(M >= 0 && I >= 0, PACT_EINVAL, "negative size (M=%lld, I=%lld)", (long long)M, (long long)I);
  REQUIRE(I % 32 == 0, PACT_ESHAPE, "I=%lld is not a multiple of 32", (long long)I);
  REQUIRE(I <= kMaxFusedCols, PACT_EUNSUPPORTED, "I=%lld exceeds %lld", (long long)I, (long long)kMaxFusedCols);
  if (M == 0 || I == 0) return ok();
  REQUIRE_PTR(gate, "gate");
  REQUIRE_PTR(up, "up");
  REQUIRE_PTR(h_codes, "h codes");
  REQUIRE_PTR(h_scales, "h scales");
  REQUIRE_PTR(g_codes, "gate_q codes");
  REQUIRE_PTR(g_scales, "gate_q scales");
  REQUIRE_PTR(u_codes, "up_q codes");
  REQUIRE_PTR(u_scales, "up_q scales");
  REQUIRE(ld >= I && ld % 8 == 0, PACT_ESHAPE, "ld=%lld must be >= I and a multiple of 8", (long long)ld);
  REQUIRE(M <= 0x7FFFFFFF, PACT_EUNSUPPORTED, "M=%lld exceeds the grid limit", (long long)M);
  return hip_status(pact::launch_silu_mul_quant(gate, up, M, I, ld, h_codes, h_scales, nullptr, g_codes, g_scales,
                                                nullptr, u_codes, u_scales, nullptr, 1, as_stream(stream)),
                    "mxfp4_silu_mul_quant launch");
}

int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, int64_t M, int64_t K, const uint8_t* b_codes,
               const uint8_t* b_scales, int64_t N, uint16_t* c, int64_t ldc, int accumulate, void* stream) {
  REQUIRE(M >= 0 && N >= 0 && K >= 0, PACT_EINVAL, "negative size");
  REQUIRE(accumulate == 0 || accumulate == 1, PACT_EINVAL, "accumulate must be 0 or 1");
  REQUIRE(K % 128 == 0, PACT_ESHAPE, "K=%lld is not a multiple of 128", (long long)K);
  if (M == 0 || N == 0) return ok();
  REQUIRE(K > 0, PACT_ESHAPE, "K must be positive");
  REQUIRE_PTR(a_codes, "a codes");
  REQUIRE_PTR(a_scales, "a scales");
  REQUIRE_PTR(b_codes, "b codes");
  REQUIRE_PTR(b_scales, "b scales");
  REQUIRE_PTR(c, "c");
  REQUIRE(ldc >= N, PACT_ESHAPE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
  REQUIRE(pact::mx_gemm_supported(M, N, K), PACT_EUNSUPPORTED, "operands exceed 2^31 bytes of codes");
  REQUIRE((M + 127) / 128 * ((N + 127) / 128) < 0x7FFFFFFF, PACT_EUNSUPPORTED, "grid too large");
  return hip_status(pact::launch_mx_gemm(a_codes, a_scales, M, K, b_codes, b_scales, N, c, ldc, accumulate,
                                         as_stream(stream)),
                    "mxfp4_gemm launch");
}

}  // extern "C"
