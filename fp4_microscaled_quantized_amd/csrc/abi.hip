// extern "C" entry points of libfp4mx: argument validation, workspace
// carving and kernel dispatch.  Every declaration, its source passage, and the
// argument contract are in include/fp4mx.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "fp4mx_internal.h"

using namespace fp4mx;

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return FP4MX_E_HIP;
}

constexpr int kMaxDevices = 64;
// Per-device cache of the architecture check, written once per device.
std::atomic<int> g_dev_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

// FP4MX_DEVICE_ARCH, when set to a name other than gfx950, stands in for the
// queried architecture: every compute call refuses with FP4MX_E_DEVICE before
// touching a device.  It lets a host without a GPU exercise the refusal path;
// set to gfx950 (or unset) it changes nothing, the real query decides.
bool arch_override_refuses() {
  const char* a = getenv("FP4MX_DEVICE_ARCH");
  return a && *a && strncmp(a, "gfx950", 6) != 0;
}

int check_device() {
  if (arch_override_refuses()) return FP4MX_E_DEVICE;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return FP4MX_E_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e);
    st = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? FP4MX_OK : FP4MX_E_DEVICE;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// Largest dimension (and GEMM output leading dimension) accepted.  The GEMM
// addresses each 256-row tile through a buffer resource whose range must stay
// at or below the 2^31-byte out-of-range offset (256 rows x 2^21 fp32 =
// 2^31 B; 256 rows x 2^21 x 1 B of FP8 codes), and the tile kernels' grid
// y-extents (cols / 64 or / 128) stay far inside the launch limits.
constexpr int64_t kMaxDim = FP4MX_MAX_DIM;
bool dim_ok(int64_t d) { return d > 0 && d % 32 == 0 && d <= kMaxDim; }

size_t round_up(size_t v) { return (v + 255) & ~(size_t)255; }
size_t mx_bytes(int64_t rows, int64_t cols) {  // codes + scales, each padded
  return round_up((size_t)rows * cols / 2) + round_up((size_t)rows * cols / 32);
}

struct Carver {
  uint8_t* p;
  uint8_t* take(size_t n) {
    uint8_t* r = p;
    p += round_up(n);
    return r;
  }
};

int check_quant_args(const void* x, int64_t rows, int64_t cols, int64_t ld, int rounding,
                     const void* codes, const void* scales) {
  if (!x || !codes || !scales) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || ld < cols) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || ld % 8 != 0) return FP4MX_E_ALIGN;
  if (rounding != FP4MX_ROUND_RTN && rounding != FP4MX_ROUND_SR) return FP4MX_E_ARG;
  return FP4MX_OK;
}

int quantize_impl(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis, int rounding,
                  bool hadamard, uint32_t sign_mask, uint64_t seed, uint32_t stream_id,
                  uint8_t* codes, uint8_t* scales, void* stream) {
  int st = check_quant_args(x, rows, cols, ld, rounding, codes, scales);
  if (st) return st;
  if (axis != FP4MX_AXIS_ROW && axis != FP4MX_AXIS_COL) return FP4MX_E_ARG;
  if ((st = check_device())) return st;
  QuantOut o{rounding, sign_mask, make_key(seed, stream_id), codes, scales};
  hipError_t e;
  if (axis == FP4MX_AXIS_ROW)
    e = launch_quant_row(static_cast<const uint16_t*>(x), rows, cols, ld, hadamard, o,
                         (hipStream_t)stream);
  else
    e = launch_quant_tile(static_cast<const uint16_t*>(x), rows, cols, ld, hadamard, nullptr, &o,
                          (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int check_gemm_args(const void* a, const void* as, const void* b, const void* bs, int64_t m,
                    int64_t n, int64_t k, const float* c, int64_t ldc) {
  if (!a || !as || !b || !bs || !c) return FP4MX_E_NULL;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k) || ldc < n || ldc > kMaxDim) return FP4MX_E_SHAPE;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c) || ldc % 4 != 0) return FP4MX_E_ALIGN;
  return FP4MX_OK;
}

size_t nv_operand_bytes(int64_t rows, int64_t cols) {  // codes + e4m3 scales + tensor scale
  return round_up((size_t)rows * cols / 2) + round_up((size_t)rows * cols / 16) + 256;
}
size_t nv_staged_bytes(int64_t rows, int64_t cols) {  // fp8 operand + e8m0 scales
  return round_up((size_t)rows * cols) + round_up((size_t)rows * cols / 32);
}

}  // namespace

extern "C" {

const char* fp4mx_status_string(int status) {
  switch (status) {
    case FP4MX_OK: return "ok";
    case FP4MX_E_NULL: return "null pointer";
    case FP4MX_E_SHAPE: return "bad shape (dimensions must be positive multiples of 32, at most 2^21)";
    case FP4MX_E_ALIGN: return "bad alignment (16-byte pointers, leading dimension multiple of 8)";
    case FP4MX_E_ARG: return "bad argument";
    case FP4MX_E_WORKSPACE: return "workspace missing or too small";
    case FP4MX_E_DEVICE: return "device is not gfx950";
    case FP4MX_E_HIP: return "HIP error";
    case FP4MX_E_SCRATCH:
      return "input needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

int fp4mx_last_hip_error(void) { return g_last_hip_error; }

uint32_t fp4mx_sign_mask(uint64_t seed, uint32_t gemm_id) {
  return (uint32_t)splitmix64(seed ^ ((uint64_t)(0x5100u + gemm_id) << 32));
}

int fp4mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis, int rounding,
                   uint64_t seed, uint32_t rng_stream, uint8_t* codes, uint8_t* scales,
                   void* stream) {
  return quantize_impl(x, rows, cols, ld, axis, rounding, false, 0u, seed, rng_stream, codes,
                       scales, stream);
}

int fp4mx_hadamard_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                            int rounding, uint32_t sign_mask, uint64_t seed, uint32_t rng_stream,
                            uint8_t* codes, uint8_t* scales, void* stream) {
  return quantize_impl(x, rows, cols, ld, axis, rounding, true, sign_mask, seed, rng_stream, codes,
                       scales, stream);
}

int fp4mx_hadamard_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                 int row_rounding, uint32_t row_sign_mask, uint32_t row_rng_stream,
                                 int col_rounding, uint32_t col_sign_mask, uint32_t col_rng_stream,
                                 uint64_t seed, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, void* stream) {
  int st = check_quant_args(x, rows, cols, ld, row_rounding, row_codes, row_scales);
  if (st) return st;
  if (!col_codes || !col_scales) return FP4MX_E_NULL;
  if (!aligned16(col_codes)) return FP4MX_E_ALIGN;
  if (col_rounding != FP4MX_ROUND_RTN && col_rounding != FP4MX_ROUND_SR) return FP4MX_E_ARG;
  if ((st = check_device())) return st;
  QuantOut ro{row_rounding, row_sign_mask, make_key(seed, row_rng_stream), row_codes, row_scales};
  QuantOut co{col_rounding, col_sign_mask, make_key(seed, col_rng_stream), col_codes, col_scales};
  hipError_t e = launch_quant_tile(static_cast<const uint16_t*>(x), rows, cols, ld, true, &ro, &co,
                                   (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, float alpha, float* c,
               int64_t ldc, void* stream) {
  int st = check_gemm_args(a_codes, a_scales, b_codes, b_scales, m, n, k, c, ldc);
  if (st) return st;
  if ((st = check_device())) return st;
  hipError_t e = launch_mx_gemm(a_codes, a_scales, b_codes, b_scales, m, n, k, alpha, c, ldc,
                                (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_gemm_bf16(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                    const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, float alpha,
                    uint16_t* c, int64_t ldc, void* stream) {
  int st = check_gemm_args(a_codes, a_scales, b_codes, b_scales, m, n, k,
                           reinterpret_cast<const float*>(c), ldc);
  if (st) return st;
  if (ldc % 8 != 0) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  hipError_t e = launch_mx_gemm_bf16(a_codes, a_scales, b_codes, b_scales, m, n, k, alpha, c, ldc,
                                     (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

size_t fp4mx_linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  const size_t fwd = mx_bytes(m, k) + mx_bytes(n, k);
  const size_t bwd = mx_bytes(m, n) + mx_bytes(n, m);
  return fwd > bwd ? fwd : bwd;
}

size_t fp4mx_ctx_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return (size_t)k * m / 2 + (size_t)k * m / 32 + (size_t)k * n / 2 + (size_t)k * n / 32;
}

// Output element type of the linear entry points.
enum class Out { F32, BF16 };

static hipError_t gemm_out(Out o, const uint8_t* a, const uint8_t* as, const uint8_t* b,
                           const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha, void* c,
                           int64_t ldc, hipStream_t s) {
  return o == Out::F32
             ? launch_mx_gemm(a, as, b, bs, m, n, k, alpha, static_cast<float*>(c), ldc, s)
             : launch_mx_gemm_bf16(a, as, b, bs, m, n, k, alpha, static_cast<uint16_t*>(c), ldc, s);
}

static int linear_fwd_impl(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                           uint64_t seed, void* y, Out yo, const fp4mx_ctx* ctx, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!x || !w || !y) return FP4MX_E_NULL;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP4MX_E_ALIGN;
  if (ctx) {
    if (!ctx->xt_codes || !ctx->xt_scales || !ctx->wt_codes || !ctx->wt_scales) return FP4MX_E_NULL;
    if (!aligned16(ctx->xt_codes) || !aligned16(ctx->wt_codes)) return FP4MX_E_ALIGN;
    if (ctx->seed != seed) return FP4MX_E_ARG;
  }
  if (!ws || ws_bytes < fp4mx_linear_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  Carver cv{static_cast<uint8_t*>(ws)};
  uint8_t* xq = cv.take((size_t)m * k / 2);
  uint8_t* xs = cv.take((size_t)m * k / 32);
  uint8_t* wq = cv.take((size_t)n * k / 2);
  uint8_t* wsc = cv.take((size_t)n * k / 32);
  const uint32_t g0 = fp4mx_sign_mask(seed, 0), g1 = fp4mx_sign_mask(seed, 1),
                 g2 = fp4mx_sign_mask(seed, 2);
  QuantOut xr{FP4MX_ROUND_RTN, g0, make_key(seed, 0), xq, xs};
  QuantOut wr{FP4MX_ROUND_RTN, g0, make_key(seed, 0), wq, wsc};
  hipError_t e;
  if (ctx) {
    QuantOut xc{FP4MX_ROUND_SR, g2, make_key(seed, 4), ctx->xt_codes, ctx->xt_scales};
    QuantOut wc{FP4MX_ROUND_SR, g1, make_key(seed, 2), ctx->wt_codes, ctx->wt_scales};
    e = launch_quant_tile_pair(static_cast<const uint16_t*>(x), m, k, k, xr, xc,
                               static_cast<const uint16_t*>(w), n, k, k, wr, wc, s);
  } else {
    e = launch_quant_row(static_cast<const uint16_t*>(x), m, k, k, true, xr, s);
    if (e == hipSuccess) e = launch_quant_row(static_cast<const uint16_t*>(w), n, k, k, true, wr, s);
  }
  if (e == hipSuccess) e = gemm_out(yo, xq, xs, wq, wsc, m, n, k, 1.0f, y, n, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

static int linear_bwd_impl(const void* dy, const fp4mx_ctx* ctx, int64_t m, int64_t n, int64_t k,
                           void* dx, void* dw, Out go, void* ws, size_t ws_bytes, void* stream) {
  if (!dy || !ctx || !dx || !dw) return FP4MX_E_NULL;
  if (!ctx->xt_codes || !ctx->xt_scales || !ctx->wt_codes || !ctx->wt_scales) return FP4MX_E_NULL;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(dw) || !aligned16(ctx->xt_codes) ||
      !aligned16(ctx->wt_codes))
    return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4mx_linear_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t seed = ctx->seed;
  Carver cv{static_cast<uint8_t*>(ws)};
  uint8_t* dq = cv.take((size_t)m * n / 2);
  uint8_t* ds = cv.take((size_t)m * n / 32);
  uint8_t* tq = cv.take((size_t)n * m / 2);
  uint8_t* ts = cv.take((size_t)n * m / 32);
  QuantOut r{FP4MX_ROUND_SR, fp4mx_sign_mask(seed, 1), make_key(seed, 1), dq, ds};
  QuantOut c{FP4MX_ROUND_SR, fp4mx_sign_mask(seed, 2), make_key(seed, 3), tq, ts};
  const float alpha = 16.0f / 9.0f;
  hipError_t e = launch_quant_tile(static_cast<const uint16_t*>(dy), m, n, n, true, &r, &c, s);
  if (e == hipSuccess) e = gemm_out(go, dq, ds, ctx->wt_codes, ctx->wt_scales, m, k, n, alpha, dx, k, s);
  if (e == hipSuccess) e = gemm_out(go, tq, ts, ctx->xt_codes, ctx->xt_scales, n, k, m, alpha, dw, k, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k, uint64_t seed,
                     float* y, const fp4mx_ctx* ctx, void* ws, size_t ws_bytes, void* stream) {
  return linear_fwd_impl(x, w, m, n, k, seed, y, Out::F32, ctx, ws, ws_bytes, stream);
}

int fp4mx_linear_fwd_bf16(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                          uint64_t seed, uint16_t* y, const fp4mx_ctx* ctx, void* ws,
                          size_t ws_bytes, void* stream) {
  return linear_fwd_impl(x, w, m, n, k, seed, y, Out::BF16, ctx, ws, ws_bytes, stream);
}

int fp4mx_linear_bwd(const void* dy, const fp4mx_ctx* ctx, int64_t m, int64_t n, int64_t k,
                     float* dx, float* dw, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(dy, ctx, m, n, k, dx, dw, Out::F32, ws, ws_bytes, stream);
}

int fp4mx_linear_bwd_bf16(const void* dy, const fp4mx_ctx* ctx, int64_t m, int64_t n, int64_t k,
                          uint16_t* dx, uint16_t* dw, void* ws, size_t ws_bytes, void* stream) {
  return linear_bwd_impl(dy, ctx, m, n, k, dx, dw, Out::BF16, ws, ws_bytes, stream);
}

// ------------------------------- QuEST -------------------------------------

static bool clip_ok(float c) { return c > 0.0f && c <= 3.0e38f; }
static bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

int fp4mx_quest_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, float clip,
                         uint32_t sign_mask, uint8_t* codes, uint8_t* scales, uint8_t* mask,
                         void* stream) {
  int st = check_quant_args(x, rows, cols, ld, FP4MX_ROUND_RTN, codes, scales);
  if (st) return st;
  if (!mask) return FP4MX_E_NULL;
  if (!aligned4(mask)) return FP4MX_E_ALIGN;
  if (!clip_ok(clip)) return FP4MX_E_ARG;
  if ((st = check_device())) return st;
  hipError_t e = launch_quest_row(static_cast<const uint16_t*>(x), rows, cols, ld, sign_mask, clip,
                                  codes, scales, mask, (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_requantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int rounding, uint32_t sign_mask, uint64_t seed, uint32_t rng_stream,
                     uint8_t* out_codes, uint8_t* out_scales, void* stream) {
  if (!codes || !scales || !out_codes || !out_scales) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols)) return FP4MX_E_SHAPE;
  if (!aligned16(codes) || !aligned16(out_codes)) return FP4MX_E_ALIGN;
  if (rounding != FP4MX_ROUND_RTN && rounding != FP4MX_ROUND_SR) return FP4MX_E_ARG;
  int st = check_device();
  if (st) return st;
  hipError_t e = launch_requant(codes, scales, rows, cols, rounding, sign_mask,
                                make_key(seed, rng_stream), out_codes, out_scales,
                                (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_unmask_inverse_hadamard(float* c, int64_t rows, int64_t cols, int64_t ldc,
                                  const uint8_t* mask, uint32_t sign_mask, void* stream) {
  if (!c || !mask) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || ldc < cols) return FP4MX_E_SHAPE;
  if (!aligned16(c) || ldc % 4 != 0 || !aligned4(mask)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipError_t e = launch_unmask_irht(c, rows, cols, ldc, mask, sign_mask, (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_gemm_unmask_irht(const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                           int64_t k, float alpha, float* c, int64_t ldc, const uint8_t* mask,
                           uint32_t sign_mask, void* stream) {
  int st = check_gemm_args(a_codes, a_scales, b_codes, b_scales, m, n, k, c, ldc);
  if (st) return st;
  if (!mask) return FP4MX_E_NULL;
  if (!aligned4(mask)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  hipError_t e = launch_mx_gemm_irht(a_codes, a_scales, b_codes, b_scales, m, n, k, alpha, c, ldc,
                                     mask, sign_mask, (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

size_t fp4mx_quest_ctx_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return mx_bytes(m, k) + mx_bytes(n, k) + round_up((size_t)m * k / 8) + round_up((size_t)n * k / 8);
}

size_t fp4mx_quest_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return 2 * mx_bytes(m, n) + mx_bytes(k, n) + mx_bytes(k, m);
}

static int quest_ctx_check(const fp4mx_quest_ctx* ctx) {
  if (!ctx) return FP4MX_E_NULL;
  if (!ctx->xq_codes || !ctx->xq_scales || !ctx->wq_codes || !ctx->wq_scales || !ctx->x_mask ||
      !ctx->w_mask)
    return FP4MX_E_NULL;
  if (!aligned16(ctx->xq_codes) || !aligned16(ctx->wq_codes) || !aligned4(ctx->x_mask) ||
      !aligned4(ctx->w_mask))
    return FP4MX_E_ALIGN;
  return FP4MX_OK;
}

int fp4mx_quest_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                           float clip, uint64_t seed, float* y, const fp4mx_quest_ctx* ctx,
                           void* stream) {
  if (!x || !w || !y) return FP4MX_E_NULL;
  int st = quest_ctx_check(ctx);
  if (st) return st;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP4MX_E_ALIGN;
  if (!clip_ok(clip) || ctx->seed != seed) return FP4MX_E_ARG;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint32_t g0 = fp4mx_sign_mask(seed, 0);
  hipError_t e = launch_quest_row(static_cast<const uint16_t*>(x), m, k, k, g0, clip,
                                  ctx->xq_codes, ctx->xq_scales, ctx->x_mask, s);
  if (e == hipSuccess)
    e = launch_quest_row(static_cast<const uint16_t*>(w), n, k, k, g0, clip, ctx->wq_codes,
                         ctx->wq_scales, ctx->w_mask, s);
  if (e == hipSuccess)
    e = launch_mx_gemm(ctx->xq_codes, ctx->xq_scales, ctx->wq_codes, ctx->wq_scales, m, n, k, 1.0f,
                       y, n, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4mx_quest_linear_bwd(const void* dy, const fp4mx_quest_ctx* ctx, int64_t m, int64_t n,
                           int64_t k, float* dx, float* dw, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!dy || !dx || !dw) return FP4MX_E_NULL;
  int st = quest_ctx_check(ctx);
  if (st) return st;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(dw)) return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4mx_quest_bwd_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  const uint64_t seed = ctx->seed;
  const uint32_t g0 = fp4mx_sign_mask(seed, 0), g1 = fp4mx_sign_mask(seed, 1),
                 g2 = fp4mx_sign_mask(seed, 2);
  Carver cv{static_cast<uint8_t*>(ws)};
  uint8_t* dq = cv.take((size_t)m * n / 2);
  uint8_t* ds = cv.take((size_t)m * n / 32);
  uint8_t* tq = cv.take((size_t)n * m / 2);
  uint8_t* ts = cv.take((size_t)n * m / 32);
  uint8_t* wtq = cv.take((size_t)k * n / 2);
  uint8_t* wts = cv.take((size_t)k * n / 32);
  uint8_t* xtq = cv.take((size_t)k * m / 2);
  uint8_t* xts = cv.take((size_t)k * m / 32);
  QuantOut r{FP4MX_ROUND_SR, g1, make_key(seed, 1), dq, ds};
  QuantOut c{FP4MX_ROUND_SR, g2, make_key(seed, 3), tq, ts};
  const float alpha = 16.0f / 9.0f;
  hipError_t e = launch_quant_tile(static_cast<const uint16_t*>(dy), m, n, n, true, &r, &c, s);
  if (e == hipSuccess)
    e = launch_requant(ctx->wq_codes, ctx->wq_scales, n, k, FP4MX_ROUND_SR, g1, make_key(seed, 2),
                       wtq, wts, s);
  if (e == hipSuccess)
    e = launch_requant(ctx->xq_codes, ctx->xq_scales, m, k, FP4MX_ROUND_SR, g2, make_key(seed, 4),
                       xtq, xts, s);
  if (e == hipSuccess)
    e = launch_mx_gemm_irht(dq, ds, wtq, wts, m, k, n, alpha, dx, k, ctx->x_mask, g0, s);
  if (e == hipSuccess)
    e = launch_mx_gemm_irht(tq, ts, xtq, xts, n, k, m, alpha, dw, k, ctx->w_mask, g0, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

// ------------------------------- NVFP4 -------------------------------------

size_t fp4nv_quantize_workspace_bytes(int64_t rows, int64_t cols) {
  (void)rows;
  (void)cols;
  return 256;
}

int fp4nv_quantize46(const void* x, int64_t rows, int64_t cols, int64_t ld, int use_46,
                     uint8_t* codes, uint8_t* scales, float* tensor_scale, void* ws,
                     size_t ws_bytes, void* stream) {
  if (!x || !codes || !scales || !tensor_scale) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || ld < cols) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 1u) || ld % 8 != 0)
    return FP4MX_E_ALIGN;
  if (use_46 != 0 && use_46 != 1) return FP4MX_E_ARG;
  if (!ws || ws_bytes < fp4nv_quantize_workspace_bytes(rows, cols)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = static_cast<uint32_t*>(ws);
  hipError_t e = launch_nv_amax(static_cast<const uint16_t*>(x), rows, cols, ld, amax, s);
  if (e == hipSuccess)
    e = launch_nv_quant(static_cast<const uint16_t*>(x), rows, cols, ld, use_46, amax, codes,
                        scales, tensor_scale, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

size_t fp4nv_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return nv_staged_bytes(m, k) + nv_staged_bytes(n, k);
}

static int nv_gemm_impl(const uint8_t* a, const uint8_t* as, const float* ga, const uint8_t* b,
                        const uint8_t* bs, const float* gb, int64_t m, int64_t n, int64_t k,
                        float* c, int64_t ldc, uint8_t* ws, hipStream_t s) {
  Carver cv{ws};
  uint8_t* fa = cv.take((size_t)m * k);
  uint8_t* ea = cv.take((size_t)m * k / 32);
  uint8_t* fb = cv.take((size_t)n * k);
  uint8_t* eb = cv.take((size_t)n * k / 32);
  hipError_t e = launch_nv_stage(a, as, m, k, fa, ea, s);
  if (e == hipSuccess) e = launch_nv_stage(b, bs, n, k, fb, eb, s);
  if (e == hipSuccess) e = launch_fp8_gemm(fa, ea, fb, eb, ga, gb, m, n, k, c, ldc, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

int fp4nv_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
               int64_t m, int64_t n, int64_t k, float* c, int64_t ldc, void* ws, size_t ws_bytes,
               void* stream) {
  int st = check_gemm_args(a_codes, a_scales, b_codes, b_scales, m, n, k, c, ldc);
  if (st) return st;
  if (!a_tensor_scale || !b_tensor_scale) return FP4MX_E_NULL;
  if (((uintptr_t)a_scales & 1u) || ((uintptr_t)b_scales & 1u)) return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_gemm_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  return nv_gemm_impl(a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_tensor_scale, m, n, k,
                      c, ldc, static_cast<uint8_t*>(ws), (hipStream_t)stream);
}

size_t fp4nv_linear_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return 512 + nv_operand_bytes(m, k) + nv_operand_bytes(n, k) + fp4nv_gemm_workspace_bytes(m, n, k);
}

int fp4nv_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k, float* y,
                     void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !y) return FP4MX_E_NULL;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_linear_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  Carver cv{static_cast<uint8_t*>(ws)};
  uint32_t* amax_x = reinterpret_cast<uint32_t*>(cv.take(4));
  uint32_t* amax_w = reinterpret_cast<uint32_t*>(cv.take(4));
  uint8_t* xq = cv.take((size_t)m * k / 2);
  uint8_t* xs = cv.take((size_t)m * k / 16);
  float* gx = reinterpret_cast<float*>(cv.take(4));
  uint8_t* wq = cv.take((size_t)n * k / 2);
  uint8_t* wsc = cv.take((size_t)n * k / 16);
  float* gw = reinterpret_cast<float*>(cv.take(4));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  hipError_t e = launch_nv_amax(xb, m, k, k, amax_x, s);
  if (e == hipSuccess) e = launch_nv_amax(wb, n, k, k, amax_w, s);
  if (e == hipSuccess) e = launch_nv_quant(xb, m, k, k, 1, amax_x, xq, xs, gx, s);
  if (e == hipSuccess) e = launch_nv_quant(wb, n, k, k, 1, amax_w, wq, wsc, gw, s);
  if (e != hipSuccess) return hip_fail(e);
  return nv_gemm_impl(xq, xs, gx, wq, wsc, gw, m, n, k, y, n, cv.p, s);
}

int fp4nv_sr_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, uint64_t seed,
                      uint32_t rng_stream, uint8_t* codes, uint8_t* scales, float* tensor_scale,
                      void* ws, size_t ws_bytes, void* stream) {
  if (!x || !codes || !scales || !tensor_scale) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || ld < cols) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 1u) || ld % 8 != 0 ||
      ((uintptr_t)tensor_scale & 3u))
    return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_quantize_workspace_bytes(rows, cols)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* amax = static_cast<uint32_t*>(ws);
  const RngKey key = make_key(seed, rng_stream);
  hipError_t e = launch_nv_amax(static_cast<const uint16_t*>(x), rows, cols, ld, amax, s);
  if (e == hipSuccess)
    e = launch_nv_sr(static_cast<const uint16_t*>(x), rows, cols, ld, amax, key.lo, key.hi, codes,
                     scales, tensor_scale, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

size_t fp4nv_msedn_workspace_bytes(int64_t rows, int64_t cols) {
  if (!dim_ok(rows) || !dim_ok(cols)) return 0;
  return round_up((size_t)rows * cols / 16 * sizeof(float)) + 256;
}

static int msedn_impl(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                      float clip_s, uint64_t seed, uint32_t gemm_id, uint32_t stream,
                      uint8_t* codes, uint8_t* scales, float* ts, float* eden_s, uint8_t* ws,
                      hipStream_t s) {
  Carver cv{ws};
  float* vbuf = reinterpret_cast<float*>(cv.take((size_t)rows * cols / 16 * sizeof(float)));
  uint32_t* gmax = reinterpret_cast<uint32_t*>(cv.take(4));
  hipError_t e = launch_msedn(static_cast<const uint16_t*>(x), rows, cols, ld, axis, clip_s, seed,
                              gemm_id, stream, codes, scales, ts, eden_s, vbuf, gmax, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

static int msedn_check(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                       float clip_s, const uint8_t* codes, const uint8_t* scales,
                       const float* tensor_scale, const float* eden_s) {
  if (!x || !codes || !scales || !tensor_scale) return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || ld < cols) return FP4MX_E_SHAPE;
  if (axis != FP4MX_AXIS_ROW && axis != FP4MX_AXIS_COL) return FP4MX_E_ARG;
  if ((axis == FP4MX_AXIS_ROW ? cols : rows) % 128 != 0) return FP4MX_E_SHAPE;
  if (!(clip_s > 0.0f) || !(clip_s < 1e30f)) return FP4MX_E_ARG;
  if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 1u) || ld % 8 != 0 ||
      ((uintptr_t)tensor_scale & 3u) || ((uintptr_t)eden_s & 3u))
    return FP4MX_E_ALIGN;
  return FP4MX_OK;
}

int fp4nv_msedn_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                         float clip_s, uint64_t seed, uint32_t gemm_id, uint32_t rng_stream,
                         uint8_t* codes, uint8_t* scales, float* tensor_scale, float* eden_s,
                         void* ws, size_t ws_bytes, void* stream) {
  int st = msedn_check(x, rows, cols, ld, axis, clip_s, codes, scales, tensor_scale, eden_s);
  if (st) return st;
  if (!ws || ws_bytes < fp4nv_msedn_workspace_bytes(rows, cols)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  return msedn_impl(x, rows, cols, ld, axis, clip_s, seed, gemm_id, rng_stream, codes, scales,
                    tensor_scale, eden_s, static_cast<uint8_t*>(ws), (hipStream_t)stream);
}

}  // extern "C"

// ---------------------- no-allocation MS-EDEN entry ----------------------
// The library's own scratch for fp4nv_msedn_quantize_noalloc: the fp32 v of
// every output 16-group and the tensor maximum, in one file-scope device
// array.  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never passes `scratch` itself to a kernel (in host code
// the name is a stand-in, not the device address): the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
namespace {

__device__ __align__(256) uint8_t scratch[FP4MX_NOALLOC_SCRATCH_BYTES];

std::atomic<uint8_t*> g_scratch_ptr[kMaxDevices];

int scratch_ptr(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return FP4MX_E_DEVICE;
  uint8_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!q) return FP4MX_E_DEVICE;
    p = static_cast<uint8_t*>(q);
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return FP4MX_OK;
}

}  // namespace

extern "C" {

int fp4nv_msedn_quantize_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                                 float clip_s, uint64_t seed, uint32_t gemm_id,
                                 uint32_t rng_stream, uint8_t* codes, uint8_t* scales,
                                 float* tensor_scale, float* eden_s, void* stream) {
  int st = msedn_check(x, rows, cols, ld, axis, clip_s, codes, scales, tensor_scale, eden_s);
  if (st) return st;
  if (fp4nv_msedn_workspace_bytes(rows, cols) > (size_t)FP4MX_NOALLOC_SCRATCH_BYTES)
    return FP4MX_E_SCRATCH;
  if ((st = check_device())) return st;
  uint8_t* p = nullptr;
  if ((st = scratch_ptr(&p))) return st;
  // msedn_impl carves the fp32 v buffer and the maximum word from `p`; the
  // maximum is cleared by a kernel and every v is written before it is read
  return msedn_impl(x, rows, cols, ld, axis, clip_s, seed, gemm_id, rng_stream, codes, scales,
                    tensor_scale, eden_s, p, (hipStream_t)stream);
}

size_t fp4nv_linear_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  // two quantized operands per GEMM (live at once), the larger MS-EDEN
  // scratch and the larger FP8 staging; operands of the two GEMMs are reused
  const size_t q1 = nv_operand_bytes(m, n) + nv_operand_bytes(k, n);
  const size_t q2 = nv_operand_bytes(n, m) + nv_operand_bytes(k, m);
  const size_t ms = std::max(fp4nv_msedn_workspace_bytes(m, n), std::max(fp4nv_msedn_workspace_bytes(n, k),
                                                                        fp4nv_msedn_workspace_bytes(m, k)));
  const size_t gs = std::max(fp4nv_gemm_workspace_bytes(m, k, n), fp4nv_gemm_workspace_bytes(n, k, m));
  return std::max(q1, q2) + ms + gs + 512;
}

// One backward operand of the NVFP4 layer: from bf16 (column axis, i.e. the
// transposed operand) or from a saved NVFP4 operand (re-quantized).
struct NvSrc {
  const void* bf16;
  const uint8_t* codes;
  const uint8_t* scales;
  const float* g;
};

static int msedn_operand(const NvSrc& src, int64_t rows, int64_t cols, uint64_t seed,
                         uint32_t gemm_id, uint32_t stream, uint8_t* codes, uint8_t* scales,
                         float* ts, uint8_t* ws, hipStream_t s) {
  if (src.bf16)
    return msedn_impl(src.bf16, rows, cols, cols, FP4MX_AXIS_COL, 6.0f, seed, gemm_id, stream, codes,
                      scales, ts, nullptr, ws, s);
  Carver cv{ws};
  float* vbuf = reinterpret_cast<float*>(cv.take((size_t)rows * cols / 16 * sizeof(float)));
  uint32_t* gmax = reinterpret_cast<uint32_t*>(cv.take(4));
  hipError_t e = launch_msedn_requant(src.codes, src.scales, src.g, rows, cols, 6.0f, seed, gemm_id,
                                      stream, codes, scales, ts, nullptr, vbuf, gmax, s);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

// dX = gemm(MSEDEN(dY), MSEDEN(W^T)) (inner n), dW = gemm(MSEDEN(dY^T), MSEDEN(X^T)) (inner m).
static int nv_bwd_impl(const void* dy, const NvSrc& x, const NvSrc& w, int64_t m, int64_t n,
                       int64_t k, uint64_t seed, float* dx, float* dw, uint8_t* base, hipStream_t s) {
  int st;
  const float clip = 6.0f;
  const size_t qmax = std::max(nv_operand_bytes(m, n) + nv_operand_bytes(k, n),
                               nv_operand_bytes(n, m) + nv_operand_bytes(k, m));
  uint8_t* ms = base + qmax;
  uint8_t* gws = ms + std::max(fp4nv_msedn_workspace_bytes(m, n),
                               std::max(fp4nv_msedn_workspace_bytes(n, k), fp4nv_msedn_workspace_bytes(m, k)));
  {
    Carver cv{base};
    uint8_t* aq = cv.take((size_t)m * n / 2);
    uint8_t* as = cv.take((size_t)m * n / 16);
    float* ag = reinterpret_cast<float*>(cv.take(256));
    uint8_t* bq = cv.take((size_t)k * n / 2);
    uint8_t* bs = cv.take((size_t)k * n / 16);
    float* bg = reinterpret_cast<float*>(cv.take(256));
    if ((st = msedn_impl(dy, m, n, n, FP4MX_AXIS_ROW, clip, seed, 1, 5, aq, as, ag, nullptr, ms, s)))
      return st;
    if ((st = msedn_operand(w, n, k, seed, 1, 6, bq, bs, bg, ms, s))) return st;
    if ((st = nv_gemm_impl(aq, as, ag, bq, bs, bg, m, k, n, dx, k, gws, s))) return st;
  }
  {
    Carver cv{base};
    uint8_t* aq = cv.take((size_t)n * m / 2);
    uint8_t* as = cv.take((size_t)n * m / 16);
    float* ag = reinterpret_cast<float*>(cv.take(256));
    uint8_t* bq = cv.take((size_t)k * m / 2);
    uint8_t* bs = cv.take((size_t)k * m / 16);
    float* bg = reinterpret_cast<float*>(cv.take(256));
    if ((st = msedn_impl(dy, m, n, n, FP4MX_AXIS_COL, clip, seed, 2, 7, aq, as, ag, nullptr, ms, s)))
      return st;
    if ((st = msedn_operand(x, m, k, seed, 2, 8, bq, bs, bg, ms, s))) return st;
    if ((st = nv_gemm_impl(aq, as, ag, bq, bs, bg, n, k, m, dw, k, gws, s))) return st;
  }
  return FP4MX_OK;
}

int fp4nv_linear_bwd(const void* dy, const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                     uint64_t seed, float* dx, float* dw, void* ws, size_t ws_bytes, void* stream) {
  if (!dy || !x || !w || !dx || !dw) return FP4MX_E_NULL;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k) || m % 128 != 0 || n % 128 != 0) return FP4MX_E_SHAPE;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(w) || !aligned16(dx) || !aligned16(dw))
    return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_linear_bwd_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  const NvSrc xs{x, nullptr, nullptr, nullptr}, wsrc{w, nullptr, nullptr, nullptr};
  return nv_bwd_impl(dy, xs, wsrc, m, n, k, seed, dx, dw, static_cast<uint8_t*>(ws),
                     (hipStream_t)stream);
}

int fp4nv_msedn_requantize(const uint8_t* codes, const uint8_t* scales, const float* tensor_scale,
                           int64_t rows, int64_t cols, float clip_s, uint64_t seed, uint32_t gemm_id,
                           uint32_t rng_stream, uint8_t* out_codes, uint8_t* out_scales,
                           float* out_tensor_scale, float* eden_s, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!codes || !scales || !tensor_scale || !out_codes || !out_scales || !out_tensor_scale)
    return FP4MX_E_NULL;
  if (!dim_ok(rows) || !dim_ok(cols) || rows % 128 != 0) return FP4MX_E_SHAPE;
  if (!(clip_s > 0.0f) || !(clip_s < 1e30f)) return FP4MX_E_ARG;
  if (!aligned16(codes) || ((uintptr_t)scales & 1u) || ((uintptr_t)tensor_scale & 3u) ||
      !aligned16(out_codes) || ((uintptr_t)out_scales & 1u) || ((uintptr_t)out_tensor_scale & 3u) ||
      ((uintptr_t)eden_s & 3u))
    return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_msedn_workspace_bytes(rows, cols)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  int st = check_device();
  if (st) return st;
  Carver cv{static_cast<uint8_t*>(ws)};
  float* vbuf = reinterpret_cast<float*>(cv.take((size_t)rows * cols / 16 * sizeof(float)));
  uint32_t* gmax = reinterpret_cast<uint32_t*>(cv.take(4));
  hipError_t e = launch_msedn_requant(codes, scales, tensor_scale, rows, cols, clip_s, seed, gemm_id,
                                      rng_stream, out_codes, out_scales, out_tensor_scale, eden_s,
                                      vbuf, gmax, (hipStream_t)stream);
  return e == hipSuccess ? FP4MX_OK : hip_fail(e);
}

size_t fp4nv_ctx_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return nv_operand_bytes(m, k) + nv_operand_bytes(n, k);
}

static int nv_ctx_check(const fp4nv_ctx* ctx) {
  if (!ctx) return FP4MX_E_NULL;
  if (!ctx->xq_codes || !ctx->xq_scales || !ctx->xq_tensor_scale || !ctx->wq_codes ||
      !ctx->wq_scales || !ctx->wq_tensor_scale)
    return FP4MX_E_NULL;
  if (!aligned16(ctx->xq_codes) || !aligned16(ctx->wq_codes) || ((uintptr_t)ctx->xq_scales & 1u) ||
      ((uintptr_t)ctx->wq_scales & 1u) || ((uintptr_t)ctx->xq_tensor_scale & 3u) ||
      ((uintptr_t)ctx->wq_tensor_scale & 3u))
    return FP4MX_E_ALIGN;
  return FP4MX_OK;
}

size_t fp4nv_linear_fwd_ctx_workspace_bytes(int64_t m, int64_t n, int64_t k) {
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return 0;
  return 512 + fp4nv_gemm_workspace_bytes(m, n, k);
}

int fp4nv_linear_fwd_ctx(const void* x, const void* w, int64_t m, int64_t n, int64_t k, float* y,
                         const fp4nv_ctx* ctx, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !y) return FP4MX_E_NULL;
  int st = nv_ctx_check(ctx);
  if (st) return st;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k)) return FP4MX_E_SHAPE;
  if (!aligned16(x) || !aligned16(w) || !aligned16(y)) return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_linear_fwd_ctx_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  hipStream_t s = (hipStream_t)stream;
  Carver cv{static_cast<uint8_t*>(ws)};
  uint32_t* amax_x = reinterpret_cast<uint32_t*>(cv.take(4));
  uint32_t* amax_w = reinterpret_cast<uint32_t*>(cv.take(4));
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* wb = static_cast<const uint16_t*>(w);
  hipError_t e = launch_nv_amax(xb, m, k, k, amax_x, s);
  if (e == hipSuccess) e = launch_nv_amax(wb, n, k, k, amax_w, s);
  if (e == hipSuccess)
    e = launch_nv_quant(xb, m, k, k, 1, amax_x, ctx->xq_codes, ctx->xq_scales, ctx->xq_tensor_scale, s);
  if (e == hipSuccess)
    e = launch_nv_quant(wb, n, k, k, 1, amax_w, ctx->wq_codes, ctx->wq_scales, ctx->wq_tensor_scale, s);
  if (e != hipSuccess) return hip_fail(e);
  return nv_gemm_impl(ctx->xq_codes, ctx->xq_scales, ctx->xq_tensor_scale, ctx->wq_codes,
                      ctx->wq_scales, ctx->wq_tensor_scale, m, n, k, y, n, cv.p, s);
}

int fp4nv_linear_bwd_ctx(const void* dy, const fp4nv_ctx* ctx, int64_t m, int64_t n, int64_t k,
                         float* dx, float* dw, void* ws, size_t ws_bytes, void* stream) {
  if (!dy || !dx || !dw) return FP4MX_E_NULL;
  int st = nv_ctx_check(ctx);
  if (st) return st;
  if (!dim_ok(m) || !dim_ok(n) || !dim_ok(k) || m % 128 != 0 || n % 128 != 0) return FP4MX_E_SHAPE;
  if (!aligned16(dy) || !aligned16(dx) || !aligned16(dw)) return FP4MX_E_ALIGN;
  if (!ws || ws_bytes < fp4nv_linear_bwd_workspace_bytes(m, n, k)) return FP4MX_E_WORKSPACE;
  if (!aligned16(ws)) return FP4MX_E_ALIGN;
  if ((st = check_device())) return st;
  const NvSrc xs{nullptr, ctx->xq_codes, ctx->xq_scales, ctx->xq_tensor_scale};
  const NvSrc wsrc{nullptr, ctx->wq_codes, ctx->wq_scales, ctx->wq_tensor_scale};
  return nv_bwd_impl(dy, xs, wsrc, m, n, k, ctx->seed, dx, dw, static_cast<uint8_t*>(ws),
                     (hipStream_t)stream);
}

}  // extern "C"
