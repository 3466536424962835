/*
 * fp4mx.h -- C ABI of libfp4mx.so, a fully-FP4 quantized linear layer for
 * AMD MI355X (gfx950): block-32 randomized Hadamard transform (RHT) fused with
 * MXFP4 quantization, the FP4 GEMMs of a linear layer's forward and backward
 * pass, and an NVFP4 forward variant.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, w, dy, codes, scales, c, y, dx, dw, ws and tensor_scale
 *   are DEVICE pointers owned by the caller.  The library never allocates or
 *   frees memory and only enqueues work on `stream` (a hipStream_t; NULL =
 *   the default stream).  Calls are asynchronous: outputs are valid once the
 *   stream has been synchronised.  No state carries from one call to the
 *   next except per-device caches of two device queries (the architecture
 *   check and the compute-unit count), each written once per device and safe
 *   to read from any thread, and the static device scratch array that
 *   fp4nv_msedn_quantize_noalloc works in (it keeps the last call's
 *   contents; that entry point's comment has the rules).
 * - Device check: a current device other than gfx950 gives FP4MX_E_DEVICE.
 *   The environment variable FP4MX_DEVICE_ARCH, when set to another
 *   architecture name, makes every compute call return FP4MX_E_DEVICE after
 *   argument validation and before any HIP call (a host-only test of the
 *   refusal); unset or "gfx950", it has no effect.
 * - Every call returns an fp4mx_status.  Arguments are validated on the host
 *   before any launch; on a validation error nothing is enqueued.  A HIP
 *   launch error returns FP4MX_E_HIP and fp4mx_last_hip_error() gives the HIP
 *   code (per calling thread).
 * - Shapes: every dimension must be a positive multiple of 32 and at most
 *   FP4MX_MAX_DIM = 2^21; a GEMM output's leading dimension ldc is at most
 *   FP4MX_MAX_DIM too (FP4MX_E_SHAPE otherwise).
 *   Pointers must be 16-byte aligned and leading dimensions (in elements) a
 *   multiple of 8 (FP4MX_E_ALIGN).  The device must be gfx950 (FP4MX_E_DEVICE).
 * - bf16 inputs are row-major with leading dimension `ld` (elements).
 *
 * MXFP4 operand layout (written by the quantizers, read by fp4mx_gemm)
 * -------------------------------------------------------------------
 *   codes  uint8 [rows][cols/2]  element 2j in the low nibble of byte j and
 *          2j+1 in the high nibble; a nibble is E2M1: bit 3 sign, bits 2..0
 *          index {0, 0.5, 1, 1.5, 2, 3, 4, 6};
 *   scales uint8 [rows][cols/32] E8M0 (value 2^(byte-127); 0xFF marks a
 *          group that held a non-finite value after the transform).
 *   Every group of 32 consecutive elements along a row shares one scale:
 *   rows are the GEMM's M (or N) index, cols its inner K index ("K-major").
 *   Sources: "Quartet: Native FP4 Training Can Be Optimal for Large Language
 *   Models" -- "The QuEST Forward-Pass Quantization" (groups of 32 along K,
 *   M x ceil(K/32) scales) and "The GPU Kernel Implementation" (Stage 1, E8M0
 *   scale from the group maximum; Stage 2 block-scaled GEMM); "Quartet II:
 *   Accurate LLM Pre-Training in NVFP4 ..." -- "NVFP4 Format and Standard
 *   Stochastic Rounding" (the E2M1 value set).
 *
 * Quantization arithmetic (bit-exact contract)
 * --------------------------------------------
 *   RHT: per 32-group, x'_j = -x_j if bit j of sign_mask is set; radix-2 fp32
 *   butterflies (a,b) -> (a+b, a-b) on pairs (i, i+h), h = 1,2,4,8,16; then
 *   y_i = t_i * fl32(1/sqrt(32)).  Scale byte e = max(biased_exponent(max|y|)
 *   - 2, 0), i.e. 2^(e-127) = 2^(floor(log2 max|y|) - 2).
 *   RTN: E2M1 round-to-nearest-even of y * 2^(127-e), saturating at 6.
 *   SR:  v = fl32(y * (0.75 * 2^(127-e))) (|v| < 6 always); with a <= |v| < b
 *        adjacent grid points and p = (|v|-a)/(b-a), take b iff
 *        floor(p * 2^22) + (r >> 10) >= 2^22 (P(b) = p for |v| >= 1, within
 *        2^-22 below it under 1); the sign is v's, so a negative value that
 *        rounds to 0 gives -0.  Here
 *        r = fmix32(lo32(i) ^ lo32(k) ^ fmix32(hi32(i) ^ hi32(k))),
 *        k = splitmix64(seed ^ (rng_stream << 32)) and i = row * cols_out + col
 *        is the element's index in the OUTPUT operand.
 *   Sources: "Quartet: Native FP4 Training ..." -- "The Hadamard Transform:
 *   Why It Is Necessary and How It Is Implemented" (block-32 Hadamard,
 *   1/sqrt(g) normalisation, random sign flips, explicit seed), "The 3/4
 *   rescaling factor" (SR(3/4 G) on the backward pass, 16/9 after the GEMM);
 *   "Quartet II ..." -- "NVFP4 Format and Standard Stochastic Rounding" (SR
 *   rounds up with probability (v-a)/(b-a)), "MS-EDEN" Step 1 (one random
 *   sign pattern for all blocks of a tensor).
 */
#ifndef FP4MX_H
#define FP4MX_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define FP4MX_API __attribute__((visibility("default")))
#else
#define FP4MX_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Largest accepted dimension (rows, cols, m, n, k) and GEMM output ldc. */
#define FP4MX_MAX_DIM 2097152

typedef enum {
  FP4MX_OK = 0,
  FP4MX_E_NULL = -1,      /* a required pointer is NULL                       */
  FP4MX_E_SHAPE = -2,     /* a dimension <= 0, not a multiple of 32, or above
                             FP4MX_MAX_DIM                                    */
  FP4MX_E_ALIGN = -3,     /* pointer not 16-B aligned / ld not multiple of 8  */
  FP4MX_E_ARG = -4,       /* bad enum value or argument combination           */
  FP4MX_E_WORKSPACE = -5, /* workspace NULL or smaller than required          */
  FP4MX_E_DEVICE = -6,    /* current device is not gfx950                     */
  FP4MX_E_HIP = -7,       /* a HIP call failed; see fp4mx_last_hip_error()    */
  FP4MX_E_SCRATCH = -8    /* the input needs more scratch than the static
                             buffer of a no-allocation entry point holds      */
} fp4mx_status;

enum { FP4MX_ROUND_RTN = 0, FP4MX_ROUND_SR = 1 };
enum { FP4MX_AXIS_ROW = 0, FP4MX_AXIS_COL = 1 };

/* Human-readable name of a status code (static string, never NULL). */
FP4MX_API const char* fp4mx_status_string(int status);

/* HIP error code of this thread's last FP4MX_E_HIP (0 if none). */
FP4MX_API int fp4mx_last_hip_error(void);

/* Host helper: the 32-bit RHT sign mask shared by both operands of GEMM
 * `gemm_id` (0 = forward Y, 1 = input gradient dX, 2 = weight gradient dW):
 * lo32(splitmix64(seed ^ ((0x5100 + gemm_id) << 32))).  Pure host function. */
FP4MX_API uint32_t fp4mx_sign_mask(uint64_t seed, uint32_t gemm_id);

/* MXFP4-quantize one GEMM operand without a transform (y = x).
 *   x       bf16 [rows][ld], the first `cols` columns are used.
 *   axis    FP4MX_AXIS_ROW: groups of 32 along each row; outputs
 *             codes [rows][cols/2], scales [rows][cols/32].
 *           FP4MX_AXIS_COL: the operand is x^T (groups of 32 down each
 *             column); outputs codes [cols][rows/2], scales [cols][rows/32].
 *   rounding FP4MX_ROUND_RTN or FP4MX_ROUND_SR (SR implies the 3/4 prescale).
 *   seed, rng_stream: the SR draw (ignored for RTN).
 * Source: "Quartet: Native FP4 Training ..." -- "The GPU Kernel
 * Implementation", Stage 1 (fused quantization kernel). */
FP4MX_API int fp4mx_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                   int rounding, uint64_t seed, uint32_t rng_stream, uint8_t* codes,
                   uint8_t* scales, void* stream);

/* As fp4mx_quantize, with the block-32 RHT (sign mask `sign_mask`) applied
 * along the grouped dimension first.  sign_mask = 0 gives the plain
 * (deterministic) Hadamard transform.
 * Source: "Quartet: Native FP4 Training ..." -- "The Hadamard Transform ..."
 * and Stage 1 of "The GPU Kernel Implementation" (transform, scale and
 * downcast fused in one kernel). */
FP4MX_API int fp4mx_hadamard_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld,
                            int axis, int rounding, uint32_t sign_mask, uint64_t seed,
                            uint32_t rng_stream, uint8_t* codes, uint8_t* scales,
                            void* stream);

/* One read of x, two RHT-quantized outputs: the ROW-axis operand (groups
 * along rows; row_* outputs [rows][cols/2], [rows][cols/32]) and the COL-axis
 * operand (x^T; col_* outputs [cols][rows/2], [cols][rows/32]), each with its
 * own rounding, sign mask and RNG stream (same seed).
 * Used for the forward pass (X, W: row RTN + col SR context) and for dY
 * (row SR + col SR).  Source: as fp4mx_hadamard_quantize; the pairing follows
 * "The Complete Quartet Algorithm" (the backward GEMMs need both dY and dY^T). */
FP4MX_API int fp4mx_hadamard_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                 int row_rounding, uint32_t row_sign_mask,
                                 uint32_t row_rng_stream, int col_rounding,
                                 uint32_t col_sign_mask, uint32_t col_rng_stream,
                                 uint64_t seed, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, void* stream);

/* C = alpha * deq(A) * deq(B)^T with fp32 accumulation and fp32 output.
 *   A: MXFP4 operand [m][k] (a_codes [m][k/2], a_scales [m][k/32]),
 *   B: MXFP4 operand [n][k] (b_codes [n][k/2], b_scales [n][k/32]),
 *   C: fp32 [m][ldc], ldc >= n, ldc a multiple of 4.
 * Source: "Quartet: Native FP4 Training ..." -- "The GPU Kernel
 * Implementation", Stage 2 (D = C + (A x SFA)(B x SFB), FP32 accumulator). */
FP4MX_API int fp4mx_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
               const uint8_t* b_scales, int64_t m, int64_t n, int64_t k, float alpha,
               float* c, int64_t ldc, void* stream);

/* The same GEMM with a bf16 output: C[i][j] = bf16_RNE(fp32 result), i.e.
 * exactly the value fp4mx_gemm writes, rounded to nearest even (NaN stays
 * NaN).  C: bf16 bits [m][ldc], 16-B aligned, ldc >= n, ldc a multiple of 8.
 * Arguments and errors otherwise as fp4mx_gemm.  Halves the output traffic
 * for callers whose layer outputs are bf16 tensors.
 * Source: the layer graphs of "Quartet II ..." -- "The Complete Quartet II
 * Computation Graph" (linear-layer outputs and gradients flow as
 * high-precision bf16 tensors between the FP4 GEMMs); the rounding step is
 * this library's design. */
FP4MX_API int fp4mx_gemm_bf16(const uint8_t* a_codes, const uint8_t* a_scales,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t m,
                              int64_t n, int64_t k, float alpha, uint16_t* c, int64_t ldc,
                              void* stream);

/* Saved forward context for the backward pass: the SR-quantized, RHT'd
 * transposed operands X^T [k][m] (groups along m) and W^T [k][n] (groups
 * along n), plus the seed.  All four buffers are caller-owned device memory:
 * xt_codes k*m/2, xt_scales k*m/32, wt_codes k*n/2, wt_scales k*n/32 bytes.
 * Source: "Quartet: Native FP4 Training ..." -- "The Complete Quartet
 * Algorithm", Context Save (quantized tensors are saved instead of bf16). */
typedef struct {
  uint8_t* xt_codes;
  uint8_t* xt_scales;
  uint8_t* wt_codes;
  uint8_t* wt_scales;
  uint64_t seed;
} fp4mx_ctx;

/* Workspace bytes needed by fp4mx_linear_fwd / fp4mx_linear_bwd. */
FP4MX_API size_t fp4mx_linear_workspace_bytes(int64_t m, int64_t n, int64_t k);
/* Bytes of the four context buffers together. */
FP4MX_API size_t fp4mx_ctx_bytes(int64_t m, int64_t n, int64_t k);

/* Forward of the fully-FP4 linear layer Y = X W^T.
 *   x bf16 [m][k] (ld k), w bf16 [n][k] (ld k), y fp32 [m][n].
 *   Both operands: RHT along k with fp4mx_sign_mask(seed, 0), RTN.
 *   ctx != NULL: also writes the backward operands from the same read of x
 *   and w: X^T with SR, mask fp4mx_sign_mask(seed, 2), RNG stream 4; W^T with
 *   SR, mask fp4mx_sign_mask(seed, 1), RNG stream 2; ctx->seed must equal seed.
 *   ws: fp4mx_linear_workspace_bytes(m, n, k) bytes of device memory.
 * Source: "Quartet: Native FP4 Training ..." -- "The Complete Quartet
 * Algorithm", forward pass; "Quartet II ..." -- "The Complete Quartet II
 * Computation Graph" (RHT on the inner dimension of both operands, same seed). */
FP4MX_API int fp4mx_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                     uint64_t seed, float* y, const fp4mx_ctx* ctx, void* ws,
                     size_t ws_bytes, void* stream);

/* Backward of the fully-FP4 linear layer.
 *   dy bf16 [m][n] (ld n) -> dx fp32 [m][k] = 16/9 Q(dY) Q(W^T)^T (inner n,
 *   mask 1, dY rows SR with RNG stream 1) and dw fp32 [n][k] = 16/9 Q(dY^T)
 *   Q(X^T)^T (inner m, mask 2, dY^T SR with RNG stream 3).
 * Source: "Quartet: Native FP4 Training ..." -- "The Complete Quartet
 * Algorithm", backward pass, and "The 3/4 rescaling factor"; "Quartet II ..."
 * -- "The Complete Quartet II Computation Graph" (no inverse transform). */
FP4MX_API int fp4mx_linear_bwd(const void* dy, const fp4mx_ctx* ctx, int64_t m, int64_t n,
                     int64_t k, float* dx, float* dw, void* ws, size_t ws_bytes,
                     void* stream);

/* fp4mx_linear_fwd and fp4mx_linear_bwd with bf16 outputs: y [m][n], dx
 * [m][k] and dw [n][k] hold bf16 bits, each the round-to-nearest-even of the
 * fp32 value the fp32 entry point writes (the GEMMs' bf16 epilogue, as in
 * fp4mx_gemm_bf16).  Arguments, context, workspace and errors as the fp32
 * forms; outputs 16-B aligned.  These let a bf16 training graph keep every
 * step of the layer in the library (no separate cast pass).
 * Source: "Quartet II ..." -- "The Complete Quartet II Computation Graph"
 * (the layer's outputs and gradients are bf16 tensors between the FP4
 * GEMMs); the rounding step is this library's design. */
FP4MX_API int fp4mx_linear_fwd_bf16(const void* x, const void* w, int64_t m, int64_t n,
                                    int64_t k, uint64_t seed, uint16_t* y, const fp4mx_ctx* ctx,
                                    void* ws, size_t ws_bytes, void* stream);
FP4MX_API int fp4mx_linear_bwd_bf16(const void* dy, const fp4mx_ctx* ctx, int64_t m, int64_t n,
                                    int64_t k, uint16_t* dx, uint16_t* dw, void* ws,
                                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * QuEST forward and the Quartet backward in the forward-rotated basis
 * (source: "Quartet: Native FP4 Training Can Be Optimal for Large Language
 * Models" -- "The Forward-Pass Quantization: QuEST in Detail", Stage 1 of
 * "The GPU Kernel Implementation", the inverse Hadamard and clipping-mask
 * correction, "The Complete Quartet Algorithm").
 * Clipping masks: uint8 [rows][cols/8], element j of a row at bit j%8 of byte
 * j/8; bit 1 = the element was clipped.  Mask pointers must be 4-B aligned.
 * ------------------------------------------------------------------------ */

/* QuEST MXFP4 quantization along rows after the block-32 RHT (sign_mask):
 * per 32-group, sigma = standard deviation about the group mean (evaluated on
 * the group scaled by 2^-E, 2^E <= max|y| < 2^(E+1)), T = clip * sigma, E8M0
 * scale e = floor(log2 T) - 2 (0 when T = 0, at most 254), codes = E2M1 RNE
 * of the group clamped to [-T, T] at scale X = 2^(e-127), mask bit =
 * |y| > min(T, 6 X) (clipped by the clamp or by the grid's end).  A
 * non-finite group gets scale 0xFF, codes 0 and mask 0.  clip must be finite
 * and > 0; the Gaussian RMSE optimum of the page's objective is 2.922475.
 *   x bf16 [rows][ld]; codes [rows][cols/2]; scales [rows][cols/32];
 *   mask [rows][cols/8].  Errors as fp4mx_quantize; E_ARG for a bad clip. */
FP4MX_API int fp4mx_quest_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, float clip,
                         uint32_t sign_mask, uint8_t* codes, uint8_t* scales, uint8_t* mask,
                         void* stream);

/* Re-quantize a saved MXFP4 operand for the backward pass: dequantize A
 * [rows][cols] (codes [rows][cols/2], scales [rows][cols/32], groups along
 * cols), transpose, apply the block-32 RHT (sign_mask) along rows and quantize
 * with `rounding` (SR includes the 3/4 prescale): out_codes [cols][rows/2],
 * out_scales [cols][rows/32].  SR draw of output element (r, c): index
 * r * rows + c of stream rng_stream.  Dequantized values are exact (0xFF
 * scales give NaN groups -> 0xFF).  Errors as fp4mx_quantize. */
FP4MX_API int fp4mx_requantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int rounding, uint32_t sign_mask, uint64_t seed, uint32_t rng_stream,
                     uint8_t* out_codes, uint8_t* out_scales, void* stream);

/* In place on fp32 c [rows][ldc] (first cols columns): per 32-group along each
 * row, zero the entries whose mask bit is 1, then apply the inverse of the
 * forward RHT, x = s o (fl32(1/sqrt(32)) * FWHT(y)).  ldc multiple of 4. */
FP4MX_API int fp4mx_unmask_inverse_hadamard(float* c, int64_t rows, int64_t cols, int64_t ldc,
                                  const uint8_t* mask, uint32_t sign_mask, void* stream);

/* fp4mx_gemm followed by fp4mx_unmask_inverse_hadamard on its output, in one
 * kernel: C = H^-1((alpha * deq(A) deq(B)^T) with the entries masked in
 * `mask` zeroed), per 32-column group of each row of C, H^-1 inverting the
 * forward RHT with sign_mask.  mask: uint8 [m][n/8] (4-B aligned), layout and
 * sense as above.  The transform runs in the GEMM's epilogue (C never takes
 * the intermediate value), with the same fp32 operations in the same order as
 * the two-call form, so the results are identical.  Errors as fp4mx_gemm;
 * E_NULL for a null mask, E_ALIGN for a misaligned one. */
FP4MX_API int fp4mx_gemm_unmask_irht(const uint8_t* a_codes, const uint8_t* a_scales,
                           const uint8_t* b_codes, const uint8_t* b_scales, int64_t m, int64_t n,
                           int64_t k, float alpha, float* c, int64_t ldc, const uint8_t* mask,
                           uint32_t sign_mask, void* stream);

/* Saved QuEST forward context: X_q [m][k] (codes, scales), W_q [n][k], the
 * clipping masks M_x [m][k/8] and M_w [n][k/8], and the seed.  Caller-owned
 * device memory; fp4mx_quest_ctx_bytes gives the total of the six buffers. */
typedef struct {
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  uint8_t* wq_codes;
  uint8_t* wq_scales;
  uint8_t* x_mask;
  uint8_t* w_mask;
  uint64_t seed;
} fp4mx_quest_ctx;

FP4MX_API size_t fp4mx_quest_ctx_bytes(int64_t m, int64_t n, int64_t k);
/* Workspace of fp4mx_quest_linear_bwd: Q(dY), Q(dY^T), Q(W_q^T), Q(X_q^T). */
FP4MX_API size_t fp4mx_quest_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Forward: X_q, M_x = QuEST(RHT X), W_q, M_w = QuEST(RHT W) along k with
 * fp4mx_sign_mask(seed, 0), written into ctx (required, ctx->seed == seed);
 * y fp32 [m][n] = X_q W_q^T. */
FP4MX_API int fp4mx_quest_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                           float clip, uint64_t seed, float* y, const fp4mx_quest_ctx* ctx,
                           void* stream);

/* Backward in the forward-rotated basis:
 *   dX = 16/9 H^-1(Q(dY) Q(W_q^T)^T with M_x entries zeroed)  [m][k],
 *   dW = 16/9 H^-1(Q(dY^T) Q(X_q^T)^T with M_w entries zeroed) [n][k];
 * Q(dY): rows SR, mask fp4mx_sign_mask(seed, 1), stream 1; Q(dY^T): SR, mask
 * 2, stream 3; W_q re-quantized along n (mask 1, stream 2); X_q along m (mask
 * 2, stream 4); H^-1 inverts the forward rotation (mask 0). */
FP4MX_API int fp4mx_quest_linear_bwd(const void* dy, const fp4mx_quest_ctx* ctx, int64_t m, int64_t n,
                           int64_t k, float* dx, float* dw, void* ws, size_t ws_bytes,
                           void* stream);

/* ------------------------------------------------------------------------
 * NVFP4 forward variant (sources: "Quartet II ..." -- "NVFP4 Format and
 * Standard Stochastic Rounding", "MS-EDEN" Step 2 (global scale amax/(s*256)),
 * "Forward Pass Design: ... Four-Over-Six").
 * Operand layout: codes uint8 [rows][cols/2] (nibbles as MXFP4), scales uint8
 * [rows][cols/16] E4M3 (OCP E4M3FN), one fp32 tensor scale g; element value
 * q * s16 * g.  Inputs must be finite.
 *   g = fl32(max|x| / 1536); per 16-group and c in {6, 4}:
 *   s_c = E4M3_RNE(fl32(max|x_b| / fl32(c*g))), q = E2M1_RNE(fl32(x / fl32(s_c*g)))
 *   (0 when s_c*g == 0), block error = pairwise fp32 sum of squared fp32
 *   residuals; candidate 4 is kept iff its error is strictly lower (use_46 = 1).
 * ------------------------------------------------------------------------ */

/* Bytes of workspace fp4nv_quantize46 needs (amax reduction). */
FP4MX_API size_t fp4nv_quantize_workspace_bytes(int64_t rows, int64_t cols);

/* NVFP4 RTN (+4/6) quantization of x bf16 [rows][ld] along rows.
 * tensor_scale: device pointer to one float (written).  cols % 32 == 0. */
FP4MX_API int fp4nv_quantize46(const void* x, int64_t rows, int64_t cols, int64_t ld, int use_46,
                     uint8_t* codes, uint8_t* scales, float* tensor_scale, void* ws,
                     size_t ws_bytes, void* stream);

/* C = deq(A) deq(B)^T (fp32 [m][ldc]) for NVFP4 operands A [m][k], B [n][k].
 * Each 32-element K block is staged to FP8 E4M3: e_blk = max exponent of the
 * block's two E4M3 scales - 5 (0 if both are 0), element = E4M3_RNE(q * s16 *
 * 2^-e_blk), and fed to the scaled FP8 MFMA with the E8M0 block scale
 * 2^e_blk; the epilogue multiplies by fl32(g_A * g_B). */
FP4MX_API int fp4nv_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_tensor_scale,
               const uint8_t* b_codes, const uint8_t* b_scales, const float* b_tensor_scale,
               int64_t m, int64_t n, int64_t k, float* c, int64_t ldc, void* ws,
               size_t ws_bytes, void* stream);

/* Workspace bytes for fp4nv_gemm (FP8-staged operands) and fp4nv_linear_fwd. */
FP4MX_API size_t fp4nv_gemm_workspace_bytes(int64_t m, int64_t n, int64_t k);
FP4MX_API size_t fp4nv_linear_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Y = X W^T with both operands NVFP4 RTN + 4/6 quantized (x [m][k], w [n][k]
 * bf16 with ld k; y fp32 [m][n]). */
FP4MX_API int fp4nv_linear_fwd(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                     float* y, void* ws, size_t ws_bytes, void* stream);

/* Standard NVFP4 stochastic rounding (the unbiased baseline of "Quartet II
 * ..." -- "NVFP4 Format and Standard Stochastic Rounding", 16/17 guard):
 *   c = fl32(96/17) (6 * 16/17 rounded once); g = fl(max|x| / fl(c * 448)) (written to tensor_scale);
 *   s16 = E4M3_RNE(fl(max|x_16| / fl(g * c))); v = fl(x / fl(s16 * g)), |v| <= 6;
 *   q = SR onto E2M1 by the 22-bit carry rule of the MXFP4 quantizers: with
 *   r the counter hash of (seed, rng_stream) at index row * cols + col and
 *   p = (|v| - a)/(b - a), b is taken iff floor(p 2^22) + (r >> 10) >= 2^22.
 * Layout and workspace as fp4nv_quantize46 (rows along which groups run). */
FP4MX_API int fp4nv_sr_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld,
                      uint64_t seed, uint32_t rng_stream, uint8_t* codes, uint8_t* scales,
                      float* tensor_scale, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Unbiased NVFP4 quantization for the backward pass: MS-EDEN.
 * Source: "Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved
 * Unbiased Gradient Estimation" -- "MS-EDEN: Microscaling EDEN" (RHT over
 * chunks of 128, RTN NVFP4 with clip factor s, EDEN correction S per chunk,
 * group scales SR_FP8(S * scale)), "The EDEN Technique and Its Precision
 * Bottleneck" (S = <x, x> / <x, Q(x)>), "Kernel Speedups on NVIDIA Blackwell
 * Hardware" (post hoc range alignment in two passes).
 * Per 128-chunk along the operand's inner dimension (rows of x for AXIS_ROW,
 * columns of x for AXIS_COL, whose output is the transposed operand):
 *   y = fl(H (s o x) c), c = fl32(1/sqrt(128)), 128-bit sign pattern of
 *   (seed, gemm_id); p = E8M3_RNE(fl(max|y_16| / clip_s)) (4 significant bits);
 *   q = E2M1_RNE_sat(fl(y / p)); S = fl(sum y^2 / sum y * q p) (pairwise fp32);
 *   v = fl(S p); tensor scale g = 2^k, k least with max v 2^-k <= 256;
 *   group scale = SR_E4M3(v 2^-k) with u = (r >> 8) 2^-24 from the counter hash
 *   of (seed, rng_stream) at the scale's flat index in the output operand.
 * Output operand layout as fp4nv_quantize46 (codes [R][C/2], E4M3 [R][C/16],
 * one fp32 g in device memory).  E[q * scale * g] = S * q * p.
 * ------------------------------------------------------------------------ */

/* Workspace bytes for fp4nv_msedn_quantize (fp32 v per 16-group + max). */
FP4MX_API size_t fp4nv_msedn_workspace_bytes(int64_t rows, int64_t cols);

/* MS-EDEN of x bf16 [rows][ld].  axis ROW: cols % 128 == 0, output [rows][cols];
 * axis COL: rows % 128 == 0, output [cols][rows].  clip_s > 0 (6 = no clip
 * beyond E8M3 rounding).  eden_s: optional fp32 [out_rows][out_cols/128]
 * receiving S (NULL to skip).  Errors as fp4mx_quantize. */
FP4MX_API int fp4nv_msedn_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                         float clip_s, uint64_t seed, uint32_t gemm_id, uint32_t rng_stream,
                         uint8_t* codes, uint8_t* scales, float* tensor_scale, float* eden_s,
                         void* ws, size_t ws_bytes, void* stream);

/* Size of the library's static device scratch (per GPU, held until the
 * process ends) used by fp4nv_msedn_quantize_noalloc: 32 MiB + 256 B. */
#define FP4MX_NOALLOC_SCRATCH_BYTES 33554688

/* fp4nv_msedn_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The scratch (fp32 v per output 16-group
 * plus the tensor maximum, fp4nv_msedn_workspace_bytes(rows, cols) bytes) is
 * a file-scope device array of FP4MX_NOALLOC_SCRATCH_BYTES in the library;
 * inputs needing more get FP4MX_E_SCRATCH (rows * cols up to 2^27
 * elements fit, e.g. 16384 x 8192).  The call allocates nothing.  Every call
 * on a GPU shares that GPU's one array: calls that overlap on one GPU (two
 * streams, or two threads) race and give undefined results; calls ordered on
 * one stream are safe.  Arguments, outputs and the other errors as
 * fp4nv_msedn_quantize. */
FP4MX_API int fp4nv_msedn_quantize_noalloc(const void* x, int64_t rows, int64_t cols, int64_t ld,
                                           int axis, float clip_s, uint64_t seed, uint32_t gemm_id,
                                           uint32_t rng_stream, uint8_t* codes, uint8_t* scales,
                                           float* tensor_scale, float* eden_s, void* stream);

/* Workspace bytes for fp4nv_linear_bwd. */
FP4MX_API size_t fp4nv_linear_bwd_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* NVFP4 backward of Y = X W^T with MS-EDEN operands (clip 6), per "The
 * Complete Quartet II Computation Graph" (RHT on the inner dimension of each
 * GEMM, no inverse, no rescale):
 *   dX [m][k] = gemm(MSEDEN_row(dY; gemm 1, stream 5), MSEDEN_col(W; gemm 1, stream 6))
 *   dW [n][k] = gemm(MSEDEN_col(dY; gemm 2, stream 7), MSEDEN_col(X; gemm 2, stream 8))
 * dy bf16 [m][n], x bf16 [m][k], w bf16 [n][k]; m % 128 == 0, n % 128 == 0,
 * k % 32 == 0.  The GEMMs are fp4nv_gemm (FP8 staging). */
FP4MX_API int fp4nv_linear_bwd(const void* dy, const void* x, const void* w, int64_t m, int64_t n,
                     int64_t k, uint64_t seed, float* dx, float* dw, void* ws, size_t ws_bytes,
                     void* stream);

/* ------------------------------------------------------------------------
 * Re-quantization of the saved forward operands for the NVFP4 backward
 * (source: "Quartet II ..." -- "The Complete Quartet II Computation Graph":
 * de-quantize the saved Q(X), Q(W), transpose, RHT on the inner dimension with
 * a seed shared by both operands of a GEMM, MS-EDEN, NVFP4 GEMM, no inverse
 * RHT; "Forward Pass Design: The Representation-Requantization Trade-Off").
 * ------------------------------------------------------------------------ */

/* MS-EDEN of the transpose of a saved NVFP4 operand A [rows][cols] (codes
 * [rows][cols/2], E4M3 scales [rows][cols/16], device fp32 tensor scale): the
 * values fl32(q * s16 * g) (one rounding of the exact product) are transposed
 * and quantized as fp4nv_msedn_quantize does along rows of the transpose
 * (128-chunks along the original rows; rows % 128 == 0): out_codes
 * [cols][rows/2], out_scales [cols][rows/16], out_tensor_scale, optional
 * eden_s [cols][rows/128].  ws: fp4nv_msedn_workspace_bytes(rows, cols). */
FP4MX_API int fp4nv_msedn_requantize(const uint8_t* codes, const uint8_t* scales,
                           const float* tensor_scale, int64_t rows, int64_t cols, float clip_s,
                           uint64_t seed, uint32_t gemm_id, uint32_t rng_stream,
                           uint8_t* out_codes, uint8_t* out_scales, float* out_tensor_scale,
                           float* eden_s, void* ws, size_t ws_bytes, void* stream);

/* Saved forward operands of the NVFP4 layer: Q(X) [m][k] and Q(W) [n][k]
 * (codes, E4M3 scales, device fp32 tensor scale each), and the backward seed.
 * Caller-owned device memory; fp4nv_ctx_bytes bounds the six buffers. */
typedef struct {
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_tensor_scale;
  uint8_t* wq_codes;
  uint8_t* wq_scales;
  float* wq_tensor_scale;
  uint64_t seed;
} fp4nv_ctx;

FP4MX_API size_t fp4nv_ctx_bytes(int64_t m, int64_t n, int64_t k);
FP4MX_API size_t fp4nv_linear_fwd_ctx_workspace_bytes(int64_t m, int64_t n, int64_t k);

/* Forward as fp4nv_linear_fwd (RTN + 4/6, FP8-staged GEMM), with Q(X) and
 * Q(W) written into ctx for the backward. */
FP4MX_API int fp4nv_linear_fwd_ctx(const void* x, const void* w, int64_t m, int64_t n, int64_t k,
                         float* y, const fp4nv_ctx* ctx, void* ws, size_t ws_bytes, void* stream);

/* Backward from the saved operands: dX = gemm(MSEDEN(dY), MSEDEN(deq(Q(W))^T))
 * (inner n; GEMM id 1, streams 5 and 6), dW = gemm(MSEDEN(dY^T),
 * MSEDEN(deq(Q(X))^T)) (inner m; GEMM id 2, streams 7 and 8), seed ctx->seed,
 * clip 6.  m % 128 == n % 128 == 0; ws: fp4nv_linear_bwd_workspace_bytes. */
FP4MX_API int fp4nv_linear_bwd_ctx(const void* dy, const fp4nv_ctx* ctx, int64_t m, int64_t n,
                         int64_t k, float* dx, float* dw, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4MX_H */
