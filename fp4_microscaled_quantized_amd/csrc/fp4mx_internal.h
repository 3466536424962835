// Internal declarations shared by the HIP translation units of libfp4mx.
// Not part of the public ABI (see include/fp4mx.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mx.h"

namespace fp4mx {

// ---------------------------------------------------------------------------
// Host-side RNG key derivation (SplitMix64 output function; the per-element
// generator fmix32 runs on the device).
// ---------------------------------------------------------------------------
inline uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

struct RngKey {
  uint32_t lo, hi;  // the two halves of splitmix64(seed ^ (stream << 32))
};

inline RngKey make_key(uint64_t seed, uint32_t stream) {
  uint64_t k = splitmix64(seed ^ ((uint64_t)stream << 32));
  return RngKey{(uint32_t)k, (uint32_t)(k >> 32)};
}

// 32-bit unsigned division by a launch constant: q = (umulhi(n, mul) + n) >> sh
// (Granlund-Montgomery round-up method), exact for n < 2^31.
struct FastDiv {
  uint32_t mul, sh, d;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t sh = 0;
  while ((1ull << sh) < d) ++sh;
  const uint64_t mul = ((1ull << 32) * ((1ull << sh) - d)) / d + 1;
  return FastDiv{(uint32_t)mul, sh, d};
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
  return (__umulhi(n, f.mul) + n) >> f.sh;
}

// Quantizer launch description for one output operand.
struct QuantOut {
  int rounding;        // FP4MX_ROUND_RTN / FP4MX_ROUND_SR
  uint32_t sign_mask;  // RHT signs (ignored when the transform is off)
  RngKey key;          // SR stream key
  uint8_t* codes;
  uint8_t* scales;
};

// Launchers (defined in quant_mx.hip / gemm_mx.hip / nvfp4.hip).  They
// assume validated arguments and return the launch's hipError_t.
hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            bool hadamard, const QuantOut& o, hipStream_t s);
hipError_t launch_quant_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                             bool hadamard, const QuantOut* row_out, const QuantOut* col_out,
                             hipStream_t s);
// The dual tile quantizer (RHT) on two operands a and b, row RTN and column SR
// for both (the linear layer's forward), in one launch; other modes, or grids
// too large for one launch, take two.
hipError_t launch_quant_tile_pair(const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ld_a,
                                  const QuantOut& ra, const QuantOut& ca, const uint16_t* xb,
                                  int64_t rows_b, int64_t cols_b, int64_t ld_b,
                                  const QuantOut& rb, const QuantOut& cb, hipStream_t s);
hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                          const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha,
                          float* c, int64_t ldc, hipStream_t s);

// QuEST and the re-quantizer (csrc/quest.hip).
hipError_t launch_quest_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            uint32_t sign_mask, float clip, uint8_t* codes, uint8_t* scales,
                            uint8_t* mask, hipStream_t s);
hipError_t launch_requant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int rounding, uint32_t sign_mask, RngKey key, uint8_t* out_codes,
                          uint8_t* out_scales, hipStream_t s);
hipError_t launch_unmask_irht(float* c, int64_t rows, int64_t cols, int64_t ldc,
                              const uint8_t* mask, uint32_t sign_mask, hipStream_t s);

// FP4 GEMM whose epilogue zeroes the entries masked in cmask ([m][n/32] words,
// bit j = column 32g + j) and applies the inverse block-32 RHT (sign_mask)
// along each row of C.
hipError_t launch_mx_gemm_irht(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                               const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha,
                               float* c, int64_t ldc, const uint8_t* cmask, uint32_t sign_mask,
                               hipStream_t s);
hipError_t launch_mx_gemm_bf16(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                               const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha,
                               uint16_t* c, int64_t ldc, hipStream_t s);

// MS-EDEN, two passes (csrc/msedn.hip).  vbuf: fp32 per output 16-group;
// gmax: one uint32 (global max of vbuf).
hipError_t launch_msedn(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                        float clip_s, uint64_t seed, uint32_t gemm_id, uint32_t stream,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale, float* eden_s,
                        float* vbuf, uint32_t* gmax, hipStream_t s);
// MS-EDEN of the transpose of a saved NVFP4 operand [rows][cols] (rows % 128 == 0).
hipError_t launch_msedn_requant(const uint8_t* qcodes, const uint8_t* qscales, const float* qg,
                                int64_t rows, int64_t cols, float clip_s, uint64_t seed,
                                uint32_t gemm_id, uint32_t stream, uint8_t* codes, uint8_t* scales,
                                float* tensor_scale, float* eden_s, float* vbuf, uint32_t* gmax,
                                hipStream_t s);
void msedn_sign_words(uint64_t seed, uint32_t gemm_id, uint32_t (&w)[4]);

hipError_t launch_nv_sr(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                        const uint32_t* amax_bits, uint32_t key_lo, uint32_t key_hi,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale, hipStream_t s);

hipError_t launch_nv_amax(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                          uint32_t* amax_bits, hipStream_t s);
hipError_t launch_nv_quant(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                           int use_46, const uint32_t* amax_bits, uint8_t* codes,
                           uint8_t* scales, float* tensor_scale, hipStream_t s);
hipError_t launch_nv_stage(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                           int64_t cols, uint8_t* fp8, uint8_t* e8, hipStream_t s);
hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                           const uint8_t* bs, const float* ga, const float* gb, int64_t m,
                           int64_t n, int64_t k, float* c, int64_t ldc, hipStream_t s);

}  // namespace fp4mx
