// Per-group device arithmetic shared by the MXFP4 kernels (quant_mx.hip,
// quest.hip): the in-register block-32 FWHT, bf16 unpacking and sign flips,
// the counter hash of the SR draws, and the MX group quantizer (E8M0 scale
// from the group maximum; RTN by the hardware converter, SR by exact fp32
// comparisons of the draw with the position between grid points).
//
// Sources: "Quartet: Native FP4 Training Can Be Optimal for Large Language
// Models" -- "The Hadamard Transform: Why It Is Necessary and How It Is
// Implemented" (blocks of 32, 1/sqrt(32), sign flips), "The GPU Kernel
// Implementation" Stage 1 (group maximum -> E8M0, FP4 downcast), "The 3/4
// rescaling factor"; "Quartet II ..." -- "NVFP4 Format and Standard
// Stochastic Rounding" (E2M1 grid, SR probability).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mx_internal.h"

namespace fp4mx {
namespace {

constexpr int kGroup = 32;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;  // fl32(1/sqrt(32)), bits 0x3E3504F3

__device__ __forceinline__ uint32_t fmix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// In-register unnormalised FWHT (Sylvester order, stages h = 1..16), then the
// 1/sqrt(32) factor.  Every operation is a single fp32 add, sub or mul.
__device__ __forceinline__ void fwht32(float (&t)[kGroup]) {
#pragma unroll
  for (int h = 1; h < kGroup; h <<= 1) {
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      if (i & h) continue;
      float a = t[i], b = t[i + h];
      t[i] = a + b;
      t[i + h] = a - b;
    }
  }
#pragma unroll
  for (int i = 0; i < kGroup; ++i) t[i] = t[i] * kInvSqrt32;
}

// bf16 pair word (element 2j low, 2j+1 high) -> two floats, exact.
__device__ __forceinline__ void unpack_pair(uint32_t w, float& lo, float& hi) {
  lo = __uint_as_float(w << 16);
  hi = __uint_as_float(w & 0xFFFF0000u);
}

// Sign-flip mask for bf16 pair word j of a group.
__device__ __forceinline__ uint32_t pair_sign(uint32_t mask, int j) {
  return (((mask >> (2 * j)) & 1u) << 15) | (((mask >> (2 * j + 1)) & 1u) << 31);
}

// Quantize one group held in registers.  Writes 4 code words (8 nibbles
// each, element 8k+2i in the low nibble of byte i of word k) and the scale
// byte.  `idx_lo` is lo32 of the output index of element 0 and `kmix` the
// per-group stream constant lo32(key) ^ fmix32(hi32(index) ^ hi32(key)).
template <int ROUND>
__device__ __forceinline__ void quant_group(const float (&y)[kGroup], uint32_t idx_lo,
                                            uint32_t kmix, uint32_t (&w)[4],
                                            uint32_t& scale) {
  // group max |y| with NaN propagation (IEEE maximum): non-finite iff the
  // result's magnitude bits reach the Inf pattern
  float am = __builtin_elementwise_maximum(__builtin_fabsf(y[30]), __builtin_fabsf(y[31]));
#pragma unroll
  for (int i = 0; i < 30; i += 3)
    am = __builtin_elementwise_maximum(
        __builtin_elementwise_maximum(am, __builtin_fabsf(y[i])),
        __builtin_elementwise_maximum(__builtin_fabsf(y[i + 1]), __builtin_fabsf(y[i + 2])));
  const uint32_t m = __float_as_uint(am) & 0x7FFFFFFFu;
  if (m >= 0x7F800000u) {  // Inf or NaN in the group
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = 0;
    scale = 0xFFu;
    return;
  }
  const int code = max((int)(m >> 23) - 2, 0);
  scale = (uint32_t)code;
  if constexpr (ROUND == FP4MX_ROUND_RTN) {
    // v_cvt_scalef32_pk_fp4_f32 computes E2M1 RNE (saturating) of y / X with
    // X = 2^(code-127); code 0 passes the subnormal fp32 2^-127, which the
    // converter takes as that power of two.
    const float X = __uint_as_float(code == 0 ? 0x00400000u : (uint32_t)code << 23);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t r = 0;
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * k + 0], y[8 * k + 1], X, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * k + 2], y[8 * k + 3], X, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * k + 4], y[8 * k + 5], X, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, y[8 * k + 6], y[8 * k + 7], X, 3);
      w[k] = r;
    }
  } else {
    // f = 0.75 * 2^(127-code), exactly representable for code <= 254.
    const float f = __builtin_ldexpf(0.75f, 127 - code);
    // The group's first index is a multiple of 32, so element i hashes
    // idx_lo ^ i, and the first xor-shift of fmix32 touches only the group
    // part: h1 ^ i equals that step's result for element i.
    const uint32_t h0 = idx_lo ^ kmix;
    const uint32_t h1 = h0 ^ (h0 >> 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * k + j;
        const float v = __builtin_fabsf(y[i]) * f;  // 0 <= v < 6
        uint32_t r = (h1 ^ (uint32_t)i) * 0x85EBCA6Bu;
        r ^= r >> 13;
        r *= 0xC2B2AE35u;
        r ^= r >> 16;
        // Grid position: with e = max(floor(log2 v), 0), w = v 2^(1-e) lies in
        // [0, 4) and element code floor(w) + 2e is the grid point below v;
        // the gap to the next one maps to [0, 1) as frac(w) exactly (powers
        // of two only).  Up iff (r >> 8) 2^-24 < frac(w), i.e. the
        // probability (v - a) / (b - a) with a 24-bit uniform.
        const uint32_t eb = max(__float_as_uint(v) >> 23, 127u);  // 127 + e
        const float w = __builtin_ldexpf(v, 128 - (int)eb);
        const float fr = __builtin_amdgcn_fractf(w);  // w - floor(w), exact for w >= 0
        const uint32_t up = (float)(r >> 8) < fr * 0x1p24f ? 1u : 0u;
        uint32_t q = (uint32_t)w + 2u * (eb - 127u) + up;  // truncation = floor for w >= 0
        q |= (__float_as_uint(y[i]) >> 28) & 8u;
        word |= q << (4 * j);
      }
      w[k] = word;
    }
  }
}

__device__ __forceinline__ uint32_t group_kmix(uint64_t idx0, uint32_t key_lo, uint32_t key_hi) {
  return key_lo ^ fmix32((uint32_t)(idx0 >> 32) ^ key_hi);
}

}  // namespace
}  // namespace fp4mx
