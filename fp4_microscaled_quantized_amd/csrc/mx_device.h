// Per-group device arithmetic shared by the MXFP4 kernels (quant_mx.hip,
// quest.hip; nvfp4.hip's SR baseline takes the hash and the SR converter
// helpers): the in-register block-32 FWHT, bf16 unpacking and sign flips,
// the counter hash of the SR draws, and the MX group quantizer (E8M0 scale
// from the group maximum; RTN and SR by the hardware converters, SR taking
// the top 22 bits of each element's draw).
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

// Pair word w with the RHT sign flips of pair j applied, as one xor whose
// result the unpacking then shifts and masks (the empty asm keeps the
// compiler from splitting the xor into a half per element, which costs two
// three-operand ops and two register copies of the constants per word).
__device__ __forceinline__ uint32_t flip_pair(uint32_t w, uint32_t mask, int j) {
  w ^= pair_sign(mask, j);
  asm("" : "+v"(w));
  return w;
}

// fmix32 of element i's counter from h1 (the group's counter after the
// first xor-shift, see quant_group).
__device__ __forceinline__ uint32_t sr_bits(uint32_t h1, int i) {
  uint32_t r = (h1 ^ (uint32_t)i) * 0x85EBCA6Bu;
  r ^= r >> 13;
  r *= 0xC2B2AE35u;
  return r ^ (r >> 16);
}

// gfx950's SR converter v_cvt_scalef32_sr_pk_fp4_f32 (scale 1.0) rounds the
// pair (a, b) into byte B of its destination and keeps the other bytes.  It
// truncates an element's position inside its E2M1 gap to 22 bits, adds the
// top 22 bits of the seed (of the seed shifted left by one for b) and keeps
// the carry; the sign is the sign of the input.  Seeded with r, element a
// rounds up iff floor(p * 2^22) + (r >> 10) >= 2^22, p being the position in
// the gap, and +0 in slot b gives nibble 0.  The compiler's builtin for this
// instruction does not keep the destination's other bytes, hence the asm
// with a read-write operand.
template <int B>
__device__ __forceinline__ void cvt_sr_fp4(uint32_t& acc, float a, float b, uint32_t seed) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  if constexpr (B == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(acc) : "v"(v), "v"(seed));
  else if constexpr (B == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]"
        : "+v"(acc) : "v"(v), "v"(seed));
  else if constexpr (B == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]"
        : "+v"(acc) : "v"(v), "v"(seed));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]"
        : "+v"(acc) : "v"(v), "v"(seed));
}

// SR of the element pair (v0, v1) with draws r0, r1 into byte B: each
// element is converted on its own in slot a (the slot that reads its draw
// as is), v0's nibble into the low nibble of byte B of `lo`, v1's into the
// low nibble of byte B of `hi`; the caller moves `hi` up by four bits.  One
// seed per pair would hand the two elements draws sharing 21 of 22 bits.
template <int B>
__device__ __forceinline__ void sr_pair(uint32_t& lo, uint32_t& hi, float v0, float v1,
                                        uint32_t r0, uint32_t r1) {
  cvt_sr_fp4<B>(lo, v0, 0.0f, r0);
  cvt_sr_fp4<B>(hi, v1, 0.0f, r1);
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
      // Even elements go to the low nibble of byte b of `lo`, odd ones to
      // the low nibble of byte b of `hi` (shifted into the high nibble
      // below); the other element of each converted pair is +0, nibble 0.
      // The four conversions write every byte of lo and hi, so their
      // starting contents do not matter: an empty asm defines them without
      // an instruction.
      uint32_t lo, hi;
      asm volatile("" : "=v"(lo), "=v"(hi));
      sr_pair<0>(lo, hi, y[8 * k + 0] * f, y[8 * k + 1] * f, sr_bits(h1, 8 * k + 0),
                 sr_bits(h1, 8 * k + 1));
      sr_pair<1>(lo, hi, y[8 * k + 2] * f, y[8 * k + 3] * f, sr_bits(h1, 8 * k + 2),
                 sr_bits(h1, 8 * k + 3));
      sr_pair<2>(lo, hi, y[8 * k + 4] * f, y[8 * k + 5] * f, sr_bits(h1, 8 * k + 4),
                 sr_bits(h1, 8 * k + 5));
      sr_pair<3>(lo, hi, y[8 * k + 6] * f, y[8 * k + 7] * f, sr_bits(h1, 8 * k + 6),
                 sr_bits(h1, 8 * k + 7));
      w[k] = lo | (hi << 4);
    }
  }
}

__device__ __forceinline__ uint32_t group_kmix(uint64_t idx0, uint32_t key_lo, uint32_t key_hi) {
  return key_lo ^ fmix32((uint32_t)(idx0 >> 32) ^ key_hi);
}

}  // namespace
}  // namespace fp4mx
