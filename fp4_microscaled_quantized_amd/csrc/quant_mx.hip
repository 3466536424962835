// Fused block-32 randomized Hadamard transform + MXFP4 quantization for gfx950.
//
// Sources (what is computed):
//  "Quartet: Native FP4 Training Can Be Optimal for Large Language Models":
//   - "The Hadamard Transform: Why It Is Necessary and How It Is Implemented":
//     blocks of 32 along the GEMM inner dimension, Sylvester Hadamard with a
//     1/sqrt(32) normalisation, random sign flips, the O(g log g) FWHT;
//   - "The GPU Kernel Implementation", Stage 1: transform, group maximum,
//     E8M0 scale and FP4 downcast fused in one kernel with one global read;
//   - "The 3/4 rescaling factor": SR(3/4 G) on the backward pass.
//  "Quartet II: Accurate LLM Pre-Training in NVFP4 ...", "NVFP4 Format and
//   Standard Stochastic Rounding": the E2M1 grid and the SR probability.
//
// Design (MI355X):
//  - One lane owns one 32-element group: the whole FWHT (5 butterfly stages)
//    runs in registers with no cross-lane traffic, the group maximum is a
//    register reduction, and the lane writes its 16 code bytes with one 16-B
//    store.  Row-axis groups are read straight from HBM with 16-B loads.
//  - Column-axis groups (the transposed operand) go through a 128 x 64 bf16
//    LDS tile: one coalesced read of the tile feeds both the row-axis and the
//    column-axis quantizer, so the dual kernel reads each input byte once.
//  - RTN uses gfx950's v_cvt_scalef32_pk_fp4_f32, which computes E2M1
//    round-to-nearest-even of x / scale with saturation (two elements per
//    instruction, the sign included); SR is done in integer/fp32 arithmetic.
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
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * k + j;
        const float v = __builtin_fabsf(y[i]) * f;  // 0 <= v < 6
        const uint32_t vb = __float_as_uint(v);
        const uint32_t r = fmix32((idx_lo + (uint32_t)i) ^ kmix);
        // round up iff (r >> 8) * 2^-24 < (v - a) / (b - a):
        //  v in [1, 6):   (v-a)/(b-a) = frac22 / 2^22  ->  (r >> 10) < frac22
        //  v in [0.5, 1): (v-a)/(b-a) = frac23 / 2^23  ->  (r >> 9)  < frac23
        //  v < 0.5:       (v-a)/(b-a) = 2v             ->  (r >> 8) < v * 2^25
        const bool hi = vb >= 0x3F800000u;
        const uint32_t lim = vb & (hi ? 0x3FFFFFu : 0x7FFFFFu);
        const uint32_t rr = r >> (hi ? 10 : 9);
        const uint32_t base = hi ? (vb >> 22) - 252u : 1u;
        const uint32_t qa = base + (rr < lim ? 1u : 0u);
        const uint32_t qb = (float)(r >> 8) < v * 0x1p25f ? 1u : 0u;
        uint32_t q = vb >= 0x3F000000u ? qa : qb;
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

// ---------------------------------------------------------------------------
// Row axis: thread = one group of one row.  Each wave stages its 64 groups
// (4 KB of bf16) through LDS so the global reads are fully coalesced 16-B
// loads (lane l reads bytes 16 l + 1024 q), then each lane reads back its own
// 64-byte group.  Groups are numbered row-major over (row, group-in-row).
// ---------------------------------------------------------------------------
constexpr int kWaveStage = 64 * 64 + 16 * 4;  // 64 groups of 64 B, 16-B pad per 16 groups

template <bool HAD, int ROUND>
__global__ __launch_bounds__(256) void quant_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint32_t key_lo, uint32_t key_hi, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, FastDiv gdiv, uint32_t ngroups) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[4 * kWaveStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* ws = stage + wave * kWaveStage;
  const uint32_t g_wave = blockIdx.x * 256u + (uint32_t)wave * 64u;  // first group of the wave
  if (g_wave >= ngroups) return;
  // cooperative coalesced load: chunk q*64 + lane (16 B) of the wave's 64 groups
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)q * 64u + (uint32_t)lane;  // 0..255
    const uint32_t g = g_wave + chunk / 4u;
    if (g < ngroups) {
      const uint32_t row32 = fastdiv(g, gdiv);
      const int64_t grp = g - row32 * gdiv.d;
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          x + (int64_t)row32 * ld + grp * kGroup + (chunk & 3u) * 8));
      *reinterpret_cast<u32x4*>(ws + chunk * 16 + (chunk / 64u) * 16) = v;
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  const uint32_t g = g_wave + (uint32_t)lane;
  if (g >= ngroups) return;
  const uint32_t row32 = fastdiv(g, gdiv);
  const int64_t row = row32, grp = g - row32 * gdiv.d;
  const int64_t gpr = gdiv.d;
  uint32_t wd[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)lane * 4u + (uint32_t)q;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ws + chunk * 16 + (chunk / 64u) * 16);
    wd[4 * q + 0] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
  }
  float t[kGroup];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t w = wd[j];
    if constexpr (HAD) w ^= pair_sign(sign_mask, j);
    unpack_pair(w, t[2 * j], t[2 * j + 1]);
  }
  if constexpr (HAD) fwht32(t);
  const uint64_t idx0 = (uint64_t)row * (uint64_t)cols + (uint64_t)grp * kGroup;
  uint32_t w[4], sc;
  quant_group<ROUND>(t, (uint32_t)idx0, group_kmix(idx0, key_lo, key_hi), w, sc);
  u32x4 o = {w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4*>(codes + row * (cols / 2) + grp * 16) = o;
  scales[row * gpr + grp] = (uint8_t)sc;
}

// ---------------------------------------------------------------------------
// LDS tile kernel: 128 rows x 64 columns of bf16, read once from HBM.
//   ROW_ROUND >= 0: row-axis groups (thread = row t/2, group t%2);
//   COL_ROUND >= 0: column-axis groups (thread = column t%64, row group t/64),
//                   written as the transposed operand.
// ---------------------------------------------------------------------------
constexpr int kTileR = 128, kTileC = 64;
constexpr int kPitch = kTileC * 2 + 16;  // bytes per LDS row (padding vs bank conflicts)

template <bool HAD, int ROW_ROUND, int COL_ROUND>
__global__ __launch_bounds__(256) void quant_tile_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    uint32_t row_mask, uint32_t row_klo, uint32_t row_khi, uint8_t* __restrict__ row_codes,
    uint8_t* __restrict__ row_scales, uint32_t col_mask, uint32_t col_klo, uint32_t col_khi,
    uint8_t* __restrict__ col_codes, uint8_t* __restrict__ col_scales) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileR * kPitch];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kTileR, c0 = (int64_t)blockIdx.y * kTileC;
  const int nr = (int)min<int64_t>(kTileR, rows - r0), nc = (int)min<int64_t>(kTileC, cols - c0);

  // Coalesced load: 1024 chunks of 16 B (8 elements), 4 per thread.
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int id = tid + 256 * it;
    const int r = id >> 3, ch = id & 7;
    if (r < nr && ch * 8 < nc) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(x + (r0 + r) * ld + c0 + ch * 8));
      *reinterpret_cast<u32x4*>(tile + r * kPitch + ch * 16) = v;
    }
  }
  __syncthreads();

  if constexpr (ROW_ROUND >= 0) {
    const int r = tid >> 1, gq = tid & 1;
    if (r < nr && gq * kGroup < nc) {
      uint32_t wd[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(tile + r * kPitch + gq * 64 + q * 16);
        wd[4 * q + 0] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
      }
      float t[kGroup];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        uint32_t w = wd[j];
        if constexpr (HAD) w ^= pair_sign(row_mask, j);
        unpack_pair(w, t[2 * j], t[2 * j + 1]);
      }
      if constexpr (HAD) fwht32(t);
      const int64_t row = r0 + r, grp = c0 / kGroup + gq;
      const uint64_t idx0 = (uint64_t)row * (uint64_t)cols + (uint64_t)grp * kGroup;
      uint32_t w[4], sc;
      quant_group<ROW_ROUND>(t, (uint32_t)idx0, group_kmix(idx0, row_klo, row_khi), w, sc);
      u32x4 o = {w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(row_codes + row * (cols / 2) + grp * 16) = o;
      row_scales[row * (cols / kGroup) + grp] = (uint8_t)sc;
    }
  }

  if constexpr (COL_ROUND >= 0) {
    const int c = tid & 63, rg = tid >> 6;
    if (c < nc && rg * kGroup < nr) {
      float t[kGroup];
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        uint32_t h = *reinterpret_cast<const uint16_t*>(tile + (rg * kGroup + i) * kPitch + c * 2);
        uint32_t b = h << 16;
        if constexpr (HAD) b ^= ((col_mask >> i) & 1u) << 31;
        t[i] = __uint_as_float(b);
      }
      if constexpr (HAD) fwht32(t);
      const int64_t orow = c0 + c, grp = r0 / kGroup + rg;
      const uint64_t idx0 = (uint64_t)orow * (uint64_t)rows + (uint64_t)grp * kGroup;
      uint32_t w[4], sc;
      quant_group<COL_ROUND>(t, (uint32_t)idx0, group_kmix(idx0, col_klo, col_khi), w, sc);
      u32x4 o = {w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4*>(col_codes + orow * (rows / 2) + grp * 16) = o;
      col_scales[orow * (rows / kGroup) + grp] = (uint8_t)sc;
    }
  }
}

template <bool HAD, int RR, int CR>
hipError_t tile_launch(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                       const QuantOut* ro, const QuantOut* co, hipStream_t s) {
  dim3 grid((unsigned)((rows + kTileR - 1) / kTileR), (unsigned)((cols + kTileC - 1) / kTileC));
  QuantOut z{};
  const QuantOut& R = ro ? *ro : z;
  const QuantOut& C = co ? *co : z;
  hipLaunchKernelGGL((quant_tile_kernel<HAD, RR, CR>), grid, dim3(256), 0, s, x, rows, cols, ld,
                     R.sign_mask, R.key.lo, R.key.hi, R.codes, R.scales, C.sign_mask, C.key.lo,
                     C.key.hi, C.codes, C.scales);
  return hipGetLastError();
}

template <bool HAD>
hipError_t tile_dispatch(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                         const QuantOut* ro, const QuantOut* co, hipStream_t s) {
  const int rr = ro ? ro->rounding : -1, cr = co ? co->rounding : -1;
#define FP4MX_TILE_CASE(A, B) \
  if (rr == (A) && cr == (B)) return tile_launch<HAD, A, B>(x, rows, cols, ld, ro, co, s);
  FP4MX_TILE_CASE(-1, 0) FP4MX_TILE_CASE(-1, 1)
  FP4MX_TILE_CASE(0, -1) FP4MX_TILE_CASE(1, -1)
  FP4MX_TILE_CASE(0, 0) FP4MX_TILE_CASE(0, 1) FP4MX_TILE_CASE(1, 0) FP4MX_TILE_CASE(1, 1)
#undef FP4MX_TILE_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            bool hadamard, const QuantOut& o, hipStream_t s) {
  const int64_t groups = rows * (cols / kGroup);
  if (groups >= (1ll << 31)) return launch_quant_tile(x, rows, cols, ld, hadamard, &o, nullptr, s);
  const FastDiv gd = make_fastdiv((uint32_t)(cols / kGroup));
  const unsigned nblk = (unsigned)((groups + 255) / 256);
  const uint32_t ng = (uint32_t)groups;
  if (hadamard) {
    if (o.rounding == FP4MX_ROUND_RTN)
      hipLaunchKernelGGL((quant_row_kernel<true, 0>), dim3(nblk), dim3(256), 0, s, x, rows, cols,
                         ld, o.sign_mask, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng);
    else
      hipLaunchKernelGGL((quant_row_kernel<true, 1>), dim3(nblk), dim3(256), 0, s, x, rows, cols,
                         ld, o.sign_mask, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng);
  } else {
    if (o.rounding == FP4MX_ROUND_RTN)
      hipLaunchKernelGGL((quant_row_kernel<false, 0>), dim3(nblk), dim3(256), 0, s, x, rows, cols,
                         ld, 0u, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng);
    else
      hipLaunchKernelGGL((quant_row_kernel<false, 1>), dim3(nblk), dim3(256), 0, s, x, rows, cols,
                         ld, 0u, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng);
  }
  return hipGetLastError();
}

hipError_t launch_quant_tile(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                             bool hadamard, const QuantOut* row_out, const QuantOut* col_out,
                             hipStream_t s) {
  if (!row_out && !col_out) return hipErrorInvalidValue;
  return hadamard ? tile_dispatch<true>(x, rows, cols, ld, row_out, col_out, s)
                  : tile_dispatch<false>(x, rows, cols, ld, row_out, col_out, s);
}

}  // namespace fp4mx
