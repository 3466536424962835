// QuEST forward quantization and the Quartet backward in the forward-rotated
// basis, on gfx950.
//
// Sources: "Quartet: Native FP4 Training Can Be Optimal for Large Language
// Models" --
//  - "The Forward-Pass Quantization: QuEST in Detail": groups of 32 along the
//    GEMM inner dimension after the Hadamard transform, the group's standard
//    deviation about its mean, the clip factor c (its Gaussian RMSE optimum
//    is a constant passed in by the caller), clamp to [-c sigma, c sigma],
//    RTN, a clipping mask bit per element;
//  - "The GPU Kernel Implementation" Stage 1: the E8M0 scale encodes the
//    value the clip factor determines; mask bit set for clipped elements;
//  - the inverse Hadamard and clipping-mask correction:
//    dx = 16/9 H^-1(dx_q with the clipped entries zeroed);
//  - "The Complete Quartet Algorithm": the backward dequantizes the saved
//    W_q and X_q, transposes them, rotates them along the backward GEMM's
//    inner dimension and quantizes with SR(3/4 .).
//
// Per group (fp32 throughout, the same steps as the oracle):
//   E = floor(log2 max|y|) (0 for a zero group); z = y 2^-E;
//   mu = tree(z)/32; var = tree((z - mu)^2)/32; sigma_z = sqrt(var);
//   T_z = c sigma_z; code = min(max(floor(log2 T_z) + E + 125, 0), 254) (0 if
//   T_z = 0); T = T_z 2^E; |y| > T -> sign(y) T; E2M1 RNE of clamped / X with
//   X = 2^(code-127); mask bit = |y| > min(T, 6 X): the power-of-two scale
//   puts the grid's end 6 X anywhere in [0.75 T, 1.5 T), and elements beyond
//   it are clipped by the saturating rounding.
// tree = adjacent pairs summed level by level in index order.
//
// Design (MI355X):
//  - QuEST quantizer: one lane owns one 32-group (FWHT, statistics, clamp,
//    codes and its 32 mask bits all in registers); each wave stages its 64
//    groups through LDS so the HBM reads are 16-B coalesced.
//  - Re-quantizer: a 128 x 64 tile of the saved MXFP4 operand is decoded to
//    bf16 in LDS (MXFP4 values have at most two significant bits, so bf16
//    holds them exactly) and each lane quantizes one column group of 32 as the
//    transposed operand: 0.53 B read per element instead of 2 B of bf16.
//  - Mask + inverse RHT over fp32 rows: lane = 4 consecutive floats (16-B
//    coalesced), 8 lanes per group; butterflies h = 1, 2 in registers and
//    h = 4, 8, 16 across lanes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mx_internal.h"
#include "mx_device.h"

namespace fp4mx {
namespace {

// fp32 sum of 32 values: adjacent pairs, level by level.
__device__ __forceinline__ float tree32(const float (&v)[kGroup]) {
  float a[16], b[8], c[4], d[2];
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = a[2 * i] + a[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = b[2 * i] + b[2 * i + 1];
  d[0] = c[0] + c[1];
  d[1] = c[2] + c[3];
  return d[0] + d[1];
}

// floor(log2 |v|) from the encoding of a positive finite float (subnormals too).
__device__ __forceinline__ int floor_log2_bits(uint32_t b) {
  return b >= 0x800000u ? (int)(b >> 23) - 127 : (31 - __builtin_clz(b)) - 149;
}

// QuEST on one group held in registers: 4 code words, the scale byte and the
// 32 mask bits (bit i <-> element i).
__device__ __forceinline__ void quest_group(const float (&y)[kGroup], float clip,
                                            uint32_t (&w)[4], uint32_t& scale, uint32_t& mbits) {
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
    mbits = 0;
    return;
  }
  const int E = m ? floor_log2_bits(m) : 0;
  float z[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) z[i] = __builtin_ldexpf(y[i], -E);
  const float mu = tree32(z) * 0.03125f;
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float d = z[i] - mu;
    z[i] = d * d;
  }
  const float var = tree32(z) * 0.03125f;
  const float sig = __builtin_sqrtf(var);
  const float tz = clip * sig;
  // E8M0 byte of T, at most 254 (an infinite T_z, i.e. clip * sigma beyond
  // the fp32 range, encodes as 254 too: floor_log2_bits(inf) = 128)
  int code = 0;
  if (tz > 0.0f) code = min(max(floor_log2_bits(__float_as_uint(tz)) + E + 125, 0), 254);
  const float T = __builtin_ldexpf(tz, E);
  scale = (uint32_t)code;
  // the converter computes E2M1 RNE (saturating) of v / X, X = 2^(code-127);
  // code 0 passes the subnormal 2^-127
  const float X = __uint_as_float(code == 0 ? 0x00400000u : (uint32_t)code << 23);
  // the grid ends at 6 X (exact; +inf for code >= 253, where no finite
  // element reaches it): elements beyond min(T, 6 X) are clipped, by the
  // clamp or by the saturating rounding, and masked
  const float lim = __builtin_fminf(T, 6.0f * X);
  uint32_t mb = 0;
  float c[kGroup];
#pragma unroll
  for (int i = 0; i < kGroup; ++i) {
    const float a = __builtin_fabsf(y[i]);
    c[i] = a > T ? __builtin_copysignf(T, y[i]) : y[i];
    mb |= (a > lim ? 1u : 0u) << i;
  }
  mbits = mb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[8 * k + 0], c[8 * k + 1], X, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[8 * k + 2], c[8 * k + 3], X, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[8 * k + 4], c[8 * k + 5], X, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c[8 * k + 6], c[8 * k + 7], X, 3);
    w[k] = r;
  }
}

// ---------------------------------------------------------------------------
// QuEST row quantizer: thread = one group of one row; the wave's 64 groups
// (4 KB of bf16) are staged through LDS for coalesced reads.
// ---------------------------------------------------------------------------
constexpr int kWaveStage = 64 * 64 + 16 * 4;

__global__ __launch_bounds__(256) void quest_row_kernel(
    const uint16_t* __restrict__ x, int64_t cols, int64_t ld, uint32_t sign_mask, float clip,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t* __restrict__ mask,
    FastDiv gdiv, uint32_t ngroups) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[4 * kWaveStage];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint8_t* ws = stage + wave * kWaveStage;
  const uint32_t g_wave = blockIdx.x * 256u + (uint32_t)wave * 64u;
  if (g_wave >= ngroups) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)q * 64u + (uint32_t)lane;
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
  uint32_t wd[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)lane * 4u + (uint32_t)q;
    const u32x4 v = *reinterpret_cast<const u32x4*>(ws + chunk * 16 + (chunk / 64u) * 16);
    wd[4 * q + 0] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
  }
  float t[kGroup];
#pragma unroll
  for (int j = 0; j < 16; ++j) unpack_pair(flip_pair(wd[j], sign_mask, j), t[2 * j], t[2 * j + 1]);
  fwht32(t);
  uint32_t w[4], sc, mb;
  quest_group(t, clip, w, sc, mb);
  u32x4 o = {w[0], w[1], w[2], w[3]};
  *reinterpret_cast<u32x4*>(codes + row * (cols / 2) + grp * 16) = o;
  scales[row * gdiv.d + grp] = (uint8_t)sc;
  mask[row * gdiv.d + grp] = mb;
}

// ---------------------------------------------------------------------------
// Re-quantizer: saved MXFP4 operand [rows][cols] (groups along cols) ->
// transposed operand [cols][rows] with the RHT and the given rounding along
// rows.  Tile = 128 source rows x 64 source columns, decoded into LDS as bf16.
// ---------------------------------------------------------------------------
constexpr int kTileR = 128, kTileC = 64;
constexpr int kPitch = kTileC * 2 + 16;
constexpr int kCoutPitch = (kTileR / kGroup) * 16 + 16;  // output staging: 64 B + pad per column

// The two E2M1 codes of byte B of w, each times X = 2^(e-127), as a bf16
// pair word (low element in the low half).  gfx950's decode converter at
// scale 1.0 gives the exact signed grid values; the products with X are exact
// in fp32 and in bf16 (two significant bits), so the bf16 bits are the upper
// halves, taken with one byte permute.  A 0xFF scale (X = NaN) makes both
// values NaN, and the group then quantizes as a non-finite group.
template <int B>
__device__ __forceinline__ void deq_pair_bf16(uint32_t w, float X, uint32_t& out) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  const float a = v.x * X, b = v.y * X;
  out = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

template <int ROUND>
__global__ __launch_bounds__(256) void requant_tile_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
    int64_t cols, uint32_t sign_mask, uint32_t klo, uint32_t khi, uint8_t* __restrict__ out_codes,
    uint8_t* __restrict__ out_scales) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileR * kPitch];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * kTileR, c0 = (int64_t)blockIdx.y * kTileC;
  const int nr = (int)min<int64_t>(kTileR, rows - r0), nc = (int)min<int64_t>(kTileC, cols - c0);
  {
    // thread = one source group: row tid/2, group (c0/32) + (tid&1)
    const int r = tid >> 1, h = tid & 1;
    if (r < nr && h * kGroup < nc) {
      const int64_t row = r0 + r, grp = c0 / kGroup + h;
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(codes + row * (cols / 2) + grp * (kGroup / 2));
      const uint32_t e = scales[row * (cols / kGroup) + grp];
      const float X = e == 0xFFu ? __uint_as_float(0x7FC00000u)
                                 : __uint_as_float(e == 0 ? 0x00400000u : e << 23);
      const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t o[4];
        deq_pair_bf16<0>(cw[k], X, o[0]);
        deq_pair_bf16<1>(cw[k], X, o[1]);
        deq_pair_bf16<2>(cw[k], X, o[2]);
        deq_pair_bf16<3>(cw[k], X, o[3]);
        const u32x4 ov = {o[0], o[1], o[2], o[3]};
        *reinterpret_cast<u32x4*>(tile + r * kPitch + h * 64 + k * 16) = ov;
      }
    }
  }
  __syncthreads();
  // output codes and scales are staged per tile and stored as whole row
  // pieces (64 code bytes and one scale word per output row), as in the
  // column-axis quantizer
  __shared__ __attribute__((aligned(16))) uint8_t cout[kTileC * kCoutPitch];
  __shared__ __attribute__((aligned(16))) uint8_t cscl[kTileC * (kTileR / kGroup)];
  const int c = tid & 63, rg = tid >> 6;
  if (c < nc && rg * kGroup < nr) {
    float t[kGroup];
#pragma unroll
    for (int i = 0; i < kGroup; ++i) {
      uint32_t hb = *reinterpret_cast<const uint16_t*>(tile + (rg * kGroup + i) * kPitch + c * 2);
      t[i] = __uint_as_float((hb << 16) ^ (((sign_mask >> i) & 1u) << 31));
    }
    fwht32(t);
    const int64_t orow = c0 + c, grp = r0 / kGroup + rg;
    const uint64_t idx0 = (uint64_t)orow * (uint64_t)rows + (uint64_t)grp * kGroup;
    uint32_t w[4], sc;
    quant_group<ROUND>(t, (uint32_t)idx0, group_kmix(idx0, klo, khi), w, sc);
    u32x4 o = {w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(cout + c * kCoutPitch + rg * 16) = o;
    cscl[c * (kTileR / kGroup) + rg] = (uint8_t)sc;
  }
  __syncthreads();
  const int oc = tid >> 2, q = tid & 3;  // output row c0 + oc, its q-th group of this tile
  if (oc < nc && q * kGroup < nr) {
    *reinterpret_cast<u32x4*>(out_codes + (c0 + oc) * (rows / 2) + (r0 / kGroup + q) * 16) =
        *reinterpret_cast<const u32x4*>(cout + oc * kCoutPitch + q * 16);
    uint8_t* sp = out_scales + (c0 + oc) * (rows / kGroup) + r0 / kGroup;
    if (nr == kTileR && (rows / kGroup) % 4 == 0 && ((uintptr_t)out_scales & 3u) == 0) {
      if (q == 0) *reinterpret_cast<uint32_t*>(sp) = *reinterpret_cast<const uint32_t*>(cscl + oc * 4);
    } else {
      sp[q] = cscl[oc * (kTileR / kGroup) + q];
    }
  }
}

// ---------------------------------------------------------------------------
// C <- H^-1(C with masked entries zeroed), per 32-group along each row of an
// fp32 matrix; H^-1 y = s o (c * FWHT(y)).  Thread = 4 consecutive floats.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void unmask_irht_kernel(float* __restrict__ c, int64_t ldc,
                                                          const uint32_t* __restrict__ mask,
                                                          int64_t mask_words_per_row,
                                                          uint32_t sign_mask, FastDiv qdiv,
                                                          uint32_t nthreads) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  // all 64 lanes take part in the shuffles; only in-range lanes load and store
  const bool live = t < nthreads;
  const uint32_t tt = live ? t : 0u;
  const uint32_t row = fastdiv(tt, qdiv);
  const uint32_t q = tt - row * qdiv.d;  // quad of 4 floats within the row
  const uint32_t col = q * 4u, j = col & 31u;
  float4* p = reinterpret_cast<float4*>(c + (int64_t)row * ldc + col);
  float4 v = live ? *p : make_float4(0.f, 0.f, 0.f, 0.f);
  const uint32_t mb = live ? (mask[(int64_t)row * mask_words_per_row + (col >> 5)] >> j) & 0xFu : 0u;
  float a[4] = {(mb & 1u) ? 0.0f : v.x, (mb & 2u) ? 0.0f : v.y, (mb & 4u) ? 0.0f : v.z,
                (mb & 8u) ? 0.0f : v.w};
  // butterflies h = 1, 2 inside the lane
  {
    const float b0 = a[0] + a[1], b1 = a[0] - a[1], b2 = a[2] + a[3], b3 = a[2] - a[3];
    a[0] = b0 + b2; a[2] = b0 - b2; a[1] = b1 + b3; a[3] = b1 - b3;
  }
  // h = 4, 8, 16: partner lane differs in bit 0, 1, 2 of the lane's quad index
  const uint32_t lane_q = threadIdx.x & 7u;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const bool upper = (lane_q & (uint32_t)d) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float o = __shfl_xor(a[i], d, 64);
      a[i] = upper ? o - a[i] : a[i] + o;
    }
  }
  if (!live) return;
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = a[i] * kInvSqrt32;
    r[i] = __uint_as_float(__float_as_uint(u) ^ (((sign_mask >> (j + i)) & 1u) << 31));
  }
  *p = make_float4(r[0], r[1], r[2], r[3]);
}

}  // namespace

hipError_t launch_quest_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            uint32_t sign_mask, float clip, uint8_t* codes, uint8_t* scales,
                            uint8_t* mask, hipStream_t s) {
  const int64_t gpr = cols / kGroup;
  const FastDiv gd = make_fastdiv((uint32_t)gpr);
  const int64_t max_rows = ((int64_t)1 << 30) / gpr;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t ng = (uint32_t)(nr * gpr);
    hipLaunchKernelGGL(quest_row_kernel, dim3((ng + 255) / 256), dim3(256), 0, s, x + r0 * ld,
                       cols, ld, sign_mask, clip, codes + r0 * (cols / 2), scales + r0 * gpr,
                       reinterpret_cast<uint32_t*>(mask + r0 * (cols / 8)), gd, ng);
  }
  return hipGetLastError();
}

hipError_t launch_requant(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                          int rounding, uint32_t sign_mask, RngKey key, uint8_t* out_codes,
                          uint8_t* out_scales, hipStream_t s) {
  dim3 grid((unsigned)((rows + kTileR - 1) / kTileR), (unsigned)((cols + kTileC - 1) / kTileC));
  if (rounding == FP4MX_ROUND_RTN)
    hipLaunchKernelGGL(requant_tile_kernel<FP4MX_ROUND_RTN>, grid, dim3(256), 0, s, codes, scales,
                       rows, cols, sign_mask, key.lo, key.hi, out_codes, out_scales);
  else
    hipLaunchKernelGGL(requant_tile_kernel<FP4MX_ROUND_SR>, grid, dim3(256), 0, s, codes, scales,
                       rows, cols, sign_mask, key.lo, key.hi, out_codes, out_scales);
  return hipGetLastError();
}

hipError_t launch_unmask_irht(float* c, int64_t rows, int64_t cols, int64_t ldc,
                              const uint8_t* mask, uint32_t sign_mask, hipStream_t s) {
  const int64_t qpr = cols / 4;  // float quads per row
  const FastDiv qd = make_fastdiv((uint32_t)qpr);
  const int64_t max_rows = ((int64_t)1 << 30) / qpr;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t nt = (uint32_t)(nr * qpr);
    hipLaunchKernelGGL(unmask_irht_kernel, dim3((nt + 255) / 256), dim3(256), 0, s, c + r0 * ldc,
                       ldc, reinterpret_cast<const uint32_t*>(mask + r0 * (cols / 8)), cols / 32,
                       sign_mask, qd, nt);
  }
  return hipGetLastError();
}

}  // namespace fp4mx
