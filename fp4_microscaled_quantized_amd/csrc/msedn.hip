// MS-EDEN: unbiased NVFP4 quantization for the backward pass, in two passes
// (post hoc range alignment), on gfx950.
//
// Sources: "Quartet II: Accurate LLM Pre-Training in NVFP4 by Improved Unbiased
// Gradient Estimation" -- "MS-EDEN: Microscaling EDEN" (RHT over chunks of
// 128, RTN NVFP4 with a clip factor s, EDEN correction S per chunk, group
// scales replaced by SR_FP8(S * scale)), "The EDEN Technique and Its Precision
// Bottleneck" (S = <x, x> / <x, Q(x)>), and "Kernel Speedups on NVIDIA
// Blackwell Hardware" (post hoc range alignment: pass 1 quantizes against
// extended-range pseudo-scales and finds the global range and the
// corrections; pass 2 reads only the scales, shifts them into FP8 range and
// rounds them stochastically).
//
// What is computed (per 128-chunk of the GEMM inner dimension):
//   y = fl(H (s o x) * c), c = fl32(1/sqrt(128)), butterflies h = 1 .. 64;
//   p_g = 4-significant-bit RNE of fl(max|y_g| / s) (E8M3 pseudo-scale);
//   q_i = E2M1 RNE (saturating) of fl(y_i / p_g); r_i = val(q_i) * p_g;
//   S = fl(sum fl(z_i^2) / sum fl(z_i t_i)), z = y 2^-E, t = r 2^-E with
//   2^E <= max|y| < 2^(E+1) over the chunk (pairwise trees in index order);
//   v_g = fl(S * p_g); pass 2: tensor scale 2^k (least k with max v * 2^-k
//   <= 256) and group scale SR_E4M3(v_g * 2^-k) with a counter-hash uniform.
//
// Design (MI355X): four lanes own one chunk, 32 elements each (element
// 32 l + i in lane l of the quad): FWHT stages 1..16 in registers, stages 32
// and 64 through lane shuffles within the quad; the dot products are the
// lane's pairwise tree followed by the quad tree, which is the chunk's
// pairwise tree.  Row axis: lanes read their 64 input bytes straight from
// HBM.  Column axis (the transposed operand): a 128 x 64 bf16 tile staged in
// LDS, each quad reading one column.  Pass 1 writes the codes, v (fp32, one
// per 16) and the global max of v; pass 2 touches only the scales.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mx_internal.h"

namespace fp4mx {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // fl32(1/sqrt(128)), bits 0x3DB504F3

__device__ __forceinline__ uint32_t hash32(uint32_t h) {  // MurmurHash3 fmix32
  h ^= h >> 16;
  h *= 0x85EBCA6Bu;
  h ^= h >> 13;
  h *= 0xC2B2AE35u;
  h ^= h >> 16;
  return h;
}

// E2M1 code (sign in bit 3) of RNE(v), saturating, by the hardware converter.
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v, 0.0f, 1.0f, 0) & 0xFu;
}

// Value of lane l ^ 1 (CTRL 0xB1, quad_perm [1,0,3,2]) or l ^ 2 (CTRL 0x4E,
// quad_perm [2,3,0,1]) within each quad of lanes, by DPP (no LDS traffic).
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  const int b = __builtin_bit_cast(int, v);
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(b, b, CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor1(float v) { return quad_xor<0xB1>(v); }
__device__ __forceinline__ float quad_xor2(float v) { return quad_xor<0x4E>(v); }

// Two E2M1 codes (byte B of w) -> their signed values, exact (gfx950's
// converter with scale 1.0); and the codes of two values into byte B.
template <int B>
__device__ __forceinline__ void e2m1_pair(uint32_t w, float& lo, float& hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
  lo = v.x;
  hi = v.y;
}
template <int B>
__device__ __forceinline__ uint32_t e2m1_pack(uint32_t w, float v0, float v1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v0, v1, 1.0f, B);
}


// fp32 rounded to 4 significant bits (nearest, ties to even) on its encoding.
__device__ __forceinline__ float e8m3_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return __uint_as_float((b + 0x7FFFFu + ((b >> 20) & 1u)) & ~0xFFFFFu);
}

// Pairwise fp32 tree over 32 values (pairs (2i, 2i+1), then pairs of sums).
__device__ __forceinline__ float tree32(float (&v)[32]) {
#pragma unroll
  for (int w = 32; w > 1; w >>= 1)
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  return v[0];
}

// The quad's part of a chunk: t[32] holds elements 32 l4 + i of the chunk
// (already sign-flipped, as fp32).  Computes the codes of the lane's 32
// elements, v for its two 16-groups and the chunk's S (same in all 4 lanes).
__device__ __forceinline__ void msedn_core(float (&t)[32], int l4, float clip_s,
                                           uint32_t (&codes)[4], float (&v)[2], float& S) {
  // FWHT stages h = 1 .. 16 within the lane
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      const float a = t[i], b = t[i + h];
      t[i] = a + b;
      t[i + h] = a - b;
    }
  }
  // stages h = 32 (lane l4 ^ 1) and h = 64 (lane l4 ^ 2): the lower lane keeps
  // a + b, the upper lane a - b with a from the lower lane
  {
    const bool upper = (l4 & 1) != 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float o = quad_xor1(t[i]);
      t[i] = upper ? o - t[i] : t[i] + o;
    }
  }
  {
    const bool upper = (l4 & 2) != 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float o = quad_xor2(t[i]);
      t[i] = upper ? o - t[i] : t[i] + o;
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = t[i] * kInvSqrt128;

  float num[32], den[32];
  float am2[2];
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, __builtin_fabsf(t[16 * gi + i]));
    am2[gi] = am;
  }
  // chunk exponent E: 2^E <= max|y| < 2^(E+1) (0 for a zero chunk); the dot
  // products use y * 2^-E so no square overflows
  float cm = fmaxf(am2[0], am2[1]);
  cm = fmaxf(cm, quad_xor1(cm));
  cm = fmaxf(cm, quad_xor2(cm));
  const uint32_t cb = __float_as_uint(cm);
  const int E = cb == 0 ? 0 : (cb >= 0x800000u ? (int)(cb >> 23) - 127 : (31 - __builtin_clz(cb)) - 149);
#pragma unroll
  for (int gi = 0; gi < 2; ++gi) {
    const float p = e8m3_rne(am2[gi] / clip_s);  // IEEE division
    v[gi] = p;
    // q = E2M1_RNE(fl(y / p)): with r the hardware reciprocal of p (v_rcp_f32,
    // within 1 ulp), fl(y r) is within 3 ulp of fl(y / p), so equal codes at
    // v (1 -+ 2^-21) settle it (compared eight codes per word); otherwise, and
    // for p outside [2^-126, 2^126], divide exactly
    const bool normal_p = p >= 0x1p-126f && p <= 0x1p126f;
    const float rcp = normal_p ? __builtin_amdgcn_rcpf(p) : 0.0f;
    bool exact = !normal_p;
    uint32_t cw[2] = {0u, 0u};
    if (!exact) {
      constexpr float kLo = 1.0f - 0x1p-21f, kHi = 1.0f + 0x1p-21f;
      uint32_t hw[2] = {0u, 0u};
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        float u[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) u[i] = t[16 * gi + 8 * w + i] * rcp;
        cw[w] = e2m1_pack<0>(cw[w], u[0] * kLo, u[1] * kLo);
        hw[w] = e2m1_pack<0>(hw[w], u[0] * kHi, u[1] * kHi);
        cw[w] = e2m1_pack<1>(cw[w], u[2] * kLo, u[3] * kLo);
        hw[w] = e2m1_pack<1>(hw[w], u[2] * kHi, u[3] * kHi);
        cw[w] = e2m1_pack<2>(cw[w], u[4] * kLo, u[5] * kLo);
        hw[w] = e2m1_pack<2>(hw[w], u[4] * kHi, u[5] * kHi);
        cw[w] = e2m1_pack<3>(cw[w], u[6] * kLo, u[7] * kLo);
        hw[w] = e2m1_pack<3>(hw[w], u[6] * kHi, u[7] * kHi);
      }
      exact = (cw[0] != hw[0]) || (cw[1] != hw[1]);
    }
    if (exact) {
      cw[0] = cw[1] = 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t q =
            p > 0.0f ? e2m1_code(t[16 * gi + i] / p) : (__float_as_uint(t[16 * gi + i]) >> 28) & 8u;
        cw[i / 8] |= q << (4 * (i % 8));
      }
    }
    codes[2 * gi] = cw[0];
    codes[2 * gi + 1] = cw[1];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float qv[8];
      e2m1_pair<0>(cw[w], qv[0], qv[1]);
      e2m1_pair<1>(cw[w], qv[2], qv[3]);
      e2m1_pair<2>(cw[w], qv[4], qv[5]);
      e2m1_pair<3>(cw[w], qv[6], qv[7]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int k = 16 * gi + 8 * w + i;
        const float r = qv[i] * p;
        const float z = __builtin_ldexpf(t[k], -E), zr = __builtin_ldexpf(r, -E);
        num[k] = z * z;
        den[k] = z * zr;
      }
    }
  }
  float sn = tree32(num), sd = tree32(den);
  // quad tree: (l0 + l1) + (l2 + l3); fp32 addition commutes, so every lane
  // ends with the same value
  sn = sn + quad_xor1(sn);
  sd = sd + quad_xor1(sd);
  sn = sn + quad_xor2(sn);
  sd = sd + quad_xor2(sd);
  S = sd > 0.0f ? sn / sd : 1.0f;  // IEEE division
  v[0] = S * v[0];
  v[1] = S * v[1];
}

__device__ __forceinline__ void block_max_atomic(float m, uint32_t* gmax) {
  uint32_t b = __float_as_uint(m);  // non-negative: orders as unsigned
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) b = max(b, (uint32_t)__shfl_xor((int)b, off, 64));
  __shared__ uint32_t wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = b;
  __syncthreads();
  if (threadIdx.x == 0) atomicMax(gmax, max(max(wm[0], wm[1]), max(wm[2], wm[3])));
}

struct Mask128 {
  uint32_t w[4];
};

__device__ __forceinline__ void unpack_signed(const uint32_t (&wd)[16], uint32_t mask, float (&t)[32]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t w = wd[j] ^ ((((mask >> (2 * j)) & 1u) << 15) | (((mask >> (2 * j + 1)) & 1u) << 31));
    t[2 * j] = __uint_as_float(w << 16);
    t[2 * j + 1] = __uint_as_float(w & 0xFFFF0000u);
  }
}

// ---------------------------------------------------------------------------
// Pass 1, row axis: thread = 32 elements of each of two chunks; quad g takes
// chunks 2g and 2g+1 (row-major over (row, chunk-in-row)).  Both chunks' loads
// are issued before either is transformed, so one memory latency covers two
// chunks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load_lane32(const uint16_t* x, int64_t ld, uint32_t chunk, int l4,
                                            FastDiv qdiv, uint32_t (&wd)[16], int64_t& row,
                                            int64_t& ch) {
  const uint32_t row32 = fastdiv(chunk, qdiv);  // qdiv.d = chunks per row
  row = row32;
  ch = chunk - row32 * qdiv.d;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + row * ld + ch * 128 + 32 * l4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 v = *(src + q);
    wd[4 * q] = v.x; wd[4 * q + 1] = v.y; wd[4 * q + 2] = v.z; wd[4 * q + 3] = v.w;
  }
}

__global__ __launch_bounds__(256) void msedn_pass1_row(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, Mask128 mask,
    float clip_s, uint8_t* __restrict__ codes, float* __restrict__ vbuf,
    float* __restrict__ eden_s, uint32_t* __restrict__ gmax, FastDiv qdiv, uint32_t nthreads,
    uint32_t nchunks) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const bool live = t < nthreads;  // every lane takes part in the shuffles
  const uint32_t tt = live ? t : 0u;
  const int l4 = (int)(tt & 3u);
  const uint32_t ca = 2u * (tt >> 2);
  const bool live_b = live && ca + 1u < nchunks;
  const uint32_t cb = live_b ? ca + 1u : ca;  // a spare lane re-reads chunk a
  uint32_t wa[16], wb[16];
  int64_t row_a, ch_a, row_b, ch_b;
  load_lane32(x, ld, ca, l4, qdiv, wa, row_a, ch_a);
  load_lane32(x, ld, cb, l4, qdiv, wb, row_b, ch_b);
  float vmax = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float tv[32];
    unpack_signed(k == 0 ? wa : wb, mask.w[l4], tv);
    uint32_t cw[4];
    float v[2], S;
    msedn_core(tv, l4, clip_s, cw, v, S);
    const bool on = k == 0 ? live : live_b;
    const int64_t row = k == 0 ? row_a : row_b, ch = k == 0 ? ch_a : ch_b;
    const int64_t c0 = ch * 128 + 32 * l4;
    if (on) {
      *reinterpret_cast<u32x4*>(codes + row * (cols / 2) + c0 / 2) = u32x4{cw[0], cw[1], cw[2], cw[3]};
      *reinterpret_cast<float2*>(vbuf + row * (cols / 16) + c0 / 16) = make_float2(v[0], v[1]);
      if (eden_s && l4 == 0) eden_s[row * (cols / 128) + ch] = S;
      vmax = fmaxf(vmax, fmaxf(v[0], v[1]));
    }
  }
  block_max_atomic(vmax, gmax);
}

// ---------------------------------------------------------------------------
// Pass 1, column axis: 128 x 128 bf16 tile in LDS; a quad takes one pair of
// adjacent columns (one 4-byte LDS read gives both), i.e. two output chunks.
// Output operand row = input column, output column = input row.
// ---------------------------------------------------------------------------
constexpr int kCPitch = 260;  // bytes per LDS row: 2-way conflicts between quads at most

__global__ __launch_bounds__(256) void msedn_pass1_col(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, Mask128 mask,
    float clip_s, uint8_t* __restrict__ codes, float* __restrict__ vbuf,
    float* __restrict__ eden_s, uint32_t* __restrict__ gmax) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[128 * kCPitch];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 128, cb = (int64_t)blockIdx.y * 128;
  const int nc = (int)min<int64_t>(128, cols - cb);
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int id = tid + 256 * it;  // 2048 chunks of 8 bf16
    const int r = id >> 4, chk = id & 15;
    if (chk * 8 < nc) {
      const u32x4 v = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(x + (r0 + r) * ld + cb + chk * 8));
      uint32_t* d = reinterpret_cast<uint32_t*>(tile + r * kCPitch + chk * 16);
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
  }
  __syncthreads();
  const int cp = tid >> 2, l4 = tid & 3;
  const bool live = 2 * cp < nc;  // nc is a multiple of 32: both columns or neither
  const int cc = live ? cp : 0;
  uint32_t wpair[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    wpair[i] = *reinterpret_cast<const uint32_t*>(tile + (32 * l4 + i) * kCPitch + 4 * cc);
  const uint32_t m = mask.w[l4];
  float vmax = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    float tv[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t b = k == 0 ? wpair[i] << 16 : wpair[i] & 0xFFFF0000u;
      tv[i] = __uint_as_float(b ^ (((m >> i) & 1u) << 31));
    }
    uint32_t cw[4];
    float v[2], S;
    msedn_core(tv, l4, clip_s, cw, v, S);
    if (live) {
      const int64_t orow = cb + 2 * cp + k, ocol = r0 + 32 * l4;
      *reinterpret_cast<u32x4*>(codes + orow * (rows / 2) + ocol / 2) = u32x4{cw[0], cw[1], cw[2], cw[3]};
      *reinterpret_cast<float2*>(vbuf + orow * (rows / 16) + ocol / 16) = make_float2(v[0], v[1]);
      if (eden_s && l4 == 0) eden_s[orow * (rows / 128) + r0 / 128] = S;
      vmax = fmaxf(vmax, fmaxf(v[0], v[1]));
    }
  }
  block_max_atomic(vmax, gmax);
}

// ---------------------------------------------------------------------------
// Pass 1 on a saved NVFP4 operand (the backward's re-quantization of the
// forward's Q(X), Q(W)): the codes and E4M3 scales of a 128 x 128 tile are
// staged in LDS as they are (9 KB); a quad takes a pair of adjacent columns,
// whose codes share one byte per row, and decodes fl(fl(q * s16) * g) as it
// reads (q * s16 is exact).  Output row = input column.
// ---------------------------------------------------------------------------
constexpr int kNCodePitch = 68;   // code bytes per LDS row (64 + pad)
constexpr int kNScalePitch = 12;  // scale bytes per LDS row (8 + pad)

// OCP E4M3FN byte (the low byte of b) -> float, exact, by gfx950's converter
// v_cvt_f32_fp8 (OCP formats on this target; 0x7F / 0xFF decode to NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// Three waves per SIMD (at most 168 registers, against 172 unconstrained):
// 8192 x 4096 re-quantization 43.8 instead of 46.3 us, a few registers
// spilled.  The other pass-1 kernels ran slower with such a cap.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void msedn_pass1_col_nv(
    const uint8_t* __restrict__ qcodes, const uint8_t* __restrict__ qscales,
    const float* __restrict__ qg, int64_t rows, int64_t cols, Mask128 mask, float clip_s,
    uint8_t* __restrict__ codes, float* __restrict__ vbuf, float* __restrict__ eden_s,
    uint32_t* __restrict__ gmax) {
  __shared__ __attribute__((aligned(16))) uint8_t tcodes[128 * kNCodePitch];
  __shared__ __attribute__((aligned(16))) uint8_t tscales[128 * kNScalePitch];
  const int tid = threadIdx.x;
  const int64_t r0 = (int64_t)blockIdx.x * 128, cb = (int64_t)blockIdx.y * 128;
  const int nc = (int)min<int64_t>(128, cols - cb);  // a multiple of 32
  {
    // codes: 128 rows x 64 bytes = 512 chunks of 16 B, two per thread
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int id = tid + 256 * it;
      const int r = id >> 2, chk = id & 3;
      if (chk * 32 < nc) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(qcodes + (r0 + r) * (cols / 2) + cb / 2 + chk * 16);
        uint32_t* d = reinterpret_cast<uint32_t*>(tcodes + r * kNCodePitch + chk * 16);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
    }
    // scales: 128 rows x 8 bytes, thread = 4 bytes (two 2-byte loads) of one row
    const int r = tid >> 1, h = tid & 1;
    const uint8_t* sp = qscales + (r0 + r) * (cols / 16) + cb / 16 + 4 * h;
    uint16_t* sd = reinterpret_cast<uint16_t*>(tscales + r * kNScalePitch + 4 * h);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if ((4 * h + 2 * u) * 16 < nc) sd[u] = *reinterpret_cast<const uint16_t*>(sp + 2 * u);
  }
  __syncthreads();
  const int cp = tid >> 2, l4 = tid & 3;
  const bool live = 2 * cp < nc;  // both columns of the pair or neither
  const int cc = live ? cp : 0;
  const float g = *qg;
  const uint32_t m = mask.w[l4];
  float ta[32], tb[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * l4 + i;
    const uint32_t byte = tcodes[row * kNCodePitch + cc];
    const float s16 = e4m3_to_f32(tscales[row * kNScalePitch + (cc >> 3)]);
    float qa, qb;
    e2m1_pair<0>(byte, qa, qb);
    const uint32_t flip = ((m >> i) & 1u) << 31;
    ta[i] = __uint_as_float(__float_as_uint((qa * s16) * g) ^ flip);
    tb[i] = __uint_as_float(__float_as_uint((qb * s16) * g) ^ flip);
  }
  float vmax = 0.0f;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t cw[4];
    float v[2], S;
    msedn_core(k == 0 ? ta : tb, l4, clip_s, cw, v, S);
    if (live) {
      const int64_t orow = cb + 2 * cp + k, ocol = r0 + 32 * l4;
      *reinterpret_cast<u32x4*>(codes + orow * (rows / 2) + ocol / 2) = u32x4{cw[0], cw[1], cw[2], cw[3]};
      *reinterpret_cast<float2*>(vbuf + orow * (rows / 16) + ocol / 16) = make_float2(v[0], v[1]);
      if (eden_s && l4 == 0) eden_s[orow * (rows / 128) + r0 / 128] = S;
      vmax = fmaxf(vmax, fmaxf(v[0], v[1]));
    }
  }
  block_max_atomic(vmax, gmax);
}

// ---------------------------------------------------------------------------
// Pass 2: thread = one group scale.  k = least integer with max * 2^-k <= 256;
// scale = SR_E4M3(v * 2^-k) with u = (r >> 8) * 2^-24, r = hash of the
// scale's flat index in the output operand.
// ---------------------------------------------------------------------------
__global__ void msedn_zero(uint32_t* p) { *p = 0u; }

__global__ __launch_bounds__(256) void msedn_pass2(const float* __restrict__ vbuf,
                                                   const uint32_t* __restrict__ gmax,
                                                   uint64_t nscales, uint32_t key_lo,
                                                   uint32_t key_hi, uint8_t* __restrict__ scales,
                                                   float* __restrict__ tensor_scale) {
  const uint32_t mb = *gmax;
  int k = 0;
  if (mb != 0) {
    // ceil(log2 max): normal 1.f * 2^(e-127); subnormal mb * 2^-149
    const int e = (int)(mb >> 23);
    const int lg = e != 0 ? e - 127 + ((mb & 0x7FFFFFu) != 0 ? 1 : 0)
                          : (mb == 1u ? 0 : 32 - __builtin_clz(mb - 1u)) - 149;
    k = lg - 8;
  }
  const uint64_t t = (uint64_t)blockIdx.x * 256u + threadIdx.x;
  if (t == 0) *tensor_scale = __builtin_ldexpf(1.0f, k);
  if (t >= nscales) return;
  const float w = __builtin_ldexpf(vbuf[t], -k);
  const uint32_t kmix = key_lo ^ hash32((uint32_t)(t >> 32) ^ key_hi);
  const uint32_t r = hash32((uint32_t)t ^ kmix);
  const uint32_t b = __float_as_uint(w);
  uint32_t code;
  if (w >= 0x1p-6f) {
    // normal E4M3: floor code from exponent and top 3 fraction bits, up iff
    // (r >> 12) < the 20 fraction bits below them
    const uint32_t fl = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
    code = fl + (((r >> 12) < (b & 0xFFFFFu)) ? 1u : 0u);
    code = min(code, 0x7Eu);  // saturate at 448
  } else {
    // subnormal step 2^-9: t = w * 2^9 < 8, up iff (r >> 8) < frac(t) * 2^24
    const float tt = w * 512.0f;
    const float a = __builtin_floorf(tt);
    code = (uint32_t)a + (((float)(r >> 8) < (tt - a) * 0x1p24f) ? 1u : 0u);
  }
  scales[t] = (uint8_t)code;
}

}  // namespace

hipError_t launch_msedn_requant(const uint8_t* qcodes, const uint8_t* qscales, const float* qg,
                                int64_t rows, int64_t cols, float clip_s, uint64_t seed,
                                uint32_t gemm_id, uint32_t stream, uint8_t* codes, uint8_t* scales,
                                float* tensor_scale, float* eden_s, float* vbuf, uint32_t* gmax,
                                hipStream_t s) {
  Mask128 m;
  msedn_sign_words(seed, gemm_id, m.w);
  const RngKey key = make_key(seed, stream);
  hipLaunchKernelGGL(msedn_zero, dim3(1), dim3(1), 0, s, gmax);
  hipLaunchKernelGGL(msedn_pass1_col_nv, dim3((unsigned)(rows / 128), (unsigned)((cols + 127) / 128)),
                     dim3(256), 0, s, qcodes, qscales, qg, rows, cols, m, clip_s, codes, vbuf,
                     eden_s, gmax);
  const int64_t nscales = cols * (rows / 16);
  hipLaunchKernelGGL(msedn_pass2, dim3((unsigned)((nscales + 255) / 256)), dim3(256), 0, s, vbuf,
                     gmax, (uint64_t)nscales, key.lo, key.hi, scales, tensor_scale);
  return hipGetLastError();
}

void msedn_sign_words(uint64_t seed, uint32_t gemm_id, uint32_t (&w)[4]) {
  const uint64_t a = splitmix64(seed ^ ((uint64_t)(0x5200u + 2u * gemm_id) << 32));
  const uint64_t b = splitmix64(seed ^ ((uint64_t)(0x5201u + 2u * gemm_id) << 32));
  w[0] = (uint32_t)a; w[1] = (uint32_t)(a >> 32); w[2] = (uint32_t)b; w[3] = (uint32_t)(b >> 32);
}

hipError_t launch_msedn(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, int axis,
                        float clip_s, uint64_t seed, uint32_t gemm_id, uint32_t stream,
                        uint8_t* codes, uint8_t* scales, float* tensor_scale, float* eden_s,
                        float* vbuf, uint32_t* gmax, hipStream_t s) {
  Mask128 m;
  msedn_sign_words(seed, gemm_id, m.w);
  const RngKey key = make_key(seed, stream);
  hipLaunchKernelGGL(msedn_zero, dim3(1), dim3(1), 0, s, gmax);  // a kernel: safe under capture
  int64_t nscales;
  if (axis == FP4MX_AXIS_ROW) {
    const int64_t cpr = cols / 128;
    const uint64_t chunks = (uint64_t)rows * (uint64_t)cpr;
    const uint64_t threads = (chunks + 1) / 2 * 4u;  // a quad per two chunks
    if (chunks >= (1ull << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(msedn_pass1_row, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       x, rows, cols, ld, m, clip_s, codes, vbuf, eden_s, gmax,
                       make_fastdiv((uint32_t)cpr), (uint32_t)threads, (uint32_t)chunks);
    nscales = rows * (cols / 16);
  } else {
    hipLaunchKernelGGL(msedn_pass1_col, dim3((unsigned)(rows / 128), (unsigned)((cols + 127) / 128)),
                       dim3(256), 0, s, x, rows, cols, ld, m, clip_s, codes, vbuf, eden_s, gmax);
    nscales = cols * (rows / 16);
  }
  hipLaunchKernelGGL(msedn_pass2, dim3((unsigned)((nscales + 255) / 256)), dim3(256), 0, s, vbuf,
                     gmax, (uint64_t)nscales, key.lo, key.hi, scales, tensor_scale);
  return hipGetLastError();
}

}  // namespace fp4mx
