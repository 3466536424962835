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
//    store.  Row-axis groups are staged per wave through LDS so the global
//    reads are coalesced 16-B loads.
//  - Column-axis groups (the transposed operand) go through a 128 x 64 bf16
//    LDS tile: one coalesced read of the tile feeds both the row-axis and the
//    column-axis quantizer, so the dual kernel reads each input byte once.
//  - RTN uses gfx950's v_cvt_scalef32_pk_fp4_f32, which computes E2M1
//    round-to-nearest-even of x / scale with saturation (two elements per
//    instruction, the sign included).  SR draws 32 bits per element from the
//    counter hash and rounds on gfx950's SR converter
//    v_cvt_scalef32_sr_pk_fp4_f32: the element's position in its E2M1 gap,
//    cut to 22 bits, plus the top 22 bits of the draw, rounds up on carry
//    (the rule and its probed behaviour are in mx_device.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp4mx_internal.h"
#include "mx_device.h"

namespace fp4mx {
namespace {

// ---------------------------------------------------------------------------
// Row axis: thread = one group of one row.  Each wave stages its 64 groups
// (4 KB of bf16) through LDS so the global reads are fully coalesced 16-B
// loads (lane l reads bytes 16 l + 1024 q), then each lane reads back its own
// 64-byte group.  Groups are numbered row-major over (row, group-in-row).
// ---------------------------------------------------------------------------
constexpr int kWaveStage = 64 * 64 + 16 * 4;  // 64 groups of 64 B, 16-B pad per 16 groups

// this wave's 4 x 16 B of block blk into registers (no LDS)
__device__ __forceinline__ void row_fetch(uint32_t blk, u32x4 (&v)[4], const uint16_t* __restrict__ x,
                                          int64_t ld, FastDiv gdiv, uint32_t ngroups) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t g_wave = blk * 256u + (uint32_t)wave * 64u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)q * 64u + (uint32_t)lane;
    const uint32_t g = g_wave + chunk / 4u;
    if (g < ngroups) {
      const uint32_t row32 = fastdiv(g, gdiv);
      const int64_t grp = g - row32 * gdiv.d;
      v[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          x + (int64_t)row32 * ld + grp * kGroup + (chunk & 3u) * 8));
    }
  }
}

template <bool HAD, int ROUND>
__device__ __forceinline__ void row_finish(uint32_t blk, const u32x4 (&v)[4], uint8_t* ws, int64_t cols,
                                           uint32_t sign_mask, uint32_t key_lo, uint32_t key_hi,
                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                           FastDiv gdiv, uint32_t ngroups) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t g_wave = blk * 256u + (uint32_t)wave * 64u;
  if (g_wave >= ngroups) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)q * 64u + (uint32_t)lane;
    *reinterpret_cast<u32x4*>(ws + chunk * 16 + (chunk / 64u) * 16) = v[q];
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  const uint32_t g = g_wave + (uint32_t)lane;
  uint32_t wd[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t chunk = (uint32_t)lane * 4u + (uint32_t)q;
    const u32x4 w4 = *reinterpret_cast<const u32x4*>(ws + chunk * 16 + (chunk / 64u) * 16);
    wd[4 * q + 0] = w4.x; wd[4 * q + 1] = w4.y; wd[4 * q + 2] = w4.z; wd[4 * q + 3] = w4.w;
  }
  if (g >= ngroups) return;
  const uint32_t row32 = fastdiv(g, gdiv);
  const int64_t row = row32, grp = g - row32 * gdiv.d;
  const int64_t gpr = gdiv.d;
  float t[kGroup];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t w = wd[j];
    if constexpr (HAD) w = flip_pair(w, sign_mask, j);
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

// Groups of workgroup-block `blk` (4 waves x 64 groups); `ws` is this wave's
// LDS stage.
template <bool HAD, int ROUND>
__device__ __forceinline__ void row_block(uint32_t blk, uint8_t* ws, const uint16_t* __restrict__ x,
                                          int64_t cols, int64_t ld, uint32_t sign_mask,
                                          uint32_t key_lo, uint32_t key_hi,
                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                          FastDiv gdiv, uint32_t ngroups) {
  u32x4 v[4] = {};
  row_fetch(blk, v, x, ld, gdiv, ngroups);
  row_finish<HAD, ROUND>(blk, v, ws, cols, sign_mask, key_lo, key_hi, codes, scales, gdiv, ngroups);
}

// RTN is bandwidth-bound: a grid of one residency (6 workgroups per CU at the
// loop's 76 registers) strides over the blocks, so no partial last wave of
// workgroups idles the memory system (8192 x 4096: 18.5 instead of 22 us),
// and each wave's loads of its next block are in flight while it quantizes
// the current one (16384 x 8192: 59.7-60.4 against 61.4-61.7 us, 5.6-5.7
// TB/s; at 8192 x 4096 within 2% either way).  SR runs one block per
// workgroup: with the loop it took 6-14% longer (8192 x 4096: 30.2 against
// 28.5 us).
template <bool HAD, int ROUND>
__global__ __launch_bounds__(256) void quant_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t sign_mask,
    uint32_t key_lo, uint32_t key_hi, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, FastDiv gdiv, uint32_t ngroups, uint32_t nblk) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[4 * kWaveStage];
  uint8_t* ws = stage + (threadIdx.x >> 6) * kWaveStage;
  if constexpr (ROUND == FP4MX_ROUND_RTN) {
    // the next block's loads are in flight while this block is quantized
    u32x4 cur[4] = {}, nxt[4] = {};
    uint32_t blk = blockIdx.x;
    if (blk < nblk) row_fetch(blk, cur, x, ld, gdiv, ngroups);
    for (; blk < nblk; blk += gridDim.x) {
      const uint32_t nb = blk + gridDim.x;
      if (nb < nblk) row_fetch(nb, nxt, x, ld, gdiv, ngroups);
      row_finish<HAD, ROUND>(blk, cur, ws, cols, sign_mask, key_lo, key_hi, codes, scales, gdiv, ngroups);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this block's LDS reads are done before the next writes
#pragma unroll
      for (int q = 0; q < 4; ++q) cur[q] = nxt[q];
    }
  } else {
    row_block<HAD, ROUND>(blockIdx.x, ws, x, cols, ld, sign_mask, key_lo, key_hi, codes, scales,
                          gdiv, ngroups);
  }
}

// ---------------------------------------------------------------------------
// LDS tile kernel: 128 rows x 64 columns of bf16, read once from HBM.
//   ROW_ROUND >= 0: row-axis groups (thread = row t/2, group t%2);
//   COL_ROUND >= 0: column-axis groups (thread = column t%64, row group t/64),
//                   written as the transposed operand.
// ---------------------------------------------------------------------------
constexpr int kTileR = 128, kTileC = 64;
constexpr int kPitch = kTileC * 2 + 16;  // bytes per LDS row (padding vs bank conflicts)
constexpr int kCoutPitch = (kTileR / kGroup) * 16 + 16;  // column-output staging: 64 B + pad per column

// One operand of the tile kernel: its bf16 input and the row-axis and
// column-axis outputs (the unused axis's fields are ignored).
struct TileJob {
  const uint16_t* x;
  int64_t rows, cols, ld;
  uint32_t row_mask, row_klo, row_khi;
  uint8_t* row_codes;
  uint8_t* row_scales;
  uint32_t col_mask, col_klo, col_khi;
  uint8_t* col_codes;
  uint8_t* col_scales;
};

// The tile at rows [r0, r0 + 128) and columns [c0, c0 + 64) of job j.
template <bool HAD, int ROW_ROUND, int COL_ROUND>
__device__ __forceinline__ void quant_tile(const TileJob& j, int64_t r0, int64_t c0) {
  const uint16_t* __restrict__ x = j.x;
  const int64_t rows = j.rows, cols = j.cols, ld = j.ld;
  const uint32_t row_mask = j.row_mask, row_klo = j.row_klo, row_khi = j.row_khi;
  const uint32_t col_mask = j.col_mask, col_klo = j.col_klo, col_khi = j.col_khi;
  uint8_t* __restrict__ row_codes = j.row_codes;
  uint8_t* __restrict__ row_scales = j.row_scales;
  uint8_t* __restrict__ col_codes = j.col_codes;
  uint8_t* __restrict__ col_scales = j.col_scales;
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileR * kPitch];
  const int tid = threadIdx.x;
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
        if constexpr (HAD) w = flip_pair(w, row_mask, j);
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
    // Codes and scales go through LDS so each output row's 4 x 16 B of this
    // tile leave as one 64-B piece and its 4 scale bytes as one word (a wave
    // stores 16 rows per instruction instead of 16 B in each of 64 rows;
    // 8192 x 4096 RTN column pass 26 -> 24 us).
    __shared__ __attribute__((aligned(16))) uint8_t cout[kTileC * kCoutPitch];
    __shared__ __attribute__((aligned(16))) uint8_t cscl[kTileC * (kTileR / kGroup)];
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
      *reinterpret_cast<u32x4*>(cout + c * kCoutPitch + rg * 16) = o;
      cscl[c * (kTileR / kGroup) + rg] = (uint8_t)sc;
    }
    __syncthreads();
    const int oc = tid >> 2, q = tid & 3;  // output row c0 + oc, its q-th group of this tile
    if (oc < nc && q * kGroup < nr) {
      *reinterpret_cast<u32x4*>(col_codes + (c0 + oc) * (rows / 2) + (r0 / kGroup + q) * 16) =
          *reinterpret_cast<const u32x4*>(cout + oc * kCoutPitch + q * 16);
      uint8_t* sp = col_scales + (c0 + oc) * (rows / kGroup) + r0 / kGroup;
      if (nr == kTileR && (rows / kGroup) % 4 == 0 && ((uintptr_t)col_scales & 3u) == 0) {
        // the row's 4 scale bytes of this tile as one aligned word
        if (q == 0) *reinterpret_cast<uint32_t*>(sp) = *reinterpret_cast<const uint32_t*>(cscl + oc * 4);
      } else {
        sp[q] = cscl[oc * (kTileR / kGroup) + q];
      }
    }
  }
}

// Grid: x = row tiles, y = column tiles.
template <bool HAD, int RR, int CR>
__global__ __launch_bounds__(256) void quant_tile_kernel(TileJob j) {
  quant_tile<HAD, RR, CR>(j, (int64_t)blockIdx.x * kTileR, (int64_t)blockIdx.y * kTileC);
}

// Two operands with the same modes in one launch, so the second's tiles fill
// the first's last partial round of workgroups: blocks [0, na) take job a's
// tiles, the rest job b's, each in quant_tile_kernel's order (row tile
// fastest; tra, trb = row tiles of a, b).
template <bool HAD, int RR, int CR>
__global__ __launch_bounds__(256) void quant_tile_pair_kernel(TileJob a, TileJob b, uint32_t na,
                                                              uint32_t tra, uint32_t trb) {
  const uint32_t blk = blockIdx.x;
  const bool first = blk < na;
  const uint32_t t = first ? blk : blk - na, tr = first ? tra : trb;
  quant_tile<HAD, RR, CR>(first ? a : b, (int64_t)(t % tr) * kTileR, (int64_t)(t / tr) * kTileC);
}

TileJob tile_job(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld, const QuantOut* ro,
                 const QuantOut* co) {
  QuantOut z{};
  const QuantOut& R = ro ? *ro : z;
  const QuantOut& C = co ? *co : z;
  return TileJob{x,       rows,     cols,     ld,          R.sign_mask, R.key.lo, R.key.hi,
                 R.codes, R.scales, C.sign_mask, C.key.lo, C.key.hi,    C.codes,  C.scales};
}

template <bool HAD, int RR, int CR>
hipError_t tile_launch(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                       const QuantOut* ro, const QuantOut* co, hipStream_t s) {
  dim3 grid((unsigned)((rows + kTileR - 1) / kTileR), (unsigned)((cols + kTileC - 1) / kTileC));
  hipLaunchKernelGGL((quant_tile_kernel<HAD, RR, CR>), grid, dim3(256), 0, s,
                     tile_job(x, rows, cols, ld, ro, co));
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

// Compute units of the current device (cached per device; 256 on MI355X).
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

hipError_t launch_quant_row(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                            bool hadamard, const QuantOut& o, hipStream_t s) {
  const int64_t groups = rows * (cols / kGroup);
  if (groups >= (1ll << 31)) return launch_quant_tile(x, rows, cols, ld, hadamard, &o, nullptr, s);
  const FastDiv gd = make_fastdiv((uint32_t)(cols / kGroup));
  const uint32_t nblk = (uint32_t)((groups + 255) / 256);
  const uint32_t ng = (uint32_t)groups;
  const uint32_t resident = (uint32_t)cu_count() * 6u;
  const unsigned grid = o.rounding == FP4MX_ROUND_RTN && nblk > resident ? resident : nblk;
  if (hadamard) {
    if (o.rounding == FP4MX_ROUND_RTN)
      hipLaunchKernelGGL((quant_row_kernel<true, 0>), dim3(grid), dim3(256), 0, s, x, rows, cols,
                         ld, o.sign_mask, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng, nblk);
    else
      hipLaunchKernelGGL((quant_row_kernel<true, 1>), dim3(grid), dim3(256), 0, s, x, rows, cols,
                         ld, o.sign_mask, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng, nblk);
  } else {
    if (o.rounding == FP4MX_ROUND_RTN)
      hipLaunchKernelGGL((quant_row_kernel<false, 0>), dim3(grid), dim3(256), 0, s, x, rows, cols,
                         ld, 0u, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng, nblk);
    else
      hipLaunchKernelGGL((quant_row_kernel<false, 1>), dim3(grid), dim3(256), 0, s, x, rows, cols,
                         ld, 0u, o.key.lo, o.key.hi, o.codes, o.scales, gd, ng, nblk);
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

hipError_t launch_quant_tile_pair(const uint16_t* xa, int64_t rows_a, int64_t cols_a, int64_t ld_a,
                                  const QuantOut& ra, const QuantOut& ca, const uint16_t* xb,
                                  int64_t rows_b, int64_t cols_b, int64_t ld_b,
                                  const QuantOut& rb, const QuantOut& cb, hipStream_t s) {
  const int64_t tra = (rows_a + kTileR - 1) / kTileR, trb = (rows_b + kTileR - 1) / kTileR;
  const int64_t na = tra * ((cols_a + kTileC - 1) / kTileC), nb = trb * ((cols_b + kTileC - 1) / kTileC);
  const bool fused = ra.rounding == FP4MX_ROUND_RTN && rb.rounding == FP4MX_ROUND_RTN &&
                     ca.rounding == FP4MX_ROUND_SR && cb.rounding == FP4MX_ROUND_SR &&
                     na + nb < (1ll << 24);  // 256 x blocks within the 32-bit grid size
  if (!fused) {
    hipError_t e = launch_quant_tile(xa, rows_a, cols_a, ld_a, true, &ra, &ca, s);
    return e == hipSuccess ? launch_quant_tile(xb, rows_b, cols_b, ld_b, true, &rb, &cb, s) : e;
  }
  hipLaunchKernelGGL((quant_tile_pair_kernel<true, FP4MX_ROUND_RTN, FP4MX_ROUND_SR>),
                     dim3((unsigned)(na + nb)), dim3(256), 0, s,
                     tile_job(xa, rows_a, cols_a, ld_a, &ra, &ca),
                     tile_job(xb, rows_b, cols_b, ld_b, &rb, &cb), (uint32_t)na, (uint32_t)tra,
                     (uint32_t)trb);
  return hipGetLastError();
}

}  // namespace fp4mx
