// Block-scaled GEMM on gfx950 MFMA: MXFP4 x MXFP4 -> fp32, and the FP8 (E4M3)
// variant used by the NVFP4 path.
//
// Computes C = alpha * deq(A) deq(B)^T with A [m][k], B [n][k] stored K-major
// (FP4: two codes per byte; FP8: one per byte) and one E8M0 scale per 32 K
// elements per row; fp32 accumulation; fp32 output, or bf16 (RNE of the
// fp32 result) for the bf16-output entry point.
// Source: "Quartet: Native FP4 Training Can Be Optimal for Large Language
// Models" -- "The GPU Kernel Implementation", Stage 2 (block-scaled GEMM
// D = C + (A x SFA)(B x SFB), FP32 accumulator and output).
//
// Design (MI355X):
//  - v_mfma_scale_f32_32x32x64_f8f6f4.  FP4: lane l holds row l%32 and the 32
//    contiguous K elements [32*(l/32), +32) of its 32x64 fragment (16 bytes =
//    one MXFP4 group) plus that group's E8M0 scale, so the quantizers' K-major
//    layout is consumed as is (no scale rearrangement pass).  FP8: lane half h
//    holds K [16h, 16h+16) and [32+16h, +16); the scale of group 2s+h again
//    comes from half h.
//  - A workgroup (4 waves) computes a 256 x 256 tile, each wave 128 x 128
//    (4 x 4 fragments, 256 fp32 accumulators).  K advances in stages of 128
//    bytes per row (256 FP4 / 128 FP8 elements) through double-buffered LDS:
//    the global loads of stage s+1 are in flight while stage s's 64 MFMAs per
//    wave run; fragments for the next K substep are read from LDS while the
//    current substep's MFMAs issue.
//  - Global traffic uses buffer resources: out-of-range rows and K chunks
//    read as zero in hardware, so there are no branches around loads.
//  - LDS rows are XOR-swizzled in 16-B chunks (conflict-free fragment
//    reads); each row's stage scales are stored as two dwords holding
//    groups {h, 2+h, 4+h, 6+h}, byte s selected by op_sel.
//  - Epilogues: fp32 stores straight from the accumulators; or, through LDS
//    staging (the stage buffers are free after the last stage), the Quartet
//    backward's C <- H^-1((alpha acc) with masked entries zeroed) per
//    32-column group, or a bf16 output with whole-row 16-B stores.
//  - Tiles are assigned XCD-aware: workgroup i runs on XCD i % 8, so each XCD
//    gets a contiguous run of tiles in grouped (4 tile-rows) order and shares
//    A and B panels in its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp4mx_internal.h"

#ifndef FP4MX_GEMM_WM
#define FP4MX_GEMM_WM 2  // waves along M
#endif
#ifndef FP4MX_GEMM_WN
#define FP4MX_GEMM_WN 2  // waves along N
#endif

namespace fp4mx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256;
constexpr int kRowBytes = 128;              // operand bytes per row per stage
constexpr int kCodeLds = (kBM + kBN) * kRowBytes;
constexpr int kScaleLds = (kBM + kBN) * 8;
constexpr int kStageLds = kCodeLds + kScaleLds;
constexpr uint32_t kOOB = 0x80000000u;      // offset beyond any num_records

// Wave layout: WM x WN waves, each owning a (256/WM) x (256/WN) sub-tile.
template <int WM, int WN>
struct Waves {
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * 64;
  static constexpr int FM = kBM / WM / 32, FN = kBN / WN / 32;  // 32x32 fragments per wave
  static constexpr int kBlocks = kCodeLds / 1024 / kWaves;      // 1-KB LDS blocks per wave per stage
  static constexpr int kMinWaves = kWaves / 4;                  // waves per SIMD
};

// LDS operand layout: row r of a 256-row operand tile holds its 128 stage
// bytes as eight 16-B chunks; chunk c is stored in slot c ^ ((r >> 1) & 7), so
// the 16-B fragment reads of 16 consecutive rows touch all 64 banks once.
__device__ __forceinline__ int lds_slot(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): loads beyond `bytes` return
// zero and stores beyond it are dropped (stride 0, gfx9 dword-3 format bits).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

__device__ __forceinline__ i32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ i32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(i32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}
// 16 B per lane straight into LDS: lane l's data lands at lds + 16 l (the
// wave writes one contiguous 1-KB block); out-of-range offsets write zeros.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, uint8_t* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
// C stores are non-temporal (cache policy nt): the output is written once
// and is far larger than L2, and letting it allocate evicts the operand
// panels that later tiles re-read (measured: 8192x14336x4096 GEMM 315 ->
// 285 us; no change at 8192x4096x4096).
constexpr int kStoreNT = 2;
__device__ __forceinline__ void buf_store4(float v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, kStoreNT);
}

// Epilogue kinds.
constexpr int kEpiF32 = 0;   // C fp32
constexpr int kEpiIrht = 1;  // C fp32 <- H^-1(mask-zeroed alpha acc) per 32-column group
constexpr int kEpiBf16 = 2;  // C bf16 = RNE(alpha acc)

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN.  Written as
// a select: an early return for NaN compiles to a branch per element.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

template <int FMT>
struct Fmt {
  static constexpr int kStageK = FMT == 4 ? 256 : 128;  // K elements per stage
  static constexpr int kGroups = kStageK / 32;          // scale groups per row per stage
  static constexpr int kSub = kStageK / 64;             // MFMA K-substeps per stage
  static constexpr int kSubBytes = kRowBytes / kSub;
};

// Workgroup -> tile, XCD-aware and grouped by 4 tile-rows.
__device__ __forceinline__ void tile_of(int wg, int gm, int gn, int& tm, int& tn) {
  const int T = gm * gn;
  int L = wg;
  if (T % 8 == 0) L = (wg % 8) * (T / 8) + wg / 8;
  constexpr int GM = 4;
  const int per_group = GM * gn;
  const int g = L / per_group, first = g * GM;
  const int gsz = min(gm - first, GM);
  const int r = L - g * per_group;
  tm = first + r % gsz;
  tn = r / gsz;
}

// ---- epilogue: lane l, reg v -> row 8(v/4) + 4(l/32) + v%4, col l%32 ----
// Shared by both main loops.  The LDS stage buffers are free when it runs.
template <int EPI, int WM, int WN>
__device__ __forceinline__ void gemm_epilogue(f32x16 (&acc)[kBM / WM / 32][kBN / WN / 32], uint8_t* lds,
                                              int lane, int wave, int m0, int n0, int M, int N,
                                              int ldc, float alpha, float* __restrict__ C,
                                              const uint32_t* __restrict__ cmask,
                                              uint32_t sign_mask) {
  constexpr int FM = kBM / WM / 32, FN = kBN / WN / 32;
  const int wm = wave / WN, wn = wave % WN;
  const int fr = lane & 31, fh = lane >> 5;
  const int rowsC = min(kBM, M - m0);
  constexpr uint32_t kCB = EPI == kEpiBf16 ? 2u : 4u;  // bytes per C element
  const rsrc_t rC = make_rsrc(reinterpret_cast<uint8_t*>(C) + (size_t)m0 * ldc * kCB,
                              (uint32_t)rowsC * (uint32_t)ldc * kCB);
  if constexpr (EPI == kEpiF32) {
    // straight from the accumulators: per instruction two 128-B row pieces
    // (measured faster here than staging through LDS for whole-row stores)
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = n0 + wn * (kBN / WN) + j * 32 + fr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wm * (kBM / WM) + i * 32 + 8 * (v / 4) + 4 * fh + (v % 4);
          const uint32_t bad = 0u - (uint32_t)(col >= N);
          const uint32_t off = ((((uint32_t)row * (uint32_t)ldc + (uint32_t)col) * 4u) & ~bad) | (kOOB & bad);
          buf_store4(alpha * acc[i][j][v], rC, off);
        }
      }
    }
  } else {
    // The stage buffers are free after the last barrier: each wave stages
    // one 32-row block of its sub-tile at a time (32 x 128 fp32, row pitch
    // 132 floats) and stores it row by row with 16-B stores.
    // IRHT: before the store every lane takes two whole 32-column groups of
    // the block and replaces each by H^-1((alpha acc) with masked entries
    // zeroed), H^-1 y = s o (c FWHT(y)) (a lane storing its own group would
    // touch 64 cache lines per instruction).  BF16: the store pass rounds
    // eight consecutive values per lane to bf16.
    static_assert(WM * WN * 32 * 132 * 4 <= 2 * kStageLds, "epilogue staging exceeds LDS");
    static_assert(FN * 32 == 128 && kBN / WN == 128, "the store pass assumes 128-column wave sub-tiles");
    float* stg = reinterpret_cast<float*>(lds) + wave * (32 * 132);
    const int gpr = N / 32;  // mask words per row
    const rsrc_t rM = make_rsrc(EPI == kEpiIrht ? cmask + (size_t)m0 * gpr : nullptr,
                                EPI == kEpiIrht ? (uint32_t)rowsC * (uint32_t)gpr * 4u : 0u);
    // IRHT: the lane's mask words of all FM blocks are loaded up front, so
    // their latency overlaps the staging of the first block
    uint32_t mbw[FM][2] = {};
    if constexpr (EPI == kEpiIrht) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int item = lane + 64 * u;             // 32 rows x 4 groups
          const int rl = item >> 2, gq = item & 3;
          const int col0 = n0 + wn * (kBN / WN) + 32 * gq;
          const uint32_t badc = 0u - (uint32_t)(col0 >= N);
          const int row = wm * (kBM / WM) + i * 32 + rl;
          const uint32_t moff = ((((uint32_t)row * (uint32_t)gpr + (uint32_t)(col0 >> 5)) * 4u) & ~badc) | (kOOB & badc);
          mbw[i][u] = buf_load4(rM, moff);
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          stg[(8 * (v / 4) + 4 * fh + (v % 4)) * 132 + 32 * j + fr] = alpha * acc[i][j][v];
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are done
      __builtin_amdgcn_wave_barrier();
      if constexpr (EPI == kEpiIrht) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int item = lane + 64 * u;             // 32 rows x 4 groups
          const int rl = item >> 2, gq = item & 3;
          float t[32];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const float4 w = *reinterpret_cast<const float4*>(stg + rl * 132 + 32 * gq + 4 * q);
            t[4 * q] = w.x; t[4 * q + 1] = w.y; t[4 * q + 2] = w.z; t[4 * q + 3] = w.w;
          }
          const uint32_t mb = mbw[i][u];
#pragma unroll
          for (int e = 0; e < 32; ++e) t[e] = ((mb >> e) & 1u) ? 0.0f : t[e];
#pragma unroll
          for (int h = 1; h < 32; h <<= 1)
#pragma unroll
            for (int e = 0; e < 32; ++e) {
              if (e & h) continue;
              const float a = t[e], b = t[e + h];
              t[e] = a + b;
              t[e + h] = a - b;
            }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            float o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int k = 4 * q + e;
              const float y = t[k] * 0x1.6a09e6p-3f;  // fl32(1/sqrt(32))
              o[e] = __uint_as_float(__float_as_uint(y) ^ (((sign_mask >> k) & 1u) << 31));
            }
            *reinterpret_cast<float4*>(stg + rl * 132 + 32 * gq + 4 * q) = float4{o[0], o[1], o[2], o[3]};
          }
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // the transformed block is in LDS
        __builtin_amdgcn_wave_barrier();
      }
      if constexpr (EPI == kEpiIrht) {
        // row-contiguous stores: one instruction covers two 128-column rows
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int f = 64 * k + lane, rl = f >> 5, c4 = f & 31;
          const float4 w = *reinterpret_cast<const float4*>(stg + rl * 132 + 4 * c4);
          const int row = wm * (kBM / WM) + i * 32 + rl;
          const int col = n0 + wn * (kBN / WN) + 4 * c4;
          const uint32_t bad = 0u - (uint32_t)(col >= N);
          const uint32_t off = ((((uint32_t)row * (uint32_t)ldc + (uint32_t)col) * 4u) & ~bad) | (kOOB & bad);
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned int, w), rC, (int)off, 0, kStoreNT);
        }
      } else {
        // bf16: eight consecutive columns per lane, one instruction covers
        // four 128-column rows
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int f = 64 * k + lane, rl = f >> 4, c8 = f & 15;
          const float4 w0 = *reinterpret_cast<const float4*>(stg + rl * 132 + 8 * c8);
          const float4 w1 = *reinterpret_cast<const float4*>(stg + rl * 132 + 8 * c8 + 4);
          const int row = wm * (kBM / WM) + i * 32 + rl;
          const int col = n0 + wn * (kBN / WN) + 8 * c8;
          const uint32_t bad = 0u - (uint32_t)(col >= N);
          const uint32_t off = ((((uint32_t)row * (uint32_t)ldc + (uint32_t)col) * 2u) & ~bad) | (kOOB & bad);
          const __attribute__((ext_vector_type(4))) unsigned int o = {
              bf16_rne(w0.x) | (bf16_rne(w0.y) << 16), bf16_rne(w0.z) | (bf16_rne(w0.w) << 16),
              bf16_rne(w1.x) | (bf16_rne(w1.y) << 16), bf16_rne(w1.z) | (bf16_rne(w1.w) << 16)};
          __builtin_amdgcn_raw_buffer_store_b128(o, rC, (int)off, 0, kStoreNT);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this block's reads are done before it is overwritten
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Scale-row load modes (SCL): 0 one byte per group (K not a multiple of the
// stage), 1 one 8-B (FP4) or 4-B (FP8) load per row per stage, 2 one 16-B
// load per row every kPack stages (FP4: 2, FP8: 4; K/32 a multiple of 16,
// scale pointers 16-B aligned).  A row's scale bytes for one stage lie in
// their own cache line, so each scale load instruction touches 64 lines;
// mode 2 issues 1/2 (FP4) or 1/4 (FP8) as many (measured bit-identical and
// 0.5-2.5% faster on the FP4 linear-layer shapes, 4-6% on the staged FP8
// GEMM).
template <int FMT, int SCL, int WM, int WN, int EPI>
__global__ __launch_bounds__(WM * WN * 64, WM * WN / 4) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, int M, int N, int K, float alpha,
    const float* __restrict__ ga, const float* __restrict__ gb, float* __restrict__ C, int ldc,
    const uint32_t* __restrict__ cmask, uint32_t sign_mask) {
  using F = Fmt<FMT>;
  using W = Waves<WM, WN>;
  constexpr int kThreads = W::kThreads, FM = W::FM, FN = W::FN;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if (ga) alpha = ga[0] * gb[0];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int gm = (M + kBM - 1) / kBM, gn = (N + kBN - 1) / kBN;
  int tm, tn;
  tile_of(blockIdx.x, gm, gn, tm, tn);
  const int m0 = tm * kBM, n0 = tn * kBN;
  const uint32_t kbytes = FMT == 4 ? (uint32_t)K / 2 : (uint32_t)K;
  const uint32_t kgroups = (uint32_t)K / 32;
  const int rowsA = min(kBM, M - m0), rowsB = min(kBN, N - n0);
  const rsrc_t rA = make_rsrc(A + (size_t)m0 * kbytes, (uint32_t)rowsA * kbytes);
  const rsrc_t rB = make_rsrc(B + (size_t)n0 * kbytes, (uint32_t)rowsB * kbytes);
  const rsrc_t rAs = make_rsrc(As + (size_t)m0 * kgroups, (uint32_t)rowsA * kgroups);
  const rsrc_t rBs = make_rsrc(Bs + (size_t)n0 * kgroups, (uint32_t)rowsB * kgroups);
  const int nst = (K + F::kStageK - 1) / F::kStageK;

  // ---- global -> LDS for one stage ----
  // Codes go straight to LDS: wave w fills 1-KB blocks w*kBlocks .. +kBlocks-1
  // (blocks 0..31 = A rows 8b..8b+7, 32..63 = B rows); lane l of a block
  // writes slot l&7 of row 8b + l/8, i.e. global chunk (l&7) ^ ((row>>1)&7).
  // Scale bytes go through registers and are rearranged after the MFMAs.
  constexpr int kSR = (kBM + kBN) / kThreads;  // scale rows per thread (2 or 1)
  uint32_t rsw[kSR][2];  // raw scale words of this thread's scale rows (8 groups)
  uint32_t rsq[kSR][4] = {};  // SCL 2: 16 B of scale bytes = kPack stages
  uint32_t rsb[kSR][8];  // byte-wise scale loads (K not a stage multiple)
  constexpr int kPack = 16 / F::kGroups;
  // Per-lane part of the load offsets: row 8b + l/8 of block b and the
  // swizzled chunk, which depends only on the parity of b (rows 8b..8b+7
  // have (row >> 1) & 7 = 4 (b & 1) + (l/8)/2).  The block part b*8*kbytes is
  // wave-uniform.  Rows past the tile edge fall outside the buffer's range.
  const uint32_t lrow8 = (uint32_t)lane >> 3;
  const uint32_t c_even = ((uint32_t)lane & 7u) ^ ((lrow8 >> 1) & 7u);
  const uint32_t c_odd = ((uint32_t)lane & 7u) ^ ((4u + (lrow8 >> 1)) & 7u);
  const uint32_t vrow = lrow8 * kbytes;
  // part p of NP issues this wave's code blocks p*kBlocks/NP .. (p+1)*kBlocks/NP-1
  // (on = false: the loads are issued with out-of-range offsets and write
  // zeros into the idle buffer; this keeps the substep free of branches)
  auto gload_codes = [&](int st, int buf, int part, int nparts, bool on) {
    uint8_t* base = lds + buf * kStageLds;
    const uint32_t kb0 = (uint32_t)st * kRowBytes;
    // lanes whose chunk lies past the row end (or all lanes when !on) get
    // an out-of-range offset; done with masks so the code stays branch-free
    const uint32_t all_off = on ? 0u : 0xFFFFFFFFu;
    const int per = W::kBlocks / nparts;
#pragma unroll
    for (int q = 0; q < per; ++q) {
      const int blk = wave * W::kBlocks + part * per + q;   // wave-uniform
      const bool isA = blk < kBM / 8;
      const uint32_t c = (blk & 1) ? c_odd : c_even;
      const uint32_t kk = kb0 + c * 16;
      uint32_t off = vrow + (uint32_t)((blk & (kBM / 8 - 1)) * 8) * kbytes + kk;
      const uint32_t bad = all_off | (0u - (uint32_t)(kk >= kbytes));
      off = (off & ~bad) | (kOOB & bad);
      buf_load16_lds(isA ? rA : rB, base + blk * 1024, off);
    }
  };
  auto gload_scales = [&](int st, bool on) {
    const uint32_t g0 = (uint32_t)st * F::kGroups;
    const uint32_t all_off = on ? 0u : 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kSR; ++w) {
      // scale row of this thread: A rows for w == 0 (kSR 2) or waves 0..3 (kSR 1)
      const bool isA = kSR == 2 ? w == 0 : wave < 4;
      const rsrc_t rr = isA ? rAs : rBs;
      const uint32_t base_s =
          (((uint32_t)(kSR == 2 ? tid : tid & 255) * kgroups + g0) & ~all_off) | (kOOB & all_off);
      if constexpr (SCL == 2) {
        // wave-uniform: the first stage of each pack fetches the whole pack
        if (st % kPack == 0) {
          const i32x4 v = buf_load16(rr, base_s);
#pragma unroll
          for (int q = 0; q < 4; ++q) rsq[w][q] = (uint32_t)v[q];
        }
      } else if constexpr (SCL == 1) {
        if constexpr (F::kGroups == 8) {
          const i32x2 v = buf_load8(rr, base_s);
          rsw[w][0] = (uint32_t)v.x;
          rsw[w][1] = (uint32_t)v.y;
        } else {
          rsw[w][0] = buf_load4(rr, base_s);
          rsw[w][1] = 0;
        }
      } else {
        rsw[w][0] = rsw[w][1] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = on && j < F::kGroups && g0 + j < kgroups;
          rsb[w][j] = buf_load1(rr, ok ? base_s + j : kOOB);
        }
      }
    }
  };
  // st: the stage whose scales are stored
  auto sstore = [&](int buf, int st) {
    uint8_t* base = lds + buf * kStageLds;
    if constexpr (SCL == 2) {
      const bool odd = st & 1;  // wave-uniform
#pragma unroll
      for (int w = 0; w < kSR; ++w) {
        if constexpr (kPack == 2) {
          rsw[w][0] = odd ? rsq[w][2] : rsq[w][0];
          rsw[w][1] = odd ? rsq[w][3] : rsq[w][1];
        } else {
          const uint32_t s01 = odd ? rsq[w][1] : rsq[w][0];
          const uint32_t s23 = odd ? rsq[w][3] : rsq[w][2];
          rsw[w][0] = (st & 2) ? s23 : s01;
          rsw[w][1] = 0;
        }
      }
    }
    // dword h of a row holds groups h, 2+h, 4+h, 6+h: in K-substep s the
    // lanes of half h carry group 2s+h's scale (byte s, picked by op_sel)
    uint32_t* sp = reinterpret_cast<uint32_t*>(base + kCodeLds);
#pragma unroll
    for (int w = 0; w < kSR; ++w) {
      uint32_t b[8];
      if constexpr (SCL >= 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = (rsw[w][0] >> (8 * j)) & 0xFFu;
          b[4 + j] = (rsw[w][1] >> (8 * j)) & 0xFFu;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = rsb[w][j];
      }
      const int row = kSR == 2 ? w * kBM + tid : tid;
      sp[row * 2] = b[0] | (b[2] << 8) | (b[4] << 16) | (b[6] << 24);
      sp[row * 2 + 1] = b[1] | (b[3] << 8) | (b[5] << 16) | (b[7] << 24);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fh = lane >> 5;
  const int arow0 = wm * (kBM / WM) + fr, brow0 = kBM + wn * (kBN / WN) + fr;

  // fragment of row `row` (0..511 over A then B) for K-substep s:
  // FP4: chunk 2s+h; FP8: chunks 4s+h and 4s+2+h
  auto frag = [&](const uint8_t* base, int row, int s) -> i32x8 {
    const int r = row & (kBM - 1);
    const uint8_t* rb = base + (row >= kBM ? kBM * kRowBytes : 0);
    if constexpr (FMT == 4) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(rb + lds_slot(r, 2 * s + fh));
      return i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    } else {
      const i32x4 v = *reinterpret_cast<const i32x4*>(rb + lds_slot(r, 4 * s + fh));
      const i32x4 u = *reinterpret_cast<const i32x4*>(rb + lds_slot(r, 4 * s + 2 + fh));
      return i32x8{v.x, v.y, v.z, v.w, u.x, u.y, u.z, u.w};
    }
  };

  gload_codes(0, 0, 0, 1, true);
  gload_scales(0, true);
  sstore(0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) lgkmcnt(0): stage 0 is in LDS
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const uint8_t* base = lds + (st & 1) * kStageLds;
    const bool more = st + 1 < nst;
    // the last stage loads nothing (every offset is out of range) but keeps
    // the loop body a single basic block
    gload_scales(st + 1, more);
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(base + kCodeLds);
    uint32_t sca[FM], scb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) sca[i] = sb[(arow0 + 32 * i) * 2 + fh];
#pragma unroll
    for (int j = 0; j < FN; ++j) scb[j] = sb[(brow0 + 32 * j) * 2 + fh];
    // One wave per SIMD (4 waves): double-buffer the fragments so the next
    // K-substep's LDS reads overlap this substep's MFMAs.  Two waves per SIMD
    // (8 waves): single buffer; the sibling wave covers the LDS latency.
    constexpr int NB = W::kMinWaves == 1 ? 2 : 1;
    i32x8 fa[NB][FM], fb[NB][FN];
    if constexpr (NB == 2) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[0][i] = frag(base, arow0 + 32 * i, 0);
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[0][j] = frag(base, brow0 + 32 * j, 0);
    }
    // substep S: the FM x FN MFMAs of S interleaved (in issue order) with the
    // LDS reads of S+1's fragments and a share of the next stage's global
    // loads, so that no more than a few LDS reads are outstanding when an
    // MFMA is due; op_sel S picks the scale byte of group 2S+h.
    auto sub = [&](auto SC) {
      constexpr int S = decltype(SC)::value;
      constexpr int cur = NB == 2 ? (S & 1) : 0;
      constexpr int NP = F::kSub;  // global-load parts, one per substep
      if constexpr (NB == 1) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[0][i] = frag(base, arow0 + 32 * i, S);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[0][j] = frag(base, brow0 + 32 * j, S);
      }
      gload_codes(st + 1, (st + 1) & 1, S, NP, more);
      if constexpr (NB == 2 && S + 1 < F::kSub) {
#pragma unroll
        for (int i = 0; i < FM; ++i) fa[cur ^ 1][i] = frag(base, arow0 + 32 * i, S + 1);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[cur ^ 1][j] = frag(base, brow0 + 32 * j, S + 1);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[cur][i], fb[cur][j], acc[i][j], FMT, FMT, S, (int)sca[i], S, (int)scb[j]);
      if constexpr (NB == 2) {
        // issue order: per group {MFMA, DS read, MFMA, VMEM, ...}
        constexpr int nmf = FM * FN;
        constexpr int nds = S + 1 < F::kSub ? (FM + FN) * (FMT == 4 ? 1 : 2) : 0;
        constexpr int nvm = W::kBlocks / NP;
#pragma unroll
        for (int g = 0; g < nmf; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
          if (g < nds) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
          if (g < nvm) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // VMEM read
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    if constexpr (F::kSub > 2) {
      sub(std::integral_constant<int, 2>{});
      sub(std::integral_constant<int, 3>{});
    }
    sstore((st + 1) & 1, st + 1);
    // keep this stage's MFMAs above the wait: otherwise the scheduler sinks
    // them below it and the next stage's loads stop overlapping the math
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0);  // the next stage's LDS-direct loads have landed
    __syncthreads();
  }

  gemm_epilogue<EPI, WM, WN>(acc, lds, lane, wave, m0, n0, M, N, ldc, alpha, C, cmask, sign_mask);
}

template <int FMT, int SCL, int WM, int WN, int EPI>
hipError_t gemm_launch_cfg(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           int64_t m, int64_t n, int64_t k, float alpha, const float* ga,
                           const float* gb, float* c, int64_t ldc, const uint32_t* cmask,
                           uint32_t sign_mask, hipStream_t s) {
  const size_t lds = 2 * (size_t)kStageLds;
  const void* fn = reinterpret_cast<const void*>(&mx_gemm_kernel<FMT, SCL, WM, WN, EPI>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  hipLaunchKernelGGL((mx_gemm_kernel<FMT, SCL, WM, WN, EPI>), dim3((unsigned)tiles),
                     dim3(Waves<WM, WN>::kThreads), lds, s, a, as, b, bs, (int)m, (int)n, (int)k,
                     alpha, ga, gb, c, (int)ldc, cmask, sign_mask);
  return hipGetLastError();
}

template <int FMT, int EPI>
hipError_t gemm_launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                       int64_t m, int64_t n, int64_t k, float alpha, const float* ga,
                       const float* gb, float* c, int64_t ldc, const uint32_t* cmask,
                       uint32_t sign_mask, hipStream_t s) {
  // scale rows split into whole per-stage words when K is a stage multiple,
  // and into whole 16-B packs when K/32 is a multiple of 16
  const int64_t kg = k / 32;
  const bool a16 = (((uintptr_t)as | (uintptr_t)bs) & 15u) == 0;
  if (kg % 16 == 0 && a16)
    return gemm_launch_cfg<FMT, 2, FP4MX_GEMM_WM, FP4MX_GEMM_WN, EPI>(
        a, as, b, bs, m, n, k, alpha, ga, gb, c, ldc, cmask, sign_mask, s);
  if (kg % Fmt<FMT>::kGroups == 0)
    return gemm_launch_cfg<FMT, 1, FP4MX_GEMM_WM, FP4MX_GEMM_WN, EPI>(
        a, as, b, bs, m, n, k, alpha, ga, gb, c, ldc, cmask, sign_mask, s);
  return gemm_launch_cfg<FMT, 0, FP4MX_GEMM_WM, FP4MX_GEMM_WN, EPI>(
      a, as, b, bs, m, n, k, alpha, ga, gb, c, ldc, cmask, sign_mask, s);
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, float alpha, float* c, int64_t ldc,
                          hipStream_t s) {
  return gemm_launch<4, kEpiF32>(a, as, b, bs, m, n, k, alpha, nullptr, nullptr, c, ldc, nullptr, 0u, s);
}

hipError_t launch_mx_gemm_irht(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                               const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha,
                               float* c, int64_t ldc, const uint8_t* cmask, uint32_t sign_mask,
                               hipStream_t s) {
  return gemm_launch<4, kEpiIrht>(a, as, b, bs, m, n, k, alpha, nullptr, nullptr, c, ldc,
                                  reinterpret_cast<const uint32_t*>(cmask), sign_mask, s);
}

hipError_t launch_mx_gemm_bf16(const uint8_t* a, const uint8_t* as, const uint8_t* b,
                               const uint8_t* bs, int64_t m, int64_t n, int64_t k, float alpha,
                               uint16_t* c, int64_t ldc, hipStream_t s) {
  return gemm_launch<4, kEpiBf16>(a, as, b, bs, m, n, k, alpha, nullptr, nullptr,
                                  reinterpret_cast<float*>(c), ldc, nullptr, 0u, s);
}

hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           const float* ga, const float* gb, int64_t m, int64_t n, int64_t k,
                           float* c, int64_t ldc, hipStream_t s) {
  return gemm_launch<0, kEpiF32>(a, as, b, bs, m, n, k, 1.0f, ga, gb, c, ldc, nullptr, 0u, s);
}

}  // namespace fp4mx
