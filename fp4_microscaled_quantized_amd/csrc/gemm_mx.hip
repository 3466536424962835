// Block-scaled GEMM on gfx950 MFMA: MXFP4 x MXFP4 -> fp32, and the FP8 (E4M3)
// variant used by the NVFP4 path.
//
// Computes C = alpha * deq(A) deq(B)^T with A [m][k], B [n][k] stored K-major
// (FP4: two codes per byte; FP8: one per byte) and one E8M0 scale per 32 K
// elements per row; fp32 accumulation and output.
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
//  - LDS rows are padded to 144 B (the 16-B fragment reads of 8 consecutive
//    rows hit distinct banks); each row's stage scales are stored as two
//    dwords holding groups {h, 2+h, 4+h, 6+h}, byte s selected by op_sel.
//  - Tiles are assigned XCD-aware: workgroup i runs on XCD i % 8, so each XCD
//    gets a contiguous run of tiles in grouped (4 tile-rows) order and shares
//    A and B panels in its own L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fp4mx_internal.h"

namespace fp4mx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 256, kBN = 256, kThreads = 256;
constexpr int kRowBytes = 128;              // operand bytes per row per stage
constexpr int kPitch = kRowBytes + 16;      // padded LDS row
constexpr int kCodeLds = (kBM + kBN) * kPitch;
constexpr int kScaleLds = (kBM + kBN) * 8;
constexpr int kStageLds = kCodeLds + kScaleLds;
constexpr int kLoads = (kBM + kBN) * (kRowBytes / 16) / kThreads;  // 16 per thread
constexpr uint32_t kOOB = 0x80000000u;      // offset beyond any num_records

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
__device__ __forceinline__ void buf_store4(float v, rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)off, 0, 0);
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

template <int FMT, bool VEC>
__global__ __launch_bounds__(kThreads, 1) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, int M, int N, int K, float alpha,
    const float* __restrict__ ga, const float* __restrict__ gb, float* __restrict__ C, int ldc) {
  using F = Fmt<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if (ga) alpha = ga[0] * gb[0];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
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

  // ---- global -> registers for one stage ----
  // Thread t loads 16-B chunk (t & 7) of rows t/8 + 32 i (i = 0..7) of A and
  // of B; a K chunk beyond the row end reads as zero through an OOB offset.
  i32x4 rga[kLoads / 2], rgb[kLoads / 2];
  uint32_t rsw[2][2];  // raw scale words of A row tid / B row tid (8 groups)
  uint32_t rsb[2][8];  // byte-wise scale loads (K not a stage multiple)
  const uint32_t lrow = (uint32_t)tid >> 3, lch = (uint32_t)tid & 7;
  auto gload = [&](int st) {
    const uint32_t kk = (uint32_t)st * kRowBytes + lch * 16;
    const bool kin = kk < kbytes;
#pragma unroll
    for (int i = 0; i < kLoads / 2; ++i) {
      const uint32_t off = (lrow + 32u * i) * kbytes + kk;
      rga[i] = buf_load16(rA, kin ? off : kOOB);
      rgb[i] = buf_load16(rB, kin ? off : kOOB);
    }
    // raw scale words; they are only rearranged in sstore, after the MFMAs,
    // so that no wait on this stage's loads happens before compute
    const uint32_t g0 = (uint32_t)st * F::kGroups, base = (uint32_t)tid * kgroups + g0;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const rsrc_t rr = w == 0 ? rAs : rBs;
      if constexpr (VEC) {
        if constexpr (F::kGroups == 8) {
          const i32x2 v = buf_load8(rr, base);
          rsw[w][0] = (uint32_t)v.x;
          rsw[w][1] = (uint32_t)v.y;
        } else {
          rsw[w][0] = buf_load4(rr, base);
          rsw[w][1] = 0;
        }
      } else {
        rsw[w][0] = rsw[w][1] = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool ok = j < F::kGroups && g0 + j < kgroups;
          rsb[w][j] = buf_load1(rr, ok ? base + j : kOOB);
        }
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = lds + buf * kStageLds;
#pragma unroll
    for (int i = 0; i < kLoads / 2; ++i) {
      *reinterpret_cast<i32x4*>(base + (lrow + 32 * i) * kPitch + lch * 16) = rga[i];
      *reinterpret_cast<i32x4*>(base + (kBM + lrow + 32 * i) * kPitch + lch * 16) = rgb[i];
    }
    // dword h of a row holds groups h, 2+h, 4+h, 6+h: in K-substep s the
    // lanes of half h carry group 2s+h's scale (byte s, picked by op_sel)
    uint32_t* sp = reinterpret_cast<uint32_t*>(base + kCodeLds);
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t b[8];
      if constexpr (VEC) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          b[j] = (rsw[w][0] >> (8 * j)) & 0xFFu;
          b[4 + j] = (rsw[w][1] >> (8 * j)) & 0xFFu;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) b[j] = rsb[w][j];
      }
      const int row = w * kBM + tid;
      sp[row * 2] = b[0] | (b[2] << 8) | (b[4] << 16) | (b[6] << 24);
      sp[row * 2 + 1] = b[1] | (b[3] << 8) | (b[5] << 16) | (b[7] << 24);
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int fr = lane & 31, fh = lane >> 5;
  const int arow0 = wm * 128 + fr, brow0 = kBM + wn * 128 + fr;

  auto frag = [&](const uint8_t* base, int row, int s) -> i32x8 {
    const uint8_t* p = base + row * kPitch + s * F::kSubBytes + fh * 16;
    const i32x4 v = *reinterpret_cast<const i32x4*>(p);
    if constexpr (FMT == 4) {
      return i32x8{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
    } else {
      const i32x4 u = *reinterpret_cast<const i32x4*>(p + 32);
      return i32x8{v.x, v.y, v.z, v.w, u.x, u.y, u.z, u.w};
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const uint8_t* base = lds + (st & 1) * kStageLds;
    if (st + 1 < nst) gload(st + 1);
    const uint32_t* sb = reinterpret_cast<const uint32_t*>(base + kCodeLds);
    uint32_t sca[4], scb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sca[i] = sb[(arow0 + 32 * i) * 2 + fh];
      scb[i] = sb[(brow0 + 32 * i) * 2 + fh];
    }
    i32x8 fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fa[0][i] = frag(base, arow0 + 32 * i, 0);
      fb[0][i] = frag(base, brow0 + 32 * i, 0);
    }
    // substep S: prefetch S+1's fragments, then 16 MFMAs; op_sel S picks the
    // scale byte of group 2S+h from each lane's scale dword
    auto sub = [&](auto SC) {
      constexpr int S = decltype(SC)::value;
      constexpr int cur = S & 1;
      if constexpr (S + 1 < F::kSub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fa[cur ^ 1][i] = frag(base, arow0 + 32 * i, S + 1);
          fb[cur ^ 1][i] = frag(base, brow0 + 32 * i, S + 1);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[cur][i], fb[cur][j], acc[i][j], FMT, FMT, S, (int)sca[i], S, (int)scb[j]);
    };
    sub(std::integral_constant<int, 0>{});
    sub(std::integral_constant<int, 1>{});
    if constexpr (F::kSub > 2) {
      sub(std::integral_constant<int, 2>{});
      sub(std::integral_constant<int, 3>{});
    }
    if (st + 1 < nst) sstore((st + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane l, reg v -> row 8(v/4) + 4(l/32) + v%4, col l%32 ----
  const int rowsC = min(kBM, M - m0);
  const rsrc_t rC = make_rsrc(C + (size_t)m0 * ldc, (uint32_t)rowsC * (uint32_t)ldc * 4u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + fr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * 128 + i * 32 + 8 * (v / 4) + 4 * fh + (v % 4);
        const uint32_t off = col < N ? ((uint32_t)row * (uint32_t)ldc + (uint32_t)col) * 4u : kOOB;
        buf_store4(alpha * acc[i][j][v], rC, off);
      }
    }
  }
}

template <int FMT>
hipError_t gemm_launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                       int64_t m, int64_t n, int64_t k, float alpha, const float* ga,
                       const float* gb, float* c, int64_t ldc, hipStream_t s) {
  const size_t lds = 2 * (size_t)kStageLds;
  // scale rows split into whole per-stage words when K is a stage multiple
  const bool vec = (k / 32) % Fmt<FMT>::kGroups == 0;
  const void* fn = vec ? reinterpret_cast<const void*>(&mx_gemm_kernel<FMT, true>)
                       : reinterpret_cast<const void*>(&mx_gemm_kernel<FMT, false>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + kBM - 1) / kBM) * ((n + kBN - 1) / kBN);
  if (vec)
    hipLaunchKernelGGL((mx_gemm_kernel<FMT, true>), dim3((unsigned)tiles), dim3(kThreads), lds, s,
                       a, as, b, bs, (int)m, (int)n, (int)k, alpha, ga, gb, c, (int)ldc);
  else
    hipLaunchKernelGGL((mx_gemm_kernel<FMT, false>), dim3((unsigned)tiles), dim3(kThreads), lds, s,
                       a, as, b, bs, (int)m, (int)n, (int)k, alpha, ga, gb, c, (int)ldc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, float alpha, float* c, int64_t ldc,
                          hipStream_t s) {
  return gemm_launch<4>(a, as, b, bs, m, n, k, alpha, nullptr, nullptr, c, ldc, s);
}

hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           const float* ga, const float* gb, int64_t m, int64_t n, int64_t k,
                           float* c, int64_t ldc, hipStream_t s) {
  return gemm_launch<0>(a, as, b, bs, m, n, k, 1.0f, ga, gb, c, ldc, s);
}

}  // namespace fp4mx
