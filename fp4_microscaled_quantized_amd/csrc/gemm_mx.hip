// MXFP4 x MXFP4 -> fp32 GEMM on gfx950 block-scaled FP4 MFMA.
//
// Computes C = alpha * deq(A) deq(B)^T with A [m][k], B [n][k] MXFP4
// (K-major codes + one E8M0 scale per 32 K-elements), fp32 accumulation.
// Source: "Quartet: Native FP4 Training Can Be Optimal for Large Language
// Models" -- "The GPU Kernel Implementation", Stage 2 (block-scaled GEMM
// D = C + (A x SFA)(B x SFB), FP32 accumulator and output).
//
// Design (MI355X):
//  - v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands: lane l holds row l%32
//    and the 32 contiguous K elements [32*(l/32), +32) of its 32x64 fragment
//    (16 bytes, exactly one MXFP4 group), plus that group's E8M0 scale -- so
//    the canonical K-major layout written by the quantizers is fed as is and
//    no scale rearrangement pass exists.
//  - A workgroup computes a BM x BN tile; K advances in stages of 256 elements
//    (128 code bytes per row) staged through LDS, double buffered: the global
//    loads of stage s+1 are in flight while the MFMAs of stage s run.
//  - LDS rows are padded to 144 B so the 16-B fragment reads of 8 consecutive
//    rows hit distinct banks.  Scale bytes are stored per row as two dwords
//    holding groups {h, 2+h, 4+h, 6+h}, so each lane reads one dword per stage.
//  - K, M and N tails are zero-filled (codes 0, scale 2^0), outputs guarded.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp4mx_internal.h"

namespace fp4mx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStageBytes = 128;          // operand bytes per row per stage
constexpr int kPitch = kStageBytes + 16;  // padded LDS row (bytes)

template <int FMT, int BM, int BN, int WM, int WN>
struct GemmCfg {
  // FMT 4: FP4, 256 K per stage (8 groups); FMT 0: FP8, 128 K per stage (4 groups)
  static constexpr int kStageK = FMT == 4 ? 256 : 128;
  static constexpr int kScalesPerStage = kStageK / 32;
  static constexpr int kSub = kStageK / 64;          // 32x32x64 MFMAs per stage along K
  static constexpr int kSubBytes = kStageBytes / kSub;
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  static constexpr int FM = TM / 32, FN = TN / 32;  // 32x32 fragments per wave
  static constexpr int kCodeBytes = (BM + BN) * kPitch;
  static constexpr int kScaleBytes = (BM + BN) * 8;
  static constexpr int kStageLds = kCodeBytes + kScaleBytes;
  static constexpr int kChunksA = BM * (kStageBytes / 16), kChunksB = BN * (kStageBytes / 16);
  static constexpr int kLoadsA = kChunksA / kThreads, kLoadsB = kChunksB / kThreads;
  static_assert(kChunksA % kThreads == 0 && kChunksB % kThreads == 0, "tile/threads");
};

template <int FMT, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void mx_gemm_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ Bs, int64_t M, int64_t N, int64_t K, float alpha,
    const float* __restrict__ ga, const float* __restrict__ gb, float* __restrict__ C, int64_t ldc) {
  using Cfg = GemmCfg<FMT, BM, BN, WM, WN>;
  constexpr int kStageK = Cfg::kStageK, kScalesPerStage = Cfg::kScalesPerStage;
  if (ga) alpha = ga[0] * gb[0];
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int64_t kbytes = FMT == 4 ? K / 2 : K, kgroups = K / 32;
  const int nstages = (int)((K + kStageK - 1) / kStageK);

  // ---- global -> register staging of one stage ----
  u32x4 ra[Cfg::kLoadsA], rb[Cfg::kLoadsB];
  uint32_t rsc[2];  // scale dwords (only threads < BM+BN use them)
  auto gload = [&](int st) {
    const int64_t kb0 = (int64_t)st * kStageBytes;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int id = tid + i * Cfg::kThreads, r = id / (kStageBytes / 16), ch = id % (kStageBytes / 16);
      const int64_t gr = m0 + r, gk = kb0 + ch * 16;
      ra[i] = (gr < M && gk < kbytes) ? *reinterpret_cast<const u32x4*>(A + gr * kbytes + gk)
                                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int id = tid + i * Cfg::kThreads, r = id / (kStageBytes / 16), ch = id % (kStageBytes / 16);
      const int64_t gr = n0 + r, gk = kb0 + ch * 16;
      rb[i] = (gr < N && gk < kbytes) ? *reinterpret_cast<const u32x4*>(B + gr * kbytes + gk)
                                      : u32x4{0, 0, 0, 0};
    }
    if (tid < BM + BN) {
      const bool isA = tid < BM;
      const int r = isA ? tid : tid - BM;
      const int64_t gr = (isA ? m0 : n0) + r, lim = isA ? M : N;
      const uint8_t* S = isA ? As : Bs;
      uint32_t b[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int64_t g = (int64_t)st * kScalesPerStage + j;
        b[j] = (j < kScalesPerStage && gr < lim && g < kgroups) ? S[gr * kgroups + g] : 127u;
      }
      // dword h holds groups h, 2+h, 4+h, 6+h (byte s = group 2s+h): in
      // K-substep s the lanes of half h carry group 2s+h's scale.
      rsc[0] = b[0] | (b[2] << 8) | (b[4] << 16) | (b[6] << 24);
      rsc[1] = b[1] | (b[3] << 8) | (b[5] << 16) | (b[7] << 24);
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = lds + buf * Cfg::kStageLds;
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsA; ++i) {
      const int id = tid + i * Cfg::kThreads, r = id / (kStageBytes / 16), ch = id % (kStageBytes / 16);
      *reinterpret_cast<u32x4*>(base + r * kPitch + ch * 16) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < Cfg::kLoadsB; ++i) {
      const int id = tid + i * Cfg::kThreads, r = id / (kStageBytes / 16), ch = id % (kStageBytes / 16);
      *reinterpret_cast<u32x4*>(base + (BM + r) * kPitch + ch * 16) = rb[i];
    }
    if (tid < BM + BN) {
      uint32_t* s = reinterpret_cast<uint32_t*>(base + Cfg::kCodeBytes) + tid * 2;
      s[0] = rsc[0];
      s[1] = rsc[1];
    }
  };

  f32x16 acc[Cfg::FM][Cfg::FN];
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i)
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  gload(0);
  sstore(0);
  __syncthreads();

  const int fr = lane & 31, fh = lane >> 5;
  for (int st = 0; st < nstages; ++st) {
    const int buf = st & 1;
    if (st + 1 < nstages) gload(st + 1);
    const uint8_t* base = lds + buf * Cfg::kStageLds;
    const uint32_t* sbase = reinterpret_cast<const uint32_t*>(base + Cfg::kCodeBytes);
    uint32_t sa[Cfg::FM], sb[Cfg::FN];
#pragma unroll
    for (int i = 0; i < Cfg::FM; ++i) sa[i] = sbase[(wm * Cfg::TM + i * 32 + fr) * 2 + fh];
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) sb[j] = sbase[(BM + wn * Cfg::TN + j * 32 + fr) * 2 + fh];
#pragma unroll
    for (int s = 0; s < Cfg::kSub; ++s) {
      i32x8 fa[Cfg::FM], fb[Cfg::FN];
      // FP4: lane half h holds K [32h, 32h+32) of the 64-K substep (16 B).
      // FP8: lane half h holds K [16h, 16h+16) and [32+16h, 32+16h+16).
      auto frag = [&](int row) -> i32x8 {
        const uint8_t* p = base + row * kPitch + s * Cfg::kSubBytes;
        if constexpr (FMT == 4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(p + fh * 16);
          return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        } else {
          const u32x4 v = *reinterpret_cast<const u32x4*>(p + fh * 16);
          const u32x4 u = *reinterpret_cast<const u32x4*>(p + 32 + fh * 16);
          return i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, (int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
      };
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i) fa[i] = frag(wm * Cfg::TM + i * 32 + fr);
#pragma unroll
      for (int j = 0; j < Cfg::FN; ++j) fb[j] = frag(BM + wn * Cfg::TN + j * 32 + fr);
#pragma unroll
      for (int i = 0; i < Cfg::FM; ++i) {
        const int sca = (int)((sa[i] >> (8 * s)) & 0xFFu);
#pragma unroll
        for (int j = 0; j < Cfg::FN; ++j) {
          const int scb = (int)((sb[j] >> (8 * s)) & 0xFFu);
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], FMT,
                                                                      FMT, 0, sca, 0, scb);
        }
      }
    }
    if (st + 1 < nstages) sstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane l, reg v -> row 8(v/4) + 4(l/32) + v%4, col l%32 ----
#pragma unroll
  for (int i = 0; i < Cfg::FM; ++i) {
#pragma unroll
    for (int j = 0; j < Cfg::FN; ++j) {
      const int64_t col = n0 + wn * Cfg::TN + j * 32 + fr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * Cfg::TM + i * 32 + 8 * (v / 4) + 4 * fh + (v % 4);
        if (row < M && col < N) __builtin_nontemporal_store(alpha * acc[i][j][v], C + row * ldc + col);
      }
    }
  }
}

template <int FMT, int BM, int BN, int WM, int WN>
hipError_t gemm_launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                       int64_t m, int64_t n, int64_t k, float alpha, const float* ga,
                       const float* gb, float* c, int64_t ldc, hipStream_t s) {
  using Cfg = GemmCfg<FMT, BM, BN, WM, WN>;
  const size_t lds = 2 * (size_t)Cfg::kStageLds;
  // The attribute is per device; setting it on every call is cheap and keeps
  // multi-device processes correct.
  hipError_t e = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&mx_gemm_kernel<FMT, BM, BN, WM, WN>),
      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)((m + BM - 1) / BM));
  hipLaunchKernelGGL((mx_gemm_kernel<FMT, BM, BN, WM, WN>), grid, dim3(Cfg::kThreads), lds, s, a,
                     as, b, bs, m, n, k, alpha, ga, gb, c, ldc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mx_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                          int64_t m, int64_t n, int64_t k, float alpha, float* c, int64_t ldc,
                          hipStream_t s) {
  return gemm_launch<4, 128, 128, 2, 2>(a, as, b, bs, m, n, k, alpha, nullptr, nullptr, c, ldc, s);
}

hipError_t launch_fp8_gemm(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                           const float* ga, const float* gb, int64_t m, int64_t n, int64_t k,
                           float* c, int64_t ldc, hipStream_t s) {
  return gemm_launch<0, 128, 128, 2, 2>(a, as, b, bs, m, n, k, 1.0f, ga, gb, c, ldc, s);
}

}  // namespace fp4mx
