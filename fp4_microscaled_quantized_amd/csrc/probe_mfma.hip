// Sustained-rate probe for the scaled MFMA the GEMMs are built on
// (v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 or FP8 operands and E8M0 scales), with
// no memory traffic in the timed loop, plus the shader clock during the run.
// Built as its own library (libfp4mx_probe.so) for the benchmark's measured
// roofline; not part of the fp4mx.h ABI.
//
// Each wave keeps the GEMM's register layout -- 4 x 4 fragments of 32 x 32
// fp32 accumulators, operand fragments of 32 FP4 codes or 32 FP8 bytes per
// lane -- and issues
// 16 independent MFMAs per iteration.  Operand words come from `words`
// (random bits, or zeros for the low-toggle case), so the pipe sees the same
// kind of data as in a real GEMM.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// FMT 4: FP4 operands (the low 4 dwords of each fragment carry 32 codes);
// FMT 0: FP8 E4M3 operands (all 8 dwords, 32 bytes per lane).
template <int FMT>
__global__ __launch_bounds__(256) void mfma_probe(const uint32_t* __restrict__ words, int iters,
                                                  float* __restrict__ sink,
                                                  uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  constexpr int NW = FMT == 4 ? 4 : 8;  // live dwords per fragment
  i32x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int va[8] = {0, 0, 0, 0, 0, 0, 0, 0}, vb[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int d = 0; d < NW; ++d) {
      va[d] = (int)words[(i * 8 + d) * 64 + lane];
      vb[d] = (int)words[(32 + i * 8 + d) * 64 + lane];
    }
    a[i] = i32x8{va[0], va[1], va[2], va[3], va[4], va[5], va[6], va[7]};
    b[i] = i32x8{vb[0], vb[1], vb[2], vb[3], vb[4], vb[5], vb[6], vb[7]};
  }
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FMT, FMT,
                                                                   0, 127, 0, 127);
  }
  __builtin_amdgcn_s_waitcnt(0);
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[i][j][v];
  sink[blockIdx.x * 256u + threadIdx.x] = s;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    clocks[0] = t0;
    clocks[1] = t1;
    clocks[2] = r0;
    clocks[3] = r1;
  }
}

}  // namespace

// fmt: 4 = FP4, 0 = FP8 (E4M3).  words: 64 x 64 uint32 (device); sink:
// blocks * 256 floats; clocks: 4 uint64 (shader-clock and 100-MHz reference
// counters at the start and end of the timed loop of block 0).  Returns the
// hipError_t of the launch.
extern "C" __attribute__((visibility("default"))) int fp4mx_probe_mfma(
    int fmt, const uint32_t* words, int iters, int blocks, float* sink, uint64_t* clocks,
    void* stream) {
  if (!words || !sink || !clocks || iters <= 0 || blocks <= 0) return (int)hipErrorInvalidValue;
  if (fmt == 4)
    hipLaunchKernelGGL(mfma_probe<4>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       words, iters, sink, clocks);
  else if (fmt == 0)
    hipLaunchKernelGGL(mfma_probe<0>, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       words, iters, sink, clocks);
  else
    return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}
