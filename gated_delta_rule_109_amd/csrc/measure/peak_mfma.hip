// Measurement helper, not part of the KDA library: loops of independent bf16
// MFMAs, to measure the dense bf16 matrix rate the chip reaches, as a
// reference beside the vendor peak. Two shapes: v_mfma_f32_16x16x32_bf16 (the
// one the KDA kernels use) and v_mfma_f32_32x32x16_bf16.
//
// Each wave keeps kChains independent accumulators, so the MFMA pipe never
// waits on a result. Nothing is stored unless iters < 0 (never true for a
// real call; the compiler cannot know that, so the work is kept).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kChains = 8;

template <int kShape>
__global__ __launch_bounds__(256) void mfma_loop(float* sink, int iters) {
  using Acc = typename std::conditional<kShape == 0, f32x4, f32x16>::type;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 5);
  }
  Acc acc[kChains];
#pragma unroll
  for (int j = 0; j < kChains; ++j) acc[j] = Acc{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      if constexpr (kShape == 0) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
      else acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kChains; ++j)
#pragma unroll
    for (int e = 0; e < (kShape == 0 ? 4 : 16); ++e) s += acc[j][e];
  if (iters < 0) sink[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// FLOPs one launch performs: blocks x 4 waves x iters x kChains x M*N*K*2
// (16*16*32 for shape 0, 32*32*16 for shape 1).
double kda_peak_mfma_flops(int32_t shape, int32_t blocks, int32_t iters) {
  const double per = shape == 0 ? 16.0 * 16 * 32 * 2 : 32.0 * 32 * 16 * 2;
  return (double)blocks * 4 * iters * kChains * per;
}

// Enqueues the loop of `shape` (0: 16x16x32, 1: 32x32x16) on `stream`:
// `blocks` workgroups of 256 threads. sink: device buffer of blocks * 256
// floats (never written for iters >= 0). Returns 0, or a HIP error code.
int32_t kda_peak_mfma_launch(int32_t shape, float* sink, int32_t blocks, int32_t iters,
                             hipStream_t stream) {
  if (blocks <= 0 || iters < 0 || !sink || (shape != 0 && shape != 1)) return (int32_t)hipErrorInvalidValue;
  if (shape == 0)
    hipLaunchKernelGGL(mfma_loop<0>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters);
  else
    hipLaunchKernelGGL(mfma_loop<1>, dim3((unsigned)blocks), dim3(256), 0, stream, sink, iters);
  return (int32_t)hipGetLastError();
}

}  // extern "C"
