// Matrix-unit reference rate for the bf16 forward: a loop of the forward's
// own MFMA (v_mfma_f32_16x16x32_bf16) on register operands, with no memory
// traffic and no dependency stalls (each wave keeps 8 independent
// accumulators, so consecutive MFMAs of a wave never wait on each other).
// Timed next to the forward, it gives the rate the chip actually reaches on
// a pure matrix load at the clock it runs then, against which the forward's
// live-FLOP rate can be compared besides the nominal peak.
#include <hip/hip_runtime.h>

#include "fsattn_internal.h"

namespace fsattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int iters, float *sink) {
  // operands that depend on the lane, so nothing folds at compile time
  const float x = 1.0f + 1e-3f * (float)(threadIdx.x & 63);
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(x * (float)(i + 1) * 1e-3f);
    b[i] = (__bf16)(x * (float)(8 - i) * 1e-3f);
  }
  f4 acc[kProbeAcc];
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeAcc; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (threadIdx.x == 0) sink[blockIdx.x] = s;
}

}  // namespace

hipError_t launch_mfma_probe(int workgroups, int iters, float *sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0, st, iters, sink);
  return hipGetLastError();
}

int64_t mfma_probe_flops(int workgroups, int iters) {
  // per wave and iteration: kProbeAcc MFMAs of 16 x 16 x 32 multiply-adds
  return (int64_t)workgroups * (kProbeThreads / 64) * iters * kProbeAcc * (2LL * 16 * 16 * 32);
}

}  // namespace fsattn
