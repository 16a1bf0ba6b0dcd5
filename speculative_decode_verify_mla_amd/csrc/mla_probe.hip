// Matrix-core throughput probe for gfx950: the bf16 MFMA rate this GPU
// actually sustains under full load, the ceiling against which the split
// kernel's achieved TFLOP/s is read next to the published dense peak. It is a
// measurement aid, not a step of the attention path.
//
// Every wave (4 per workgroup, one per SIMD) runs `iters` rounds of 16
// independent v_mfma_f32_32x32x16_bf16 with accumulators in the AGPR file and
// fixed bf16 operands of N(0,1)-like magnitude (operand values change the
// chip's power draw and so its clock; zeros would overstate the rate), then
// writes one float per thread so nothing is optimised away.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mlav {
namespace {

constexpr int kProbeChains = 16;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_probe_mfma_kernel(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float t = (float)(threadIdx.x * 8 + i);
    a[i] = (__bf16)(2.0f * __sinf(0.7311f * t + 0.25f));
    b[i] = (__bf16)(2.0f * __cosf(1.3177f * t - 0.5f));
  }
  f32x16 acc[kProbeChains];
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kProbeChains; ++j) acc[j] = mfma32(a, b, acc[j]);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kProbeChains; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_mfma(float* sink, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mla_probe_mfma_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace mlav
