// Matrix-core throughput probe for gfx950: the bf16 MFMA rate this GPU
// actually sustains under full load, the ceiling against which the split
// kernel's achieved TFLOP/s is read next to the published dense peak. It is a
// measurement aid, not a step of the attention path.
//
// Every wave (4 per workgroup, one per SIMD) runs `iters` rounds of 16
// independent v_mfma_f32_32x32x16_bf16 with accumulators in the AGPR file and
// fixed bf16 operands of N(0,1)-like magnitude (operand values change the
// chip's power draw and so its clock; zeros would overstate the rate), then
// writes one float per thread so nothing is optimised away. Threads 0 and 1 of
// each workgroup instead write the workgroup's elapsed shader-clock cycles
// (s_memtime) and constant-rate real-time ticks (s_memrealtime, 100 MHz) over
// its MFMA loop: their ratio is the clock the chip ran at.
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
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
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
  // the sums depend on every MFMA, so the stamps below follow the whole loop
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) s = (float)(c1 - c0) + 0.f * s;
  if (threadIdx.x == 1) s = (float)(r1 - r0) + 0.f * s;
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe_mfma(float* sink, int blocks, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mla_probe_mfma_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters);
  return hipGetLastError();
}

}  // namespace mlav

// Row-gather probe: the rate at which this GPU gathers cache rows (a 1,024-byte
// latent row plus its 128-byte rope row) by index, with no compute, the ceiling
// against which the sparse path's gathered bytes can be read. One workgroup of
// 4 waves per (group, 64 indices); each wave issues the loads of its 16 rows
// before using any (one 16-byte load per lane per latent row, lanes 0..7 for the
// rope row) and folds them into one word per thread.
namespace mlav {
namespace {

__global__ void __launch_bounds__(256) mla_probe_gather_kernel(GatherProbeArgs a) {
  const int chunks = (a.per_group + 63) / 64;
  const int g = blockIdx.x / chunks, c = blockIdx.x - g * chunks;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t base = (int64_t)(g / a.tokens_per_seq) * a.kv_seq_stride;
  // rows this group's indices may select: its sequence's (all from `base` when
  // kv_seq_stride is 0), within the cache
  const int64_t left = base < a.kv_rows ? a.kv_rows - base : 0;
  const int seq_rows = (int)(a.kv_seq_stride > 0 && a.kv_seq_stride < left ? a.kv_seq_stride : left);
  // lane k holds index k of this chunk (-1: skipped); buffer range checks return
  // zeros for skipped rows, so every load is issued unconditionally
  const int k = c * 64 + lane;
  const int idx = k < a.per_group ? a.indices[(int64_t)g * a.per_group + k] : -1;
  const int row = idx >= 0 && idx < seq_rows ? idx : -1;
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.c_kv + base * 512, (uint32_t)seq_rows * 1024u);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(a.k_rope + base * 64, (uint32_t)seq_rows * 128u);
  u32x4 lat[16], rope[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = __builtin_amdgcn_readlane(row, wave * 16 + i);
    const unsigned ol = r >= 0 ? (unsigned)r * 1024u + (unsigned)lane * 16u : 0x80000000u;
    const unsigned orp = r >= 0 && lane < 8 ? (unsigned)r * 128u + (unsigned)lane * 16u : 0x80000000u;
    lat[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rl, ol, 0, 0));
    rope[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, orp, 0, 0));
  }
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) x ^= lat[i][0] ^ lat[i][1] ^ lat[i][2] ^ lat[i][3] ^ rope[i][0] ^ rope[i][3];
  a.sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = __uint_as_float(x);
}

}  // namespace

hipError_t launch_probe_gather(const GatherProbeArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.groups * (unsigned)((a.per_group + 63) / 64);
  hipLaunchKernelGGL(mla_probe_gather_kernel, dim3(grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
