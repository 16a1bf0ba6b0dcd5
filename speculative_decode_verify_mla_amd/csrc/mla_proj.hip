// Per-head projections either side of absorbed MLA attention, on gfx950.
//
// Absorbed MLA ("The Shared Memory Ceiling", section "The Broader Context:
// Building a Custom sm_120 Verify Kernel": attention over the shared MLA
// latent) needs each head's query in latent space before the verify call and
// brings each head's latent output back to its value space after it:
//     q_lat[m, h, :]  = q_nope[m, h, :] . W_UK[h]     (128 -> 512 per head)
//     o_head[m, h, :] = out_lat[m, h, :] . W_UV[h]    (512 -> 128 per head)
// Both are y[m, h, :] = x[m, h, :] . W[h] for tokens m, with W[h] row-major
// [in_dim, out_dim] in bf16, fp32 accumulation and a bf16 (RNE) result.
//
// With a verify step's few tokens the product is bound by reading the weights
// (8.4 MB per projection at 64 heads). One workgroup owns 32 output columns of
// one head: it DMAs that weight slice (in_dim rows x 64 B) into LDS once, then
// for each 32-token tile runs in_dim/16 MFMAs 32x32x16 computing Y^T = W^T X^T:
// W^T fragments come from the row-major slice through transposing LDS reads
// (the same access as the attention kernel's V^T operand), X^T fragments are
// 16-byte loads of 8 consecutive input dims of one token. A long input dim is
// split over up to 4 waves (at least 8 MFMA steps each), each loading and
// multiplying its own rows of the slice; the partial sums meet in LDS. That
// puts 4x more weight bytes in flight per workgroup for the 512 -> 128 map,
// which otherwise has only one wave per CU.
#include <hip/hip_runtime.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mlav {

namespace {

constexpr int kProjCols = 32;  // output columns per wave (one MFMA tile)
constexpr int kXBatch = 16;    // k-steps whose token loads are issued together

// Waves sharing one workgroup's input dim: 1..4, at least 8 MFMA steps (128 dims) each.
__host__ __device__ __forceinline__ int proj_waves(int in_dim) {
  const int steps = in_dim / 16;
  return steps >= 32 ? 4 : (steps >= 16 ? 2 : 1);
}

__global__ void __launch_bounds__(256) mla_proj_kernel(ProjArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t wslice[];  // in_dim rows x 64 B, then partials
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int S = proj_waves(a.in_dim);
  // Head fastest: workgroups are dealt to the 8 XCDs round-robin, so with a
  // multiple of 8 heads every column slice of one head lands on one XCD, whose
  // L2 then serves the 128-byte weight lines that neighbouring 64-byte slices
  // share (head-major order fetched each such line from HBM twice).
  const int h = blockIdx.x % a.heads;
  const int n0 = (blockIdx.x / a.heads) * kProjCols;
  const int K = a.in_dim;
  const int ksteps = K / 16;
  // this wave's MFMA steps (16 input dims each)
  const int kb = wave * ksteps / S, ke = (wave + 1) * ksteps / S;
  float* red = reinterpret_cast<float*>(wslice + (size_t)K * 64);  // (S-1) x 64 lanes x 16

  // ---- this wave's rows of the weight slice W[h, :, n0:n0+32] -> LDS ----------
  // One DMA instruction moves 16 rows: lane l fetches row 16i + l/4, chunk l%4.
  {
    const uint16_t* wbase = a.w + (int64_t)h * K * a.out_dim + n0;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(wbase, (uint32_t)((int64_t)K * a.out_dim * 2));
    for (int i = kb; i < ke; ++i) {
      const unsigned off = (unsigned)(((16 * i + (lane >> 2)) * a.out_dim) * 2 + (lane & 3) * 16);
      buffer_to_lds(rs, wslice + i * 1024, off);
    }
  }

  // A operand (W^T, rows = output column n, k = input dim): lane l needs column
  // l%32 at input dims k0 + 8*(l/32) + 0..7. In each 16-lane group G, lane i of a
  // transposing read addresses row (k) base + i/4, columns 4*(i%4)..+3, and gets
  // column i of the group's 16 columns for the 4 rows.
  const int G = lane >> 4, i = lane & 15;
  const unsigned abase = (unsigned)((8 * (G >> 1) + (i >> 2)) * 64 + (16 * (G & 1) + 4 * (i & 3)) * 2);

  const int M = a.tokens;
  bool slice_ready = false;
  for (int m0 = 0; m0 < M; m0 += 32) {
    // B operand (X^T, k = input dim, column = token m): lane l reads token
    // m0 + l%32, input dims k0 + 8*(l/32) + 0..7 (16 bytes). Tokens past M reuse
    // the last token and are not stored.
    const int m = min(m0 + (lane & 31), M - 1);
    const uint16_t* xrow = a.x + ((int64_t)m * a.heads + h) * K + 8 * (lane >> 5);
    f32x16 acc = {};
    for (int c0 = kb; c0 < ke; c0 += kXBatch) {
      bf16x8 xb[kXBatch];
#pragma unroll
      for (int j = 0; j < kXBatch; ++j)
        if (c0 + j < ke) xb[j] = *reinterpret_cast<const bf16x8*>(xrow + 16 * (c0 + j));
      if (!slice_ready) {
        // the first token loads are in flight with the weight DMA: one wait for both
        __builtin_amdgcn_s_waitcnt(0);
        slice_ready = true;
      }
#pragma unroll
      for (int j = 0; j < kXBatch; ++j) {
        if (c0 + j < ke) {
          const int k0 = 16 * (c0 + j);
          const bf16x4 w0 = lds_read_tr(wslice, abase + (unsigned)(k0 * 64));
          const bf16x4 w1 = lds_read_tr(wslice, abase + (unsigned)((k0 + 4) * 64));
          const bf16x8 wa = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]};
          acc = mfma32(wa, xb[j], acc);
        }
      }
    }
    if (S > 1) {
      // waves 1..S-1 hand their partial sums to wave 0 (same register layout)
      if (wave > 0) {
        float* dst = red + ((wave - 1) * 64 + lane) * 16;
#pragma unroll
        for (int r = 0; r < 16; r += 4)
          *reinterpret_cast<f32x4*>(dst + r) = f32x4{acc[r], acc[r + 1], acc[r + 2], acc[r + 3]};
      }
      __syncthreads();
      if (wave == 0) {
        for (int w = 1; w < S; ++w) {
          const float* src = red + ((w - 1) * 64 + lane) * 16;
#pragma unroll
          for (int r = 0; r < 16; r += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(src + r);
            acc[r] += v[0];
            acc[r + 1] += v[1];
            acc[r + 2] += v[2];
            acc[r + 3] += v[3];
          }
        }
      }
    }
    // C layout: lane l holds token m0 + l%32 and output columns
    // 8*(r/4) + 4*(l/32) + r%4, r = 0..15: four runs of 4 consecutive columns.
    if (wave == 0 && m0 + (lane & 31) < M) {
      uint16_t* yrow = a.y + ((int64_t)(m0 + (lane & 31)) * a.heads + h) * a.out_dim + n0 + 4 * (lane >> 5);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk;
        pk.x = pack_bf16x2(acc[4 * g + 0], acc[4 * g + 1]);
        pk.y = pack_bf16x2(acc[4 * g + 2], acc[4 * g + 3]);
        *reinterpret_cast<uint2*>(yrow + 8 * g) = pk;
      }
    }
    if (S > 1) __syncthreads();  // the partial area is reused by the next token tile
  }
}

}  // namespace

hipError_t launch_proj_kernel(const ProjArgs& a, hipStream_t stream) {
  const unsigned grid = (unsigned)a.heads * (unsigned)(a.out_dim / kProjCols);
  const int waves = proj_waves(a.in_dim);
  const size_t lds = (size_t)a.in_dim * kProjCols * 2 + (size_t)(waves - 1) * 64 * 16 * 4;
  hipLaunchKernelGGL(mla_proj_kernel, dim3(grid), dim3(64 * waves), lds, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
