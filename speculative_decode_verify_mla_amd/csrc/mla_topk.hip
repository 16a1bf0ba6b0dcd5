// Top-k index selection for the sparse path on gfx950 ("The SMEM Ceiling",
// section "The Problem Space: Sparse Decode on Blackwell": each decode token
// attends to the top-k set an index-selection step picks; the scores are
// inputs here).
//
// Positions rank by score (IEEE-754 total order of float32, NaN lowest), ties
// by lower position, which makes the selected set unique; the result is
// written in ascending position order, -1 padded to k.
//
// One workgroup of 1024 threads per row:
//  * Radix select of the k-th key over an order-preserving 32-bit map of the
//    scores, in three passes of 12, 12 and 8 bits: each pass histograms the
//    keys that still match the fixed high digits (LDS atomics), then a block
//    prefix over the bins finds the digit where the count of larger keys
//    reaches k. Keys above the final threshold are all selected; of the keys
//    equal to it, the lowest positions fill the remaining slots.
//  * One more pass walks the positions in order, 4,096 at a time, and places
//    each selected position by a block prefix count, so the output comes out
//    sorted without a sort.
// Scores are read 16 bytes per lane with 16 per thread in flight; a row is
// read four times, after the first pass from L2.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mlav {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kMaxBins = 4096;  // 12-bit digits

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;  // NaN ranks below every number
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Block-wide exclusive prefix of one count per thread; `total` gets the sum.
// Every thread of the block must call it (it synchronises twice).
__device__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int below = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int t = wave_tot[w];
    below += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();  // wave_tot is reused by the next scan
  total = tot;
  return below + x - v;
}

// Four consecutive scores p .. p+3 (p a multiple of 4; rows are 16-byte aligned).
__device__ __forceinline__ float4 load4(const float* s, int p) {
  return *reinterpret_cast<const float4*>(s + p);
}

__global__ void __launch_bounds__(kTopkThreads) mla_topk_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kMaxBins];
  __shared__ int wave_tot[kTopkWaves];
  __shared__ uint32_t sel_digit;
  __shared__ int sel_above;
  const int row = blockIdx.x, tid = threadIdx.x;
  int n = a.row_lens != nullptr ? a.row_lens[row] : a.row_len;
  n = n < 0 ? 0 : (n > a.row_len ? a.row_len : n);
  const int k = a.k;
  const int kk = min(k, n);
  const float* s = a.scores + (int64_t)row * a.row_stride;
  int32_t* out = a.indices + (int64_t)row * k;
  constexpr int kSpan = 4 * kTopkThreads;  // scores per block-wide step (4 per thread)

  uint32_t prefix = 0u, pmask = 0u;
  int k_rem = kk;  // keys still to take at or below the current prefix
  if (kk > 0) {
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
      const int nb = pass == 2 ? 256 : kMaxBins;
      for (int i = tid; i < nb; i += kTopkThreads) hist[i] = 0u;
      __syncthreads();
      // 4 steps of 4 scores per thread in flight before their histogram updates
      for (int base = 0; base < n; base += 4 * kSpan) {
        float4 v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = base + j * kSpan + 4 * tid;
          v[j] = p < n ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int p = base + j * kSpan + 4 * tid;
          const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t u = order_key(e[q]);
            if (p + q < n && (u & pmask) == prefix)
              atomicAdd(&hist[(u >> shift) & (uint32_t)(nb - 1)], 1u);
          }
        }
      }
      __syncthreads();
      // Thread t owns bins 4t .. 4t+3; keys in higher bins = total - inclusive prefix.
      const int b0 = 4 * tid;
      int c[4], own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = b0 + j < nb ? (int)hist[b0 + j] : 0;
        own += c[j];
      }
      int total;
      const int excl = block_excl_scan(own, wave_tot, total);
      int above = total - excl - own;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < k_rem && k_rem <= above + c[j]) {  // exactly one bin of the block
          sel_digit = (uint32_t)(b0 + j);
          sel_above = above;
        }
        above += c[j];
      }
      __syncthreads();
      prefix |= sel_digit << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      k_rem -= sel_above;
      __syncthreads();  // hist and sel_* are rewritten by the next pass
    }
  }

  // Every key above the threshold `prefix`, and the first k_rem keys equal to
  // it, in position order. One block scan per 4,096 scores carries both counts
  // (keys above in the low 16 bits, keys equal in the high 16 bits).
  int out_base = 0, eq_seen = 0;
  for (int base = 0; kk > 0 && base < n; base += kSpan) {
    const int p = base + 4 * tid;
    const float4 v = p < n ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
    const float e[4] = {v.x, v.y, v.z, v.w};
    bool gt[4], eq[4];
    int ngt = 0, neq = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t u = order_key(e[q]);
      gt[q] = p + q < n && u > prefix;
      eq[q] = p + q < n && u == prefix;
      ngt += gt[q];
      neq += eq[q];
    }
    int tot;
    const int ex = block_excl_scan(ngt | (neq << 16), wave_tot, tot);
    int gt_before = ex & 0xffff, eq_before = ex >> 16;
    const int eq_left = max(k_rem - eq_seen, 0);  // equal keys this step may still take
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool take = gt[q] || (eq[q] && eq_before < eq_left);
      const int pos = out_base + gt_before + min(eq_before, eq_left);
      if (take && pos < kk) out[pos] = p + q;  // (the counts give exactly kk)
      gt_before += gt[q];
      eq_before += eq[q];
    }
    out_base += (tot & 0xffff) + min(tot >> 16, eq_left);
    eq_seen += tot >> 16;
  }
  for (int i = kk + tid; i < k; i += kTopkThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_kernel(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_topk_kernel, dim3(a.rows), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
