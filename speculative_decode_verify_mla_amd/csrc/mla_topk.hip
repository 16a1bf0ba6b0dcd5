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
//  * The selected positions are then placed in position order: each wave
//    counts the keys above / equal to the threshold in its contiguous segment,
//    the segments' totals give each its starting offsets, and each wave walks
//    its segment again placing elements by wave-local prefix sums, so the
//    output comes out sorted without a sort.
// Scores are read 16 bytes per lane with 16 per thread in flight; a row is
// read four times, after the first pass from L2.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mlav {

namespace {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kMaxBins = 4096;  // 12-bit digits
constexpr int kWalkBatch = 8;   // 256-score wave steps whose loads are issued together

__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;  // NaN ranks below every number
  const uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
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
  // it, in position order. An element x goes to slot G(x) + min(E(x), k_rem),
  // G and E counting the keys above and equal to the threshold before x. Each
  // wave owns one contiguous segment of the row: it counts its segment, the
  // 16 wave totals give every segment's starting G and E, and the wave walks
  // its segment again placing elements with wave-local prefix sums (no block
  // barrier inside either walk).
  if (kk > 0) {
    const int lane = tid & 63, wave = tid >> 6;
    const int seg = (n + kTopkWaves * 256 - 1) / (kTopkWaves * 256) * 256;  // whole 256-score steps
    const int w0 = wave * seg, w1 = min(w0 + seg, n);
    int ngt = 0, neq = 0;
    for (int base = w0; base < w1; base += kWalkBatch * 256) {
      float4 v[kWalkBatch];  // the batch's loads are all in flight before any is used
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
        const int p = base + 256 * j + 4 * lane;
        v[j] = p < w1 ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
        const int p = base + 256 * j + 4 * lane;
        const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = order_key(e[q]);
          ngt += (p + q < w1 && u > prefix);
          neq += (p + q < w1 && u == prefix);
        }
      }
    }
    const int wgt = wave_sum_i(ngt), weq = wave_sum_i(neq);
    __shared__ int seg_gt[kTopkWaves], seg_eq[kTopkWaves];
    if (lane == 0) {
      seg_gt[wave] = wgt;
      seg_eq[wave] = weq;
    }
    __syncthreads();
    int G = 0, E = 0;  // keys above / equal before this wave's segment
    for (int w = 0; w < wave; ++w) {
      G += seg_gt[w];
      E += seg_eq[w];
    }
    for (int base = w0; base < w1; base += kWalkBatch * 256) {
      float4 vb[kWalkBatch];
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
        const int pj = base + 256 * j + 4 * lane;
        vb[j] = pj < w1 ? load4(s, pj) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
      const int p = base + 256 * j + 4 * lane;
      const float4 v = vb[j];
      const float e[4] = {v.x, v.y, v.z, v.w};
      bool gt[4], eq[4];
      int cg = 0, ce = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t u = order_key(e[q]);
        gt[q] = p + q < w1 && u > prefix;
        eq[q] = p + q < w1 && u == prefix;
        cg += gt[q];
        ce += eq[q];
      }
      // wave-exclusive prefix of (cg, ce), packed as cg | ce << 16
      const int packed = cg | (ce << 16);
      int incl = packed;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const int step_tot = __shfl(incl, 63);
      int g = G + ((incl - packed) & 0xffff), eqb = E + ((incl - packed) >> 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool take = gt[q] || (eq[q] && eqb < k_rem);
        const int pos = g + min(eqb, k_rem);
        if (take && pos < kk) out[pos] = p + q;  // (the counts give exactly kk)
        g += gt[q];
        eqb += eq[q];
      }
      G += step_tot & 0xffff;
      E += step_tot >> 16;
      }
    }
  }
  for (int i = kk + tid; i < k; i += kTopkThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_kernel(const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(mla_topk_kernel, dim3(a.rows), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
