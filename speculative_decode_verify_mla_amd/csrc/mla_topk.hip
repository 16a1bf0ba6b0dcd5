// Top-k index selection for the sparse path on gfx950 ("The SMEM Ceiling",
// section "The Problem Space: Sparse Decode on Blackwell": each decode token
// attends to the top-k set an index-selection step picks; the scores are
// inputs here).
//
// Positions rank by score (IEEE-754 total order of float32, NaN lowest), ties
// by lower position, which makes the selected set unique; the result is
// written in ascending position order, -1 padded to k.
//
// Two paths with identical results. Called without a workspace, one workgroup
// of 1024 threads per row (mla_topk_kernel, below). With one, a batch of rows
// too short to fill the GPU is spread over several workgroups per row
// (mla_topk_level_kernel x 4, mla_topk_place_kernel; see the section further
// down).
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

// ---------------------------------------------------------------------------
// Several workgroups per row. With few rows, one workgroup per row leaves most
// CUs idle, so each row is cut into `chunks` pieces, one 256-thread workgroup
// per (row, piece), and the radix select runs over 8-bit digits in four
// launches, most significant digit first. Launch L:
//  * every workgroup of a row first settles digit L-1: it sums the pieces'
//    level L-1 histograms (256 bins x pieces) and finds the bin where the count
//    of larger keys reaches the number still to take (all workgroups of the
//    row reach the same answer; piece 0 records the new state for launch L+1)
//    and records its own count of keys in the bins above the settled digit;
//  * then it histograms digit L of its piece's keys that match the digits
//    fixed so far and stores the 256 counts (no atomics outside LDS, no
//    clearing: every piece writes all of its bins).
// A fifth launch settles the last digit, which gives the threshold key T and
// how many keys equal to T are taken. A piece's count of keys above T is the
// sum over levels of its keys above that level's digit, and its count of keys
// equal to T is its last-level bin of T, so the pieces before it give each
// piece its output offsets. The piece then places its selected positions in
// position order as the one-workgroup kernel does.
// ---------------------------------------------------------------------------
constexpr int kMwThreads = 256;
constexpr int kMwWaves = kMwThreads / 64;

struct MwState {
  uint32_t prefix, pmask;  // digits fixed so far, and their bits
  int32_t k_rem, pad;      // keys still to take among those matching prefix
};

__device__ __forceinline__ uint32_t* mw_hist(const TopkArgs& a, int level, int row, int piece) {
  return reinterpret_cast<uint32_t*>(a.ws) +
         (((int64_t)level * a.rows + row) * a.chunks + piece) * 256;
}
__device__ __forceinline__ MwState* mw_state(const TopkArgs& a, int row, int level) {
  uint8_t* base = reinterpret_cast<uint8_t*>(a.ws) + (int64_t)kTopkLevels * a.rows * a.chunks * 256 * 4;
  return reinterpret_cast<MwState*>(base) + (int64_t)row * kTopkLevels + level;
}
// Keys of a piece whose digit `level` (< kTopkLevels - 1) is above the settled
// one (they match the digits above it): written by launch level + 1.
__device__ __forceinline__ int* mw_above(const TopkArgs& a, int level, int row, int piece) {
  uint8_t* base = reinterpret_cast<uint8_t*>(a.ws) + (int64_t)kTopkLevels * a.rows * a.chunks * 256 * 4 +
                  (int64_t)a.rows * kTopkLevels * 16;
  return reinterpret_cast<int*>(base) + ((int64_t)level * a.rows + row) * a.chunks + piece;
}

// Block-wide exclusive prefix over the 256 threads (one count each).
__device__ int mw_excl_scan(int v, int* wave_tot, int& total) {
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
  for (int w = 0; w < kMwWaves; ++w) {
    const int t = wave_tot[w];
    below += w < wave ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return below + x - v;
}

// Settles digit `level` of a row from the pieces' level histograms: returns
// the digit; `taken_above` gets the count of matching keys in higher bins.
// Every thread of the block must call it; requires k_rem >= 1.
__device__ uint32_t mw_settle(const TopkArgs& a, int row, int level, int k_rem, int* wave_tot,
                              uint32_t* s_digit, int* s_above, int& taken_above) {
  const int tid = threadIdx.x;
  uint32_t v[kTopkMaxChunks];  // every piece's count of this bin, all loads in flight
#pragma unroll
  for (int i = 0; i < kTopkMaxChunks; ++i) v[i] = i < a.chunks ? mw_hist(a, level, row, i)[tid] : 0u;
  int c = 0;
#pragma unroll
  for (int i = 0; i < kTopkMaxChunks; ++i) c += (int)v[i];
  int total;
  const int excl = mw_excl_scan(c, wave_tot, total);
  const int above = total - excl - c;  // matching keys in bins above this thread's
  if (above < k_rem && k_rem <= above + c) {  // exactly one bin of the block
    *s_digit = (uint32_t)tid;
    *s_above = above;
  }
  __syncthreads();
  const uint32_t d = *s_digit;
  taken_above = *s_above;
  __syncthreads();
  return d;
}

__device__ __forceinline__ int mw_row_len(const TopkArgs& a, int row) {
  int n = a.row_lens != nullptr ? a.row_lens[row] : a.row_len;
  return n < 0 ? 0 : (n > a.row_len ? a.row_len : n);
}

// Histogram copies in LDS for the first digit: lanes add to copy lane % 16 (at
// most 4 lanes of a wave instruction per address when keys share a bin, as the
// top digits of real scores do), 257-word stride so one bin's copies sit in 16
// different banks. Later digits only count the few keys matching the digits
// fixed so far and use one copy.
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;

__global__ void __launch_bounds__(kMwThreads) mla_topk_level_kernel(TopkArgs a, int level) {
  __shared__ uint32_t hist[kHistCopies * kHistStride];
  __shared__ int wave_tot[kMwWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;
  const int row = blockIdx.x / a.chunks, piece = blockIdx.x - row * a.chunks;
  const int tid = threadIdx.x;
  const int n = mw_row_len(a, row);
  const int kk = min(a.k, n);

  MwState st{0u, 0u, kk, 0};
  if (level > 0) {
    st = *mw_state(a, row, level - 1);
    if (kk > 0) {
      const int shift = 24 - 8 * (level - 1);
      int taken;
      const uint32_t d = mw_settle(a, row, level - 1, st.k_rem, wave_tot, &s_digit, &s_above, taken);
      st.prefix |= d << shift;
      st.pmask |= 0xffu << shift;
      st.k_rem -= taken;
      // this piece's keys above the settled digit (block sum over the bins above d)
      const int mine = (uint32_t)tid > d ? (int)mw_hist(a, level - 1, row, piece)[tid] : 0;
      int piece_above;
      mw_excl_scan(mine, wave_tot, piece_above);
      if (tid == 0) *mw_above(a, level - 1, row, piece) = piece_above;
    } else if (tid == 0) {
      *mw_above(a, level - 1, row, piece) = 0;
    }
  }
  if (piece == 0 && tid == 0) *mw_state(a, row, level) = st;

  const int copies = level == 0 ? kHistCopies : 1;
  for (int i = tid; i < copies * kHistStride; i += kMwThreads) hist[i] = 0u;
  __syncthreads();
  const int shift = 24 - 8 * level;
  uint32_t* const my_hist = hist + (tid & (copies - 1)) * kHistStride;
  const int p0 = piece * a.chunk, p1 = min(p0 + a.chunk, n);
  const float* s = a.scores + (int64_t)row * a.row_stride;
  constexpr int kSpan = 4 * kMwThreads;
  constexpr int kBatch = 8;  // 8 x 16 bytes per thread in flight
  if (kk > 0) {
    for (int base = p0; base < p1; base += kBatch * kSpan) {
      float4 v[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int p = base + j * kSpan + 4 * tid;
        v[j] = p < p1 ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int p = base + j * kSpan + 4 * tid;
        const float e[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = order_key(e[q]);
          if (p + q < p1 && (u & st.pmask) == st.prefix) atomicAdd(&my_hist[(u >> shift) & 0xffu], 1u);
        }
      }
    }
  }
  __syncthreads();
  uint32_t c = 0u;
  for (int i = 0; i < copies; ++i) c += hist[i * kHistStride + tid];
  mw_hist(a, level, row, piece)[tid] = c;
}

__global__ void __launch_bounds__(kMwThreads) mla_topk_place_kernel(TopkArgs a) {
  __shared__ int wave_tot[kMwWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;
  __shared__ int seg_gt[kMwWaves], seg_eq[kMwWaves];
  const int row = blockIdx.x / a.chunks, piece = blockIdx.x - row * a.chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = mw_row_len(a, row);
  const int kk = min(a.k, n);
  int32_t* out = a.indices + (int64_t)row * a.k;

  if (kk > 0) {
    MwState st = *mw_state(a, row, kTopkLevels - 1);
    int taken;
    const uint32_t d = mw_settle(a, row, kTopkLevels - 1, st.k_rem, wave_tot, &s_digit, &s_above, taken);
    const uint32_t T = st.prefix | d;  // the threshold key
    const int k_eq = st.k_rem - taken;  // keys equal to T that are taken

    // keys above / equal to T in the pieces before this one
    // Earlier levels: the recorded per-piece counts (thread i < pieces, level
    // i / pieces); last level: bin counts of the pieces before this one.
    int g_part = 0, e_part = 0;
    for (int t = tid; t < (kTopkLevels - 1) * a.chunks; t += kMwThreads) {
      const int lv = t / a.chunks, i = t - lv * a.chunks;
      if (i < piece) g_part += *mw_above(a, lv, row, i);
    }
    {
      const bool above = (uint32_t)tid > d, at = (uint32_t)tid == d;
      uint32_t v[kTopkMaxChunks];  // pieces before this one, all loads in flight
#pragma unroll
      for (int i = 0; i < kTopkMaxChunks; ++i)
        v[i] = (i < piece && (above || at)) ? mw_hist(a, kTopkLevels - 1, row, i)[tid] : 0u;
#pragma unroll
      for (int i = 0; i < kTopkMaxChunks; ++i) {
        g_part += above ? (int)v[i] : 0;
        e_part += at ? (int)v[i] : 0;
      }
    }
    int G0, E0;
    mw_excl_scan(g_part, wave_tot, G0);
    mw_excl_scan(e_part, wave_tot, E0);

    // Each wave owns one contiguous segment of the piece (whole 256-score steps):
    // count, exchange the wave totals, then walk again placing positions.
    const float* s = a.scores + (int64_t)row * a.row_stride;
    const int p0 = piece * a.chunk, p1 = min(p0 + a.chunk, n);
    const int len = max(p1 - p0, 0);
    const int seg = (len + kMwWaves * 256 - 1) / (kMwWaves * 256) * 256;
    const int w0 = p0 + wave * seg, w1 = min(w0 + seg, p1);
    int ngt = 0, neq = 0;
    for (int base = w0; base < w1; base += kWalkBatch * 256) {
      float4 v[kWalkBatch];
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
          ngt += (p + q < w1 && u > T);
          neq += (p + q < w1 && u == T);
        }
      }
    }
    const int wgt = wave_sum_i(ngt), weq = wave_sum_i(neq);
    if (lane == 0) {
      seg_gt[wave] = wgt;
      seg_eq[wave] = weq;
    }
    __syncthreads();
    int G = G0, E = E0;
    for (int w = 0; w < wave; ++w) {
      G += seg_gt[w];
      E += seg_eq[w];
    }
    for (int base = w0; base < w1; base += kWalkBatch * 256) {
      float4 vb[kWalkBatch];
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
        const int p = base + 256 * j + 4 * lane;
        vb[j] = p < w1 ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int j = 0; j < kWalkBatch; ++j) {
        const int p = base + 256 * j + 4 * lane;
        const float e[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
        bool gt[4], eq[4];
        int cg = 0, ce = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t u = order_key(e[q]);
          gt[q] = p + q < w1 && u > T;
          eq[q] = p + q < w1 && u == T;
          cg += gt[q];
          ce += eq[q];
        }
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
          const bool take = gt[q] || (eq[q] && eqb < k_eq);
          const int pos = g + min(eqb, k_eq);
          if (take && pos < kk) out[pos] = p + q;
          g += gt[q];
          eqb += eq[q];
        }
        G += step_tot & 0xffff;
        E += step_tot >> 16;
      }
    }
  }
  if (piece == 0)
    for (int i = kk + tid; i < a.k; i += kMwThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_kernel(const TopkArgs& a, hipStream_t stream) {
  if (a.chunks <= 1) {
    hipLaunchKernelGGL(mla_topk_kernel, dim3(a.rows), dim3(kTopkThreads), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)a.rows * (unsigned)a.chunks;
  for (int level = 0; level < kTopkLevels; ++level) {
    hipLaunchKernelGGL(mla_topk_level_kernel, dim3(grid), dim3(kMwThreads), 0, stream, a, level);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mla_topk_place_kernel, dim3(grid), dim3(kMwThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
