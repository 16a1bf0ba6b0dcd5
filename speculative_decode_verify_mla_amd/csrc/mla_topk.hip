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
// (mla_topk_hist_kernel, mla_topk_compact_kernel, mla_topk_place_kernel; see
// the section further down).
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

// Inclusive prefix sum over the 64 lanes of a wave: row shifts within each
// 16-lane row, then the row broadcasts (lane 15 into rows 1 and 3, lane 31
// into rows 2 and 3). Lane-to-lane data paths, no LDS round trips.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Block-wide exclusive prefix of one count per thread; `total` gets the sum.
// Every thread of the block must call it (it synchronises twice).
__device__ int block_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
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
      const int incl = wave_incl_scan(packed);
      const int step_tot = __builtin_amdgcn_readlane(incl, 63);
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
// per (row, piece) for the two passes over the scores, in three launches:
//  1. mla_topk_hist_kernel: each piece histograms the top 8 bits (digit 0) of
//     its keys and stores the 256 counts.
//  2. mla_topk_compact_kernel: every workgroup of a row sums the pieces'
//     histograms and finds the digit-0 bin d0 where the count of larger keys
//     reaches k (all reach the same answer). Keys above d0 are all selected;
//     keys in bin d0 are candidates. Each wave walks its segment of the piece
//     and writes both kinds (position, key), in position order, to a region of
//     its own: the row's entries, usually a few percent of it.
//  3. mla_topk_place_kernel: one 1024-thread workgroup per row gathers the
//     row's entries into LDS and settles the remaining 24 bits (two 12-bit
//     digits) over the candidates among them, which gives the threshold key T and how many
//     keys equal to T are taken (the lowest positions). Entries above T are
//     all taken; a block prefix over the entries, in position order, gives
//     every taken entry its output slot. The scores are read twice in all.
// The workspace holds the histograms, the entry counts and the entry regions
// (room for every key of a row: a row whose keys share their top 8 bits is
// correct, only slower). Every call rewrites what it reads.
// ---------------------------------------------------------------------------
constexpr int kMwThreads = 256;
constexpr int kMwWaves = kMwThreads / 64;
constexpr int kMwRegions = 4 * kTopkMaxChunks;  // (piece, wave) candidate regions per row, at most
static_assert(kMwRegions <= kMwThreads, "one region count per thread");
constexpr int kEntLds = 16384;  // entries of a row staged in LDS by the placement (more: read from L2)

struct MwLayout {
  uint32_t* hist;   // [rows][chunks][256] digit-0 counts
  int* ccount;      // [rows][chunks][4] entries per (piece, wave) segment
  int4* settle;     // [rows][chunks] digit-0 bin d0 and the count above it (x, y)
  uint2* cand;      // [rows][chunks][4][chunk / 4] entries (position, key)
};
__device__ __forceinline__ MwLayout mw_layout(const TopkArgs& a) {
  uint8_t* p = reinterpret_cast<uint8_t*>(a.ws);
  const int64_t rp = (int64_t)a.rows * a.chunks;
  MwLayout l;
  l.hist = reinterpret_cast<uint32_t*>(p);
  p += rp * 256 * 4;
  l.ccount = reinterpret_cast<int*>(p);
  p += rp * 4 * 4;
  l.settle = reinterpret_cast<int4*>(p);
  p += rp * 16;
  l.cand = reinterpret_cast<uint2*>(p);
  return l;
}

// Block-wide exclusive prefix over the 256 threads (one count each).
__device__ int mw_excl_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
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

// Thread t holds the count c of bin t of a 256-bin histogram of the keys that
// match the digits fixed so far. Returns the bin where the count of keys in
// higher bins first reaches k_rem (>= 1, and at most the total); `above` gets
// that count. Every thread of the block must call it.
__device__ uint32_t mw_pick(int c, int k_rem, int* wave_tot, uint32_t* s_digit, int* s_above,
                            int& above) {
  int total;
  const int excl = mw_excl_scan(c, wave_tot, total);
  const int hi = total - excl - c;  // keys in bins above this thread's
  if (hi < k_rem && k_rem <= hi + c) {  // exactly one bin of the block
    *s_digit = (uint32_t)threadIdx.x;
    *s_above = hi;
  }
  __syncthreads();
  const uint32_t d = *s_digit;
  above = *s_above;
  __syncthreads();
  return d;
}

// The digit-0 bin of a row from its pieces' histograms (all loads in flight).
__device__ uint32_t mw_settle0(const TopkArgs& a, const MwLayout& l, int row, int kk, int* wave_tot,
                               uint32_t* s_digit, int* s_above, int& above) {
  const int tid = threadIdx.x;
  uint32_t v[kTopkMaxChunks];  // unconditional loads (clamped), masked in the sum
#pragma unroll
  for (int i = 0; i < kTopkMaxChunks; ++i)
    v[i] = l.hist[((int64_t)row * a.chunks + min(i, a.chunks - 1)) * 256 + tid];
  int c = 0;
#pragma unroll
  for (int i = 0; i < kTopkMaxChunks; ++i) c += i < a.chunks ? (int)v[i] : 0;
  return mw_pick(c, kk, wave_tot, s_digit, s_above, above);
}

__device__ __forceinline__ int mw_row_len(const TopkArgs& a, int row) {
  int n = a.row_lens != nullptr ? a.row_lens[row] : a.row_len;
  return n < 0 ? 0 : (n > a.row_len ? a.row_len : n);
}

// Histogram copies in LDS for digit 0: lanes add to copy lane % 16 (at most 4
// lanes of a wave instruction per address when keys share a bin, as the top
// digits of real scores do), 257-word stride so one bin's copies sit in 16
// different banks.
constexpr int kHistCopies = 16;
constexpr int kHistStride = 257;

__global__ void __launch_bounds__(kMwThreads) mla_topk_hist_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kHistCopies * kHistStride];
  const int row = blockIdx.x / a.chunks, piece = blockIdx.x - row * a.chunks;
  const int tid = threadIdx.x;
  const int n = mw_row_len(a, row);
  for (int i = tid; i < kHistCopies * kHistStride; i += kMwThreads) hist[i] = 0u;
  __syncthreads();
  uint32_t* const my_hist = hist + (tid & (kHistCopies - 1)) * kHistStride;
  const int p0 = piece * a.chunk, p1 = min(p0 + a.chunk, n);
  const float* s = a.scores + (int64_t)row * a.row_stride;
  constexpr int kSpan = 4 * kMwThreads;
  constexpr int kBatch = 8;  // 8 x 16 bytes per thread in flight
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
      for (int q = 0; q < 4; ++q)
        if (p + q < p1) atomicAdd(&my_hist[order_key(e[q]) >> 24], 1u);
    }
  }
  __syncthreads();
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < kHistCopies; ++i) c += hist[i * kHistStride + tid];
  const MwLayout l = mw_layout(a);
  l.hist[((int64_t)row * a.chunks + piece) * 256 + tid] = c;
}

__global__ void __launch_bounds__(kMwThreads) mla_topk_compact_kernel(TopkArgs a) {
  __shared__ int wave_tot[kMwWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;
  const int row = blockIdx.x / a.chunks, piece = blockIdx.x - row * a.chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = mw_row_len(a, row);
  const int kk = min(a.k, n);
  const MwLayout l = mw_layout(a);
  const int64_t rp = (int64_t)row * a.chunks + piece;
  const int seg = a.chunk / kMwWaves;  // whole 256-score steps (chunk is a multiple of 1024)
  uint2* const region = l.cand + (rp * kMwWaves + wave) * seg;
  if (kk == 0) {  // nothing selected: empty entry regions
    if (lane == 0) l.ccount[rp * kMwWaves + wave] = 0;
    return;
  }
  // this wave's segment: write every key at or above bin d0 (above it: all
  // selected; in it: candidates) as (position, key), in position order. The
  // first batch of scores is loaded before d0 is settled, so its round trip
  // overlaps the one of the pieces' histograms.
  const float* s = a.scores + (int64_t)row * a.row_stride;
  const int p1 = min(piece * a.chunk + a.chunk, n);
  const int w0 = piece * a.chunk + wave * seg, w1 = min(w0 + seg, p1);
  float4 vb[kWalkBatch];
  auto load_batch = [&](int base) {
#pragma unroll
    for (int j = 0; j < kWalkBatch; ++j) {
      const int p = base + 256 * j + 4 * lane;
      vb[j] = p < w1 ? load4(s, p) : float4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_batch(w0);
  int taken;
  const uint32_t d0 = mw_settle0(a, l, row, kk, wave_tot, &s_digit, &s_above, taken);
  if (tid == 0) l.settle[rp] = make_int4((int)d0, taken, 0, 0);

  int count = 0;
  for (int base = w0; base < w1; base += kWalkBatch * 256) {
    if (base != w0) load_batch(base);
#pragma unroll
    for (int j = 0; j < kWalkBatch; ++j) {
      const int p = base + 256 * j + 4 * lane;
      const float e[4] = {vb[j].x, vb[j].y, vb[j].z, vb[j].w};
      uint32_t u[4];
      bool c[4];
      int cn = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u[q] = order_key(e[q]);
        c[q] = p + q < w1 && (u[q] >> 24) >= d0;
        cn += c[q];
      }
      const int incl = wave_incl_scan(cn);
      int at = count + incl - cn;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (c[q]) region[at++] = make_uint2((uint32_t)(p + q), u[q]);
      }
      count += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (lane == 0) l.ccount[rp * kMwWaves + wave] = count;
}

__global__ void __launch_bounds__(kTopkThreads) mla_topk_place_kernel(TopkArgs a) {
  __shared__ uint2 ent[kEntLds];       // the row's entries (position, key), position order
  __shared__ int off[kMwRegions + 1];  // exclusive prefix of the regions' entry counts
  __shared__ int cnt[kMwRegions];
  __shared__ uint32_t hist[4 * kTopkThreads];
  __shared__ int wave_tot[kTopkWaves];
  __shared__ uint32_t s_digit;
  __shared__ int s_above;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = mw_row_len(a, row);
  const int kk = min(a.k, n);
  int32_t* out = a.indices + (int64_t)row * a.k;

  if (kk > 0) {
    const MwLayout l = mw_layout(a);
    const int regions = a.chunks * kMwWaves;
    const int seg = a.chunk / kMwWaves;
    const uint2* const rc = l.cand + (int64_t)row * regions * seg;
    // One memory round trip: the digit-0 settlement the compaction recorded
    // (piece 0's copy), the regions' entry counts (thread = region) and the
    // first 64 entry slots of every region (wave w: regions w, w + 16, ...;
    // loaded before the counts are known, slots past a count unused).
    constexpr int kSlots = kMwRegions / kTopkWaves;
    const int wave = tid >> 6, lane = tid & 63;
    uint2 v[kSlots];
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
      v[j] = rc[(int64_t)min(wave + kTopkWaves * j, regions - 1) * seg + lane];
    const int4 st0 = l.settle[(int64_t)row * a.chunks];
    const int c_ld = l.ccount[(int64_t)row * regions + min(tid, regions - 1)];
    const uint32_t d0 = (uint32_t)st0.x;
    int k_rem = kk - st0.y;  // keys still to take among the candidates (bin d0)
    int n_ent;
    const int ex = block_excl_scan(tid < regions ? c_ld : 0, wave_tot, n_ent);
    if (tid < regions) {
      off[tid] = ex;
      cnt[tid] = c_ld;
    }
    if (tid == 0) off[regions] = n_ent;
    __syncthreads();

    // Entry i of the row: region r with off[r] <= i < off[r + 1], slot i - off[r].
    auto global_entry = [&](int i) -> uint2 {
      int lo = 0, hi = regions - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= i) lo = mid; else hi = mid - 1;
      }
      return rc[(int64_t)lo * seg + (i - off[lo])];
    };
    const bool staged = n_ent <= kEntLds;
    if (staged) {  // (longer regions continue in a second loop)
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        const int r = wave + kTopkWaves * j;
        if (r < regions && lane < cnt[r]) ent[off[r] + lane] = v[j];
      }
      for (int r = wave; r < regions; r += kTopkWaves)
        for (int e = 64 + lane; e < cnt[r]; e += 64) ent[off[r] + e] = rc[(int64_t)r * seg + e];
      __syncthreads();
    }
    auto entry = [&](int i) -> uint2 { return staged ? ent[i] : global_entry(i); };

    // the low 24 bits over the candidates (entries whose top byte is d0), as
    // two 12-bit digits: thread t holds bins 4t .. 4t+3 of a 4096-bin histogram
    uint32_t prefix = d0 << 24, pmask = 0xff000000u;
    for (int shift = 12; shift >= 0; shift -= 12) {
#pragma unroll
      for (int j = 0; j < 4; ++j) hist[4 * tid + j] = 0u;
      __syncthreads();
      for (int i = tid; i < n_ent; i += kTopkThreads) {
        const uint32_t u = entry(i).y;
        if ((u & pmask) == prefix) atomicAdd(&hist[(u >> shift) & 0xfffu], 1u);
      }
      __syncthreads();
      uint32_t h4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h4[j] = hist[4 * tid + j];
      const int c4 = (int)(h4[0] + h4[1] + h4[2] + h4[3]);
      int total;
      const int excl = block_excl_scan(c4, wave_tot, total);
      int hi = total - excl - c4;  // keys in bins above this thread's four
      if (hi < k_rem && k_rem <= hi + c4) {  // exactly one thread of the block
#pragma unroll
        for (int j = 3; j >= 0; --j) {
          if (hi < k_rem && k_rem <= hi + (int)h4[j]) {
            s_digit = (uint32_t)(4 * tid + j);
            s_above = hi;
          }
          hi += (int)h4[j];
        }
      }
      __syncthreads();
      const uint32_t d = s_digit;
      const int above = s_above;
      __syncthreads();
      prefix |= d << shift;
      pmask |= 0xfffu << shift;
      k_rem -= above;
    }
    const uint32_t T = prefix;  // the threshold key
    const int k_eq = k_rem;     // keys equal to T that are taken (the lowest positions)

    // Every entry above T is taken, and the first k_eq entries equal to T: each
    // thread counts its contiguous run of entries, two block prefixes give its
    // starting output slot and equal-rank, and it places its run in order.
    const int per = (n_ent + kTopkThreads - 1) / kTopkThreads;
    const int e0 = min(tid * per, n_ent), e1 = min(e0 + per, n_ent);
    int gt = 0, eq = 0;
    for (int i = e0; i < e1; ++i) {
      const uint32_t u = entry(i).y;
      gt += u > T;
      eq += u == T;
    }
    int G, E, tg, te;
    if (staged) {  // both counts below 2^16: one prefix of the packed pair
      const int gq = block_excl_scan(gt | (eq << 16), wave_tot, tg);
      G = gq & 0xffff;
      E = gq >> 16;
    } else {
      G = block_excl_scan(gt, wave_tot, tg);
      E = block_excl_scan(eq, wave_tot, te);
    }
    for (int i = e0; i < e1; ++i) {
      const uint2 v = entry(i);
      if (v.y > T) {
        out[G + min(E, k_eq)] = (int32_t)v.x;
        ++G;
      } else if (v.y == T) {
        if (E < k_eq) out[G + E] = (int32_t)v.x;
        ++E;
      }
    }
  }
  for (int i = kk + tid; i < a.k; i += kTopkThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_kernel(const TopkArgs& a, hipStream_t stream) {
  if (a.chunks <= 1) {
    hipLaunchKernelGGL(mla_topk_kernel, dim3(a.rows), dim3(kTopkThreads), 0, stream, a);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)a.rows * (unsigned)a.chunks;
  hipLaunchKernelGGL(mla_topk_hist_kernel, dim3(grid), dim3(kMwThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_topk_compact_kernel, dim3(grid), dim3(kMwThreads), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_topk_place_kernel, dim3(a.rows), dim3(kTopkThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
