// Post-verify KV compaction on gfx950: after the verifier accepts a path of
// draft tokens, their cache rows move to the front of the draft region so the
// next decoding step sees prefix + accepted tokens contiguously ("The Shared
// Memory Ceiling", section "The Broader Context: Building a Custom sm_120
// Verify Kernel", names this "defrag" step of the plan).
//
// One workgroup per sequence: it resolves the (source, destination) physical
// rows of its at most 64 moves, stages every source row (1,152 bytes: the
// 512-wide latent row and the 64-wide rope row) in LDS, and only then writes
// the destinations, so moves whose rows overlap are well defined. The work is
// a few hundred kilobytes of 16-byte copies, bound by launch latency and HBM.
#include <hip/hip_runtime.h>

#include "mla_internal.h"

namespace mlav {

namespace {

constexpr int kChunksLat = kDL * 2 / 16;  // 64 sixteen-byte chunks per latent row
constexpr int kChunksRope = kDR * 2 / 16; // 8 per rope row
constexpr int kChunksRow = kChunksLat + kChunksRope;
constexpr int kMaxMoves = 64;             // one per draft slot (T <= 64)

__device__ __forceinline__ int64_t phys_row(const CompactArgs& a, int b, int p) {
  int64_t r;
  if (a.page_table == nullptr) {
    r = (int64_t)b * a.kv_seq_stride + p;
  } else {
    const int page = a.page_table[(int64_t)b * a.max_pages + p / a.page_size];
    if (page < 0) return -1;
    r = (int64_t)page * a.page_size + p % a.page_size;
  }
  return r < a.kv_rows ? r : -1;
}

__global__ void __launch_bounds__(256) mla_compact_kernel(CompactArgs a) {
  __shared__ uint4 stage[kMaxMoves * kChunksRow];  // 73,728 B
  __shared__ int64_t src_row[kMaxMoves], dst_row[kMaxMoves];
  const int b = blockIdx.x;
  const int T = a.T;
  int kv = a.kv_lens[b];
  kv = kv < 0 ? 0 : (kv > a.max_kv_len ? a.max_kv_len : kv);
  int n = a.num_accepted[b];
  n = n < 0 ? 0 : (n > T ? T : n);
  const int P = kv - T;

  if (threadIdx.x < kMaxMoves) {
    const int i = threadIdx.x;
    int64_t rs = -1, rd = -1;
    if (i < n) {
      const int d = a.accepted[(int64_t)b * T + i];
      const int src = P + d, dst = P + i;
      if (d >= 0 && d < T && src >= 0 && src < kv && dst >= 0 && dst < kv) {
        rs = phys_row(a, b, src);
        rd = phys_row(a, b, dst);
        if (rs < 0 || rd < 0) rs = rd = -1;
      }
    }
    src_row[i] = rs;
    dst_row[i] = rd;
  }
  __syncthreads();

  const int total = n * kChunksRow;
  for (int k = threadIdx.x; k < total; k += blockDim.x) {
    const int i = k / kChunksRow, c = k - i * kChunksRow;
    const int64_t rs = src_row[i];
    if (rs >= 0) {
      stage[k] = c < kChunksLat ? reinterpret_cast<const uint4*>(a.c_kv + rs * kDL)[c]
                                : reinterpret_cast<const uint4*>(a.k_rope + rs * kDR)[c - kChunksLat];
    }
  }
  __syncthreads();  // every source row is in LDS before any destination is written
  for (int k = threadIdx.x; k < total; k += blockDim.x) {
    const int i = k / kChunksRow, c = k - i * kChunksRow;
    const int64_t rd = dst_row[i];
    if (rd >= 0) {
      if (c < kChunksLat) reinterpret_cast<uint4*>(a.c_kv + rd * kDL)[c] = stage[k];
      else reinterpret_cast<uint4*>(a.k_rope + rd * kDR)[c - kChunksLat] = stage[k];
    }
  }
  if (threadIdx.x == 0) a.new_kv_lens[b] = P + n > 0 ? P + n : 0;  // after every read of kv_lens[b]
}

}  // namespace

hipError_t launch_compact_kernel(const CompactArgs& a, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(mla_compact_kernel, dim3(batch), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mlav
