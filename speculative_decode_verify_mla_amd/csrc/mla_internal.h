// Internal types shared by the host dispatcher and the kernels of libmla_verify.
// Not part of the public ABI (that is include/mla_verify.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlav {

constexpr int kDL = 512;             // latent width (values and the first score term)
constexpr int kDR = 64;              // rotary width (second score term only)
constexpr int kTile = 64;            // keys per LDS tile
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kRowsPerWave = 32;     // query rows owned by one wave (one per lane pair)
constexpr int kRowsPerBlock = kWaves * kRowsPerWave;  // 128
constexpr int kThreads = kWaves * 64;

// Workspace record: one wave's 32 rows x 512 partial output (fp16, normalised by its
// split's own sum of rounded terms, times a per-row power-of-two scale), plus three
// fp32 values per row: the split's log2-sum-exp from fp32 terms, the same from the
// rounded terms, and the row's fp16 scale.
constexpr int kRecElems = kRowsPerWave * kDL;  // 16384
constexpr int kRecRowStats = 3;
constexpr int kMaxSplits = 256;  // per query group (combine weights live in LDS)
// Fewest 64-key tiles per split when the library picks the split count: the
// per-split partial (1 KiB per row, written and read back) and the split's fixed
// start-up stay small next to its KV reads and matrix work.
constexpr int kMinChunkDense = 2;
constexpr int kMinChunkSparse = 4;
constexpr size_t kRecBytes = (size_t)kRecElems * 2 + (size_t)kRecRowStats * kRowsPerWave * 4;
// Groups of more than this many splits, whose split count the host knows
// (sparse calls, single sequences), combine in the wide kernel: one workgroup
// per 32 rows x 8 dims with every split's loads in flight at once.
constexpr int kOneStageMaxSplits = 32;

enum Mode : int { kContig = 0, kPaged = 1, kSparse = 2, kSparsePaged = 3 };

struct MainArgs {
  const uint16_t* q_lat;
  const uint16_t* q_rope;
  const uint16_t* c_kv;
  const uint16_t* k_rope;
  const int32_t* page_table;
  const uint8_t* tree_mask;
  const int32_t* kv_lens;
  const int32_t* indices;
  uint16_t* out;
  float* lse;
  uint16_t* ws_o; // [records][16384] fp16, register-native order
  float* ws_lse;  // [records][3][32] fp32: lse2 (fp32 terms), lse2 (rounded terms), scale
  int2* ws_meta;  // dense: [groups] (first slot, splits holding keys), written by the split kernel
  int64_t kv_seq_stride;
  int64_t kv_rows;
  int32_t T, H;
  int32_t rows_per_group;
  int32_t num_groups;
  int32_t row_blocks;
  int32_t page_size;
  int32_t max_pages;
  int32_t max_kv_len;
  int32_t topk;
  int32_t num_splits;   // sparse: splits per token (uniform)
  int32_t chunk_tiles;  // sparse: tiles per split
  int32_t split_slots;  // dense: (sequence, split) slots per row block
  int32_t slot_stride;  // dense: workgroups per row block in the grid (= split_slots)
  int32_t fixed_chunk;  // dense: tiles per split when requested, 0 = chosen on the device
  int32_t final_out;    // 1: single split for every group, write out/lse directly
  int32_t wide_combine;  // != 0: groups of more than 32 splits (sparse, or one sequence): wide combine
  float scale_log2;    // scale * log2(e)
};

// Post-verify KV compaction (mla_compact.hip).
struct CompactArgs {
  uint16_t* c_kv;
  uint16_t* k_rope;
  const int32_t* page_table;
  const int32_t* kv_lens;
  const int32_t* accepted;      // [B, T] draft indices in path order
  const int32_t* num_accepted;  // [B]
  int32_t* new_kv_lens;         // [B], may alias kv_lens
  int64_t kv_seq_stride;
  int64_t kv_rows;
  int32_t T;
  int32_t page_size;
  int32_t max_pages;
  int32_t max_kv_len;
};
hipError_t launch_compact_kernel(const CompactArgs& a, int batch, hipStream_t stream);

// Per-head projections around absorbed attention (mla_proj.hip).
struct ProjArgs {
  const uint16_t* x;  // [tokens, heads, in_dim] bf16
  const uint16_t* w;  // [heads, in_dim, out_dim] bf16
  uint16_t* y;        // [tokens, heads, out_dim] bf16
  int32_t tokens, heads, in_dim, out_dim;
};
hipError_t launch_proj_kernel(const ProjArgs& a, hipStream_t stream);

// Top-k index selection (mla_topk.hip).
struct TopkArgs {
  const float* scores;      // [rows, row_stride] fp32
  const int32_t* row_lens;  // [rows] candidates per row, or NULL (all row_len)
  int32_t* indices;         // [rows, k] ascending, -1 padded
  int64_t row_stride;
  int32_t rows, row_len, k;
  // Several workgroups per row (chunks > 1): the row is cut into `chunks`
  // pieces of `chunk` scores; the workspace holds the per-piece digit
  // histograms and the per-row selection state.
  int32_t chunks, chunk;
  void* ws;
};
constexpr int kTopkMaxChunks = 32;   // pieces per row
constexpr int kTopkMinChunk = 4096;  // scores per piece, at least
// Workspace bytes of the several-workgroup path for `rows` rows cut into
// `chunks` pieces of `chunk` scores: per piece a 256-bin histogram, an entry
// count per wave segment and a 16-byte digit-0 record, and entry room for
// every score (8 bytes each).
constexpr int64_t topk_piece_bytes = 256 * 4 + 16 + 16;
constexpr int64_t topk_workspace_bytes(int64_t rows, int64_t chunks, int64_t chunk) {
  return rows * chunks * topk_piece_bytes + rows * chunks * chunk * 8;
}
hipError_t launch_topk_kernel(const TopkArgs& a, hipStream_t stream);

// Launchers (defined in mla_kernels.hip). Return the hipError_t of the launch.
hipError_t launch_split_kernel(const MainArgs& a, int mode, hipStream_t stream);
hipError_t launch_combine_kernel(const MainArgs& a, int mode, hipStream_t stream);

// Matrix-core throughput and row-gather probes (measurement aids).
hipError_t launch_probe_mfma(float* sink, int blocks, int iters, hipStream_t stream);
struct GatherProbeArgs {
  const uint16_t* c_kv;    // [kv_rows, 512] bf16
  const uint16_t* k_rope;  // [kv_rows, 64] bf16
  const int32_t* indices;  // [groups, per_group]; row = (g / tokens_per_seq) * kv_seq_stride + index
  float* sink;             // one float per thread of the launch
  int64_t kv_seq_stride, kv_rows;
  int32_t groups, per_group, tokens_per_seq;
};
hipError_t launch_probe_gather(const GatherProbeArgs& a, hipStream_t stream);

}  // namespace mlav
