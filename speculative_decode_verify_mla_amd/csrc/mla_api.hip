// Host side of libmla_verify: argument checks, work decomposition (split
// plan), workspace sizing and kernel dispatch behind the C ABI of
// include/mla_verify.h. Every check runs before the first HIP call; no call
// allocates, frees, synchronises or reads device memory on the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <atomic>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mla_internal.h"
#include "mla_verify.h"
#include "mla_verify_probe.h"

namespace {

using mlav::kRowsPerBlock;
using mlav::kTile;
using mlav::kWaves;

constexpr int kMaxDevices = 64;
// Per-device cache: 0 = unknown, 1 = gfx950, -1 = other.
std::atomic<int> g_arch_state[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Host-side shape checks shared by both entry points. Returns MLA_OK or MLA_ERR_INVALID.
int check_dims(const mla_dims* d, bool sparse, bool paged) {
  if (d == nullptr) return MLA_ERR_INVALID;
  if (d->batch < 1 || d->num_q < 1 || d->num_q > MLA_MAX_DRAFT || d->num_heads < 1)
    return MLA_ERR_INVALID;
  if (d->num_splits < 0 || d->reserved != 0) return MLA_ERR_INVALID;
  if (d->phase < MLA_PHASE_ALL || d->phase > MLA_PHASE_COMBINE) return MLA_ERR_INVALID;
  if (d->max_kv_len < 1 || d->kv_rows < 1) return MLA_ERR_INVALID;
  if (!sparse && d->max_kv_len < d->num_q) return MLA_ERR_INVALID;
  if (sparse && d->topk < 1) return MLA_ERR_INVALID;
  // the dense split plan sums 64-key tiles over the batch in 32-bit integers
  if (!sparse && (int64_t)d->batch * ceil_div(d->max_kv_len, kTile) > 0x7fffffffLL) return MLA_ERR_INVALID;
  // row counts must fit 32-bit grid arithmetic
  const int64_t rows_total = (int64_t)d->batch * d->num_q * d->num_heads;
  if (rows_total > (int64_t)1 << 30) return MLA_ERR_INVALID;
  if (paged) {
    if (d->page_size <= 0 || d->page_size % kTile != 0) return MLA_ERR_INVALID;
    if (d->max_pages < 1) return MLA_ERR_INVALID;
    if ((int64_t)d->max_pages * d->page_size < d->max_kv_len) return MLA_ERR_INVALID;
    if (sparse && d->kv_rows > ((int64_t)1 << 21)) return MLA_ERR_INVALID;
  } else {
    if (d->kv_seq_stride < d->max_kv_len) return MLA_ERR_INVALID;
    if ((int64_t)(d->batch - 1) * d->kv_seq_stride + d->max_kv_len > d->kv_rows)
      return MLA_ERR_INVALID;
    if (sparse && d->kv_seq_stride > ((int64_t)1 << 21)) return MLA_ERR_INVALID;
  }
  return MLA_OK;
}

// Compute units the plans are made for: gfx950 (MI355X) has 256. The plans are
// pure functions of their arguments (no device query), so a workspace size
// never depends on which device happens to be current.
constexpr int kPlanCUs = 256;

// Pieces per row for top-k selection: enough (row, piece) workgroups for about
// two per CU, at most kTopkMaxChunks pieces of at least kTopkMinChunk scores,
// each a whole number of 1024-score steps (`chunk`, if non-NULL). 1 = one
// workgroup per row. Rows longer than 2^30 keep one workgroup (piece offsets
// stay far from the 32-bit limit).
int topk_pieces(int64_t rows, int64_t row_len, int cus, int* chunk) {
  if (row_len > (int64_t(1) << 30)) return 1;
  int64_t s = ceil_div(2 * (int64_t)cus, rows);
  s = std::min<int64_t>(s, mlav::kTopkMaxChunks);
  s = std::min<int64_t>(s, ceil_div(row_len, mlav::kTopkMinChunk));
  s = std::max<int64_t>(s, 1);
  const int64_t c = ceil_div(ceil_div(row_len, s), 1024) * 1024;
  if (chunk) *chunk = (int)c;
  return (int)ceil_div(row_len, c);
}

// MLA_OK on gfx950, MLA_ERR_UNSUPPORTED elsewhere, MLA_ERR_HIP if the runtime fails.
int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MLA_ERR_HIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MLA_OK : MLA_ERR_UNSUPPORTED;
}

// Groups of more than 32 splits whose split count the host knows (sparse calls:
// uniform; one dense sequence: its slots) combine in the wide kernel.
bool plan_wide_combine(bool sparse, int64_t groups, int64_t splits) {
  return (sparse || groups == 1) && splits > mlav::kOneStageMaxSplits;
}

int make_plan(const mla_dims* d, bool sparse, mla_plan_info* p) {
  const int64_t groups = sparse ? (int64_t)d->batch * d->num_q : d->batch;
  const int64_t rows = sparse ? d->num_heads : (int64_t)d->num_q * d->num_heads;
  const int64_t row_blocks = ceil_div(rows, kRowsPerBlock);
  const int64_t keys = sparse ? d->topk : d->max_kv_len;
  const int64_t tiles = ceil_div(keys, kTile);
  // One workgroup per CU (LDS-bound). Splits keep a minimum of tiles each
  // (mlav::kMinChunkSparse / kMinChunkDense) so the per-split partial (1 KiB per
  // row) stays small next to the split's KV reads and matrix work.
  const int64_t min_chunk = sparse ? mlav::kMinChunkSparse : mlav::kMinChunkDense;
  const int64_t cap = std::max<int64_t>(1, std::min<int64_t>(tiles / min_chunk, mlav::kMaxSplits));
  int64_t splits, chunk, slots;
  int64_t fixed_chunk = 0;
  if (sparse) {
    // Every token has the same number of index tiles: uniform splits.
    splits = d->num_splits > 0 ? d->num_splits
                               : std::max<int64_t>(1, std::min(kPlanCUs / (groups * row_blocks), cap));
    splits = std::min<int64_t>(std::min<int64_t>(splits, tiles), mlav::kMaxSplits);
    chunk = ceil_div(tiles, splits);
    splits = ceil_div(tiles, chunk);
    slots = splits * groups;
  } else {
    // Dense: the host fixes the (sequence, split) slots per row block; the
    // kernels share them out by the sequences' actual lengths (kv_lens lives on
    // the device) and spread each sequence's tiles evenly over its slots.
    if (groups == 1) {
      // One sequence: every slot is one of its splits. Automatic: the fewest
      // splits whose longest one is as short as one workgroup per CU allows
      // (65 tiles over at most 32 slots: 22 splits of at most 3 tiles, not 32
      // of 2-3, which only add partials to write and combine).
      if (d->num_splits > 0) {
        slots = std::min<int64_t>(std::min<int64_t>(d->num_splits, tiles), mlav::kMaxSplits);
      } else {
        const int64_t most = std::max<int64_t>(1, std::min<int64_t>(kPlanCUs / row_blocks, cap));
        slots = ceil_div(tiles, ceil_div(tiles, most));
      }
      splits = slots;
    } else if (d->num_splits > 0) {
      // A requested split count fixes the chunk every sequence is cut by.
      const int64_t req = std::min<int64_t>(std::min<int64_t>(d->num_splits, tiles), mlav::kMaxSplits);
      fixed_chunk = ceil_div(tiles, req);
      splits = ceil_div(tiles, fixed_chunk);
      slots = groups * splits;
    } else {
      slots = std::max<int64_t>(groups, std::min<int64_t>(kPlanCUs / row_blocks, groups * cap));
      splits = std::max<int64_t>(1, slots / groups);  // as if every sequence had max_kv_len keys
      splits = ceil_div(tiles, ceil_div(tiles, splits));
    }
    chunk = ceil_div(tiles, splits);
  }
  const int64_t slot_stride = slots;
  const int64_t grid = sparse ? row_blocks * slots : row_blocks * slot_stride;
  if (grid > 0x7fffffff || slots > 0x7fffffff) return MLA_ERR_INVALID;
  p->num_splits = (int32_t)splits;
  p->chunk_tiles = (int32_t)(fixed_chunk > 0 ? fixed_chunk : chunk);
  p->row_blocks = (int32_t)row_blocks;
  p->num_groups = (int32_t)groups;
  p->rows_per_group = (int32_t)rows;
  p->split_slots = (int32_t)slots;
  // One slot in all: the split kernel writes out/lse directly, no workspace.
  const bool single = sparse ? splits == 1 : slots == 1;
  // records, then (dense, several sequences) the per-sequence record map
  const size_t meta = (!sparse && groups > 1) ? (size_t)groups * sizeof(int2) : 0;
  p->workspace_bytes = single ? 0 : (size_t)slots * row_blocks * kWaves * mlav::kRecBytes + meta;
  return MLA_OK;
}

// ---------------------------------------------------------------------------
// Fixed device scratch of the allocation-free entry point: the split partials
// of calls that cannot allocate a workspace live here. In host code `scratch`
// names only a host-side stand-in: its device address on each GPU comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept; only that address ever reaches a kernel. Every call on one GPU
// shares the array, so calls that overlap on one GPU race.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (first call on a device: looked up
// and kept). MLA_OK, or MLA_ERR_HIP when the runtime fails.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MLA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MLA_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return MLA_ERR_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MLA_OK;
}

// `use_scratch`: take the split partials' memory from the fixed device scratch
// (workspace and workspace_bytes are ignored; a call needing more than
// kScratchBytes is MLA_ERR_SCRATCH) instead of the caller's workspace.
int run(const mla_dims* d, bool sparse, const uint16_t* q_lat, const uint16_t* q_rope,
        const uint16_t* c_kv, const uint16_t* k_rope, const int32_t* page_table,
        const uint8_t* tree_mask, const int32_t* indices, const int32_t* kv_lens, float scale,
        uint16_t* out, float* lse, void* workspace, size_t workspace_bytes, void* stream,
        bool use_scratch = false) {
  if (d == nullptr) return MLA_ERR_INVALID;
  // a page table and a page size come together, or neither does
  if ((page_table != nullptr) != (d->page_size != 0)) return MLA_ERR_INVALID;
  int rc = check_dims(d, sparse, page_table != nullptr);
  if (rc != MLA_OK) return rc;
  if (!q_lat || !q_rope || !c_kv || !k_rope || !kv_lens || !out || !lse) return MLA_ERR_INVALID;
  if (sparse && !indices) return MLA_ERR_INVALID;
  if (!aligned(q_lat, 16) || !aligned(q_rope, 16) || !aligned(c_kv, 16) || !aligned(k_rope, 16) ||
      !aligned(out, 16) || !aligned(lse, 4) || !aligned(kv_lens, 4))
    return MLA_ERR_INVALID;
  if ((page_table && !aligned(page_table, 4)) || (indices && !aligned(indices, 4)))
    return MLA_ERR_INVALID;
  // softmax scale: finite and positive (masked keys are -inf scores)
  if (!(scale > 0.0f) || !(scale < __builtin_inff())) return MLA_ERR_INVALID;
  mla_plan_info p;
  rc = make_plan(d, sparse, &p);
  if (rc != MLA_OK) return rc;
  if (use_scratch) {
    if (p.workspace_bytes > kScratchBytes) return MLA_ERR_SCRATCH;
  } else if (p.workspace_bytes > 0) {
    if (workspace == nullptr || workspace_bytes < p.workspace_bytes || !aligned(workspace, 16))
      return MLA_ERR_WORKSPACE;
  }
  rc = check_device();
  if (rc != MLA_OK) return rc;
  if (use_scratch && p.workspace_bytes > 0) {
    rc = scratch_address(&workspace);
    if (rc != MLA_OK) return rc;
  }

  mlav::MainArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q_lat = q_lat;
  a.q_rope = q_rope;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.page_table = page_table;
  a.tree_mask = sparse ? nullptr : tree_mask;
  a.kv_lens = kv_lens;
  a.indices = sparse ? indices : nullptr;
  a.out = out;
  a.lse = lse;
  if (p.workspace_bytes > 0) {
    const size_t records = (size_t)p.split_slots * p.row_blocks * kWaves;
    a.ws_o = static_cast<uint16_t*>(workspace);
    a.ws_lse = reinterpret_cast<float*>(a.ws_o + records * mlav::kRecElems);
    if (!sparse && p.num_groups > 1)
      a.ws_meta = reinterpret_cast<int2*>(a.ws_lse + records * mlav::kRecRowStats * mlav::kRowsPerWave);
    a.wide_combine = plan_wide_combine(sparse, p.num_groups, p.num_splits) ? 1 : 0;
  }
  a.kv_seq_stride = page_table ? 0 : d->kv_seq_stride;
  a.kv_rows = d->kv_rows;
  a.T = d->num_q;
  a.H = d->num_heads;
  a.rows_per_group = p.rows_per_group;
  a.num_groups = p.num_groups;
  a.row_blocks = p.row_blocks;
  a.page_size = page_table ? d->page_size : 0;
  a.max_pages = page_table ? d->max_pages : 0;
  a.max_kv_len = d->max_kv_len;
  a.topk = sparse ? d->topk : 0;
  a.num_splits = p.num_splits;
  a.chunk_tiles = p.chunk_tiles;
  a.split_slots = p.split_slots;
  a.slot_stride = p.split_slots;
  a.fixed_chunk = (!sparse && d->num_splits > 0) ? p.chunk_tiles : 0;
  a.final_out = p.workspace_bytes == 0 ? 1 : 0;
  a.scale_log2 = scale * 1.4426950408889634f;

  const int mode = sparse ? (page_table ? mlav::kSparsePaged : mlav::kSparse)
                          : (page_table ? mlav::kPaged : mlav::kContig);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // With a single split the split kernel writes out/lse itself and there is
  // nothing to combine.
  if (d->phase != MLA_PHASE_COMBINE) {
    if (mlav::launch_split_kernel(a, mode, s) != hipSuccess) return MLA_ERR_HIP;
  }
  if (!a.final_out && d->phase != MLA_PHASE_PARTIAL) {
    if (mlav::launch_combine_kernel(a, mode, s) != hipSuccess) return MLA_ERR_HIP;
  }
  return MLA_OK;
}

}  // namespace

extern "C" {

int mla_verify_plan(const mla_dims* dims, int sparse, mla_plan_info* plan) {
  if (plan == nullptr || dims == nullptr) return MLA_ERR_INVALID;
  const int rc = check_dims(dims, sparse != 0, dims->page_size != 0);
  if (rc != MLA_OK) return rc;
  return make_plan(dims, sparse != 0, plan);
}

size_t mla_verify_workspace_bytes(const mla_dims* dims, int sparse) {
  mla_plan_info p;
  if (mla_verify_plan(dims, sparse, &p) != MLA_OK) return 0;
  return p.workspace_bytes;
}

int mla_verify_attn(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                    const uint16_t* c_kv, const uint16_t* k_rope, const int32_t* page_table,
                    const uint8_t* tree_mask, const int32_t* kv_lens, float scale,
                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return run(dims, false, q_lat, q_rope, c_kv, k_rope, page_table, tree_mask, nullptr, kv_lens,
             scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_sparse_attn(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                    const uint16_t* c_kv, const uint16_t* k_rope, const int32_t* page_table,
                    const int32_t* indices, const int32_t* kv_lens, float scale,
                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream) {
  return run(dims, true, q_lat, q_rope, c_kv, k_rope, page_table, nullptr, indices, kv_lens,
             scale, out, lse, workspace, workspace_bytes, stream);
}

int mla_verify_attn_noalloc(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                            const uint16_t* c_kv, const uint16_t* k_rope,
                            const int32_t* page_table, const uint8_t* tree_mask,
                            const int32_t* kv_lens, float scale, uint16_t* out, float* lse,
                            void* stream) {
  return run(dims, false, q_lat, q_rope, c_kv, k_rope, page_table, tree_mask, nullptr, kv_lens,
             scale, out, lse, nullptr, 0, stream, /*use_scratch=*/true);
}

int mla_compact_kv(const mla_dims* dims, uint16_t* c_kv, uint16_t* k_rope,
                   const int32_t* page_table, const int32_t* kv_lens, const int32_t* accepted,
                   const int32_t* num_accepted, int32_t* new_kv_lens, void* stream) {
  if (dims == nullptr) return MLA_ERR_INVALID;
  if ((page_table != nullptr) != (dims->page_size != 0)) return MLA_ERR_INVALID;
  int rc = check_dims(dims, false, page_table != nullptr);
  if (rc != MLA_OK) return rc;
  if (!c_kv || !k_rope || !kv_lens || !accepted || !num_accepted || !new_kv_lens)
    return MLA_ERR_INVALID;
  if (!aligned(c_kv, 16) || !aligned(k_rope, 16) || !aligned(kv_lens, 4) || !aligned(accepted, 4) ||
      !aligned(num_accepted, 4) || !aligned(new_kv_lens, 4) || (page_table && !aligned(page_table, 4)))
    return MLA_ERR_INVALID;
  rc = check_device();
  if (rc != MLA_OK) return rc;
  mlav::CompactArgs a;
  std::memset(&a, 0, sizeof(a));
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.page_table = page_table;
  a.kv_lens = kv_lens;
  a.accepted = accepted;
  a.num_accepted = num_accepted;
  a.new_kv_lens = new_kv_lens;
  a.kv_seq_stride = page_table ? 0 : dims->kv_seq_stride;
  a.kv_rows = dims->kv_rows;
  a.T = dims->num_q;
  a.page_size = page_table ? dims->page_size : 0;
  a.max_pages = page_table ? dims->max_pages : 0;
  a.max_kv_len = dims->max_kv_len;
  if (mlav::launch_compact_kernel(a, dims->batch, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_head_project(int32_t tokens, int32_t heads, int32_t in_dim, int32_t out_dim,
                     const uint16_t* x, const uint16_t* w, uint16_t* y, void* stream) {
  if (tokens < 1 || heads < 1 || in_dim < 16 || in_dim > 1024 || in_dim % 16 != 0 ||
      out_dim < 32 || out_dim % 32 != 0)
    return MLA_ERR_INVALID;
  if ((int64_t)in_dim * out_dim >= ((int64_t)1 << 30)) return MLA_ERR_INVALID;
  if ((int64_t)tokens * heads * std::max(in_dim, out_dim) >= ((int64_t)1 << 40)) return MLA_ERR_INVALID;
  if ((int64_t)heads * (out_dim / 32) > 0x7fffffff) return MLA_ERR_INVALID;
  if (!x || !w || !y || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return MLA_ERR_INVALID;
  const int rc = check_device();
  if (rc != MLA_OK) return rc;
  mlav::ProjArgs a;
  a.x = x;
  a.w = w;
  a.y = y;
  a.tokens = tokens;
  a.heads = heads;
  a.in_dim = in_dim;
  a.out_dim = out_dim;
  if (mlav::launch_proj_kernel(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

size_t mla_select_topk_workspace_bytes(int32_t rows, int32_t row_len) {
  if (rows < 1 || row_len < 1) return 0;
  // Any device cuts a row into at most `pieces` pieces (the count for unlimited
  // CUs) of whole 1024-score steps, so pieces x chunk <= row_len + 1024 x pieces.
  const int pieces = topk_pieces(rows, row_len, INT32_MAX / 4, nullptr);
  if (pieces <= 1) return 0;
  return (size_t)((int64_t)rows * pieces * mlav::topk_piece_bytes +
                  (int64_t)rows * ((int64_t)row_len + 1024 * (int64_t)pieces) * 8);
}

int mla_select_topk(int32_t rows, int32_t row_len, int64_t row_stride, int32_t k,
                    const float* scores, const int32_t* row_lens, int32_t* indices,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (rows < 1 || row_len < 1 || row_stride < row_len || k < 1 || k > (1 << 20)) return MLA_ERR_INVALID;
  if (row_stride % 4 != 0) return MLA_ERR_INVALID;  // rows are read 16 bytes at a time
  if (!scores || !indices || !aligned(scores, 16) || !aligned(indices, 4) ||
      (row_lens && !aligned(row_lens, 4)) || (workspace && !aligned(workspace, 16)))
    return MLA_ERR_INVALID;
  int chunk = row_len;
  const int pieces = workspace ? topk_pieces(rows, row_len, kPlanCUs, &chunk) : 1;
  if (pieces > 1 && workspace_bytes < (size_t)mlav::topk_workspace_bytes(rows, pieces, chunk))
    return MLA_ERR_WORKSPACE;
  const int rc = check_device();
  if (rc != MLA_OK) return rc;
  mlav::TopkArgs a;
  a.scores = scores;
  a.row_lens = row_lens;
  a.indices = indices;
  a.row_stride = row_stride;
  a.rows = rows;
  a.row_len = row_len;
  a.k = k;
  a.chunks = pieces;
  a.chunk = pieces > 1 ? chunk : row_len;
  a.ws = pieces > 1 ? workspace : nullptr;
  if (mlav::launch_topk_kernel(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_probe_mfma_bf16(int32_t blocks, int32_t iters, float* sink, void* stream) {
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000) return MLA_ERR_INVALID;
  if (!sink || !aligned(sink, 4)) return MLA_ERR_INVALID;
  const int rc = check_device();
  if (rc != MLA_OK) return rc;
  if (mlav::launch_probe_mfma(sink, blocks, iters, static_cast<hipStream_t>(stream)) != hipSuccess)
    return MLA_ERR_HIP;
  return MLA_OK;
}

int mla_probe_gather_rows(const uint16_t* c_kv, const uint16_t* k_rope, int64_t kv_rows,
                          int64_t kv_seq_stride, const int32_t* indices, int32_t groups,
                          int32_t per_group, int32_t tokens_per_seq, float* sink, void* stream) {
  if (!c_kv || !k_rope || !indices || !sink || !aligned(c_kv, 16) || !aligned(k_rope, 16) ||
      !aligned(indices, 4) || !aligned(sink, 4))
    return MLA_ERR_INVALID;
  if (kv_rows < 1 || kv_seq_stride < 0 || groups < 1 || per_group < 1 || tokens_per_seq < 1)
    return MLA_ERR_INVALID;
  // byte offsets within one sequence's rows stay below 2^31
  if ((kv_seq_stride > 0 ? kv_seq_stride : kv_rows) > ((int64_t)1 << 21)) return MLA_ERR_INVALID;
  if ((int64_t)groups * ((per_group + 63) / 64) > 0x7fffffffLL) return MLA_ERR_INVALID;
  const int rc = check_device();
  if (rc != MLA_OK) return rc;
  mlav::GatherProbeArgs a;
  a.c_kv = c_kv;
  a.k_rope = k_rope;
  a.indices = indices;
  a.sink = sink;
  a.kv_seq_stride = kv_seq_stride;
  a.kv_rows = kv_rows;
  a.groups = groups;
  a.per_group = per_group;
  a.tokens_per_seq = tokens_per_seq;
  if (mlav::launch_probe_gather(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MLA_ERR_HIP;
  return MLA_OK;
}

const char* mla_verify_strerror(int code) {
  switch (code) {
    case MLA_OK: return "success";
    case MLA_ERR_INVALID: return "invalid argument";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP runtime or launch failure";
    case MLA_ERR_UNSUPPORTED: return "device is not gfx950";
    case MLA_ERR_SCRATCH: return "call needs more than the fixed device scratch of the allocation-free entry point";
    default: return "unknown error code";
  }
}

}  // extern "C"
