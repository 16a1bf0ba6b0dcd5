/*
 * mla_verify.h — C ABI of the MI355X (gfx950) MLA tree-verify attention library.
 *
 * Operation (both entry points): absorbed Multi-head Latent Attention for the
 * draft tokens of a speculative-decoding tree. Every head of every draft token
 * attends to one latent cache shared by all heads — a 512-wide latent row
 * (c_kv) plus a 64-wide rotary row (k_rope) per cached token — under a
 * prefix-plus-tree-ancestor mask, with a streaming (online) softmax that never
 * materialises a score row.
 *   - "The Shared Memory Ceiling", section "The Broader Context: Building a
 *     Custom sm_120 Verify Kernel": verify attention inside DFlash/DDTree
 *     speculative decoding; the MLA latent read once per head-tile instead of
 *     once per head.
 *   - same page, section "The Guard: Turning a Limitation into a
 *     Demonstration": the Dl (latent) and Dr (rope) widths.
 *   - same page, section "Technical Deep Dive: Why Shared Memory Matters":
 *     score every visible key, normalise, take the weighted sum of the
 *     512-dimensional values; online softmax keeps a running max and sum and
 *     rescales earlier accumulations when the max grows.
 *   - "The SMEM Ceiling", section "The Problem Space: Sparse Decode on
 *     Blackwell": the sparse variant, where each token attends only to a top-k
 *     index set, computed by a split kernel.
 *
 * For sequence b, draft token t, head h (row r = t*H + h):
 *     s_p  = scale * (q_lat[b,t,h,:] . c_kv[row(p),:] + q_rope[b,t,h,:] . k_rope[row(p),:])
 *     lse  = ln sum_{p in V} exp(s_p)                           (natural log, fp32)
 *     out  = sum_{p in V} exp(s_p - lse) * c_kv[row(p),:]       (bf16, round-to-nearest-even)
 * The values are the latent rows themselves: out stays in the 512-wide latent
 * space (the per-head up-projection is outside this library), and k_rope is
 * used only in the scores. RoPE is not applied here: q_rope and k_rope arrive
 * already rotated. An empty visible set yields out = 0 and lse = -inf.
 *
 * Visible set V:
 *   dense  (mla_verify_attn): the prefix positions p < kv_lens[b] - T, and
 *          draft position kv_lens[b] - T + j whenever tree_mask[b,t,j] != 0
 *          (a NULL tree_mask means a chain: j <= t). The T draft keys are the
 *          last T positions of each sequence.
 *   sparse (mla_sparse_attn): the positions indices[b,t,0..topk), shared by
 *          all heads of token (b,t). Entries outside [0, kv_lens[b]) select
 *          nothing (so -1 pads a short index list).
 *
 * Physical row of logical position p of sequence b:
 *   contiguous (page_size == 0, page_table == NULL): b * kv_seq_stride + p
 *   paged      (page_size  > 0, page_table != NULL):
 *              page_table[b * max_pages + p / page_size] * page_size + p % page_size
 *
 * Layouts (all row-major, all device memory, all caller-owned):
 *   q_lat   bf16 [B, T, H, 512]        q_rope  bf16 [B, T, H, 64]
 *   c_kv    bf16 [kv_rows, 512]        k_rope  bf16 [kv_rows, 64]
 *   out     bf16 [B, T, H, 512]        lse     fp32 [B, T, H]
 *   kv_lens i32  [B]                   tree_mask u8 [B, T, T] or NULL
 *   page_table i32 [B, max_pages] or NULL   indices i32 [B, T, topk]
 *   bf16 is passed as its 16-bit pattern (uint16_t).
 *
 * Ownership and execution: the library never allocates, frees or
 * synchronises, and never reads device data on the host. Work is enqueued
 * on `stream` (a hipStream_t; NULL = the default stream) and returns
 * immediately; inputs must stay alive until the stream work completes. Calls
 * keep no state between them (a per-device capability check is cached) and
 * may be captured into a HIP graph. Split-KV calls need a caller-provided
 * device workspace of mla_verify_plan(...).workspace_bytes bytes; two calls in
 * flight at once must not share one workspace.
 *
 * Errors: every function returns 0 on success or a negative MLA_ERR_* code.
 * All argument checks run before any HIP call. Outputs are unspecified after
 * an error. kv_lens[b] values are clamped to [0, max_kv_len] on the device;
 * page_table entries that point outside [0, kv_rows) read as absent keys.
 * No C++ exception crosses this boundary.
 */
#ifndef MLA_VERIFY_H
#define MLA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_OK 0
#define MLA_ERR_INVALID (-1)     /* bad argument: see the checks listed below */
#define MLA_ERR_WORKSPACE (-2)   /* workspace NULL or smaller than the plan's workspace_bytes */
#define MLA_ERR_HIP (-3)         /* a HIP runtime call or kernel launch failed */
#define MLA_ERR_UNSUPPORTED (-4) /* the current device is not gfx950 */
#define MLA_ERR_SCRATCH (-5)     /* mla_verify_attn_noalloc: the call's partials exceed the
                                    library's fixed device scratch */

#define MLA_LATENT_DIM 512
#define MLA_ROPE_DIM 64
#define MLA_MAX_DRAFT 64  /* T limit: one 64-bit visibility word per query row */
#define MLA_KV_TILE 64    /* keys per LDS tile; page_size must be a multiple */
/* fixed device scratch behind mla_verify_attn_noalloc (per GPU, process lifetime) */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* Which kernels a call enqueues. PARTIAL runs only the split-KV kernel (it
 * writes the per-split partial results into the workspace, or the final
 * out/lse when the plan has one split); COMBINE runs only the log-sum-exp
 * merge of those partials into out/lse. ALL runs both. A PARTIAL call
 * followed by a COMBINE call with identical arguments equals one ALL call. */
#define MLA_PHASE_ALL 0
#define MLA_PHASE_PARTIAL 1
#define MLA_PHASE_COMBINE 2

typedef struct mla_dims {
  int32_t batch;         /* B >= 1 */
  int32_t num_q;         /* T, 1..64 draft (query) tokens per sequence */
  int32_t num_heads;     /* H >= 1 */
  int32_t page_size;     /* 0 = contiguous cache; else tokens per page (multiple of 64) */
  int32_t max_pages;     /* paged: entries per sequence in page_table */
  int32_t max_kv_len;    /* host-known upper bound on kv_lens[]; plans the grid */
  int64_t kv_seq_stride; /* contiguous: rows between consecutive sequences */
  int64_t kv_rows;       /* rows of the c_kv and k_rope allocations */
  int32_t topk;          /* sparse: index-list length per token (ignored by the dense call) */
  int32_t num_splits;    /* 0 = automatic; else requested KV splits per query group, capped
                            at the group's 64-key tile count and at 256 (the plan reports
                            the splits used). A single dense sequence spreads its tiles
                            evenly over exactly that many splits; batches and sparse
                            calls cut every group into chunks of ceil(tiles / splits). */
  int32_t phase;         /* MLA_PHASE_* */
  int32_t reserved;      /* must be 0 */
} mla_dims;

typedef struct mla_plan_info {
  int32_t num_splits;     /* KV splits per query group (dense: for a group of max_kv_len keys) */
  int32_t chunk_tiles;    /* most 64-key tiles in one split (dense: for a group of max_kv_len keys) */
  int32_t row_blocks;     /* 128-row blocks per query group */
  int32_t num_groups;     /* query groups: B (dense) or B*T (sparse) */
  int32_t rows_per_group; /* T*H (dense) or H (sparse) */
  int32_t split_slots;    /* (group, split) slots per row block; the workspace holds
                             split_slots * row_blocks * 4 records */
  size_t workspace_bytes; /* device bytes the call needs; 0 when there is one slot in all */
} mla_plan_info;

/* Work decomposition of a call with these dims (sparse != 0: mla_sparse_attn).
 * A pure function of the dims: host arithmetic only, no HIP call, planned for
 * gfx950's 256 compute units whatever device is current. Returns
 * MLA_ERR_INVALID for dims the call would reject. */
int mla_verify_plan(const mla_dims* dims, int sparse, mla_plan_info* plan);

/* Convenience: mla_verify_plan(...).workspace_bytes, or 0 on invalid dims. */
size_t mla_verify_workspace_bytes(const mla_dims* dims, int sparse);

/* Dense tree-verify attention (see the file comment for the operation).
 * Checks (MLA_ERR_INVALID): dims, q_lat, q_rope, c_kv, k_rope, kv_lens, out,
 * lse non-NULL; bf16 arrays 16-byte aligned, lse/kv_lens/page_table 4-byte
 * aligned; scale finite and > 0; B >= 1, 1 <= T <= 64, H >= 1;
 * T <= max_kv_len; B * ceil(max_kv_len / 64) < 2^31; num_splits >= 0;
 * phase valid; reserved == 0; contiguous: page_table NULL, page_size 0,
 * kv_seq_stride >= max_kv_len and (B-1)*kv_seq_stride + max_kv_len <= kv_rows;
 * paged: page_table non-NULL, page_size a positive multiple of 64,
 * max_pages * page_size >= max_kv_len. */
int mla_verify_attn(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                    const uint16_t* c_kv, const uint16_t* k_rope, const int32_t* page_table,
                    const uint8_t* tree_mask, const int32_t* kv_lens, float scale,
                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Allocation-free variant of mla_verify_attn, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid allocation. Same arguments, checks, operation and
 * results as mla_verify_attn with a workspace (the same kernels run), but the
 * split partials live in a fixed device array inside the library instead of a
 * caller workspace: MLA_NOALLOC_SCRATCH_BYTES bytes (64 MiB), held on
 * each GPU the library runs on until the process ends. A call whose plan needs
 * more (mla_verify_plan(...).workspace_bytes larger than that) returns
 * MLA_ERR_SCRATCH before any HIP call. The first call on each device looks up
 * that device's copy of the array (a runtime symbol lookup, no allocation by
 * the library); no call allocates or frees. Every call on one GPU shares the
 * array, which keeps the last call's contents (the kernels write every record
 * before reading it, so nothing needs clearing): calls that overlap on one
 * GPU (other streams, other threads) race and give undefined results. */
int mla_verify_attn_noalloc(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                            const uint16_t* c_kv, const uint16_t* k_rope,
                            const int32_t* page_table, const uint8_t* tree_mask,
                            const int32_t* kv_lens, float scale, uint16_t* out, float* lse,
                            void* stream);

/* Sparse top-k attention: token (b,t) sees indices[b,t,0..topk) (logical
 * positions of sequence b), shared by its H heads; no tree mask. Same checks
 * as mla_verify_attn (minus the tree mask), plus: indices non-NULL and 4-byte
 * aligned, topk >= 1; contiguous: kv_seq_stride <= 2^21 rows; paged:
 * kv_rows <= 2^21 (the gather addresses rows with 32-bit byte offsets). */
int mla_sparse_attn(const mla_dims* dims, const uint16_t* q_lat, const uint16_t* q_rope,
                    const uint16_t* c_kv, const uint16_t* k_rope, const int32_t* page_table,
                    const int32_t* indices, const int32_t* kv_lens, float scale,
                    uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Post-verify KV compaction. "The Shared Memory Ceiling", section "The Broader
 * Context: Building a Custom sm_120 Verify Kernel", names a "defrag" step after
 * verification; its plain reading: the cache rows of the accepted draft tokens
 * move, in path order, to the front of the draft region, so the next decoding
 * step sees prefix + accepted tokens as one contiguous run.
 *
 * For sequence b: kv = kv_lens[b] clamped to [0, max_kv_len], P = kv - T,
 * n = num_accepted[b] clamped to [0, T], and for i < n
 *     row(P + i) <- row(P + accepted[b, i])        (c_kv and k_rope rows)
 *     new_kv_lens[b] = max(P + n, 0).
 * Every source row is read before any destination row is written, so moves
 * that overlap are well defined (a root-to-node path has accepted[b,i] >= i;
 * any order is accepted). A move is skipped when its draft index is outside
 * [0, T), either position is outside [0, kv), or either physical row is absent
 * (page-table entry < 0 or row >= kv_rows). Rows of other positions are not
 * touched. Sequences must not share the pages that hold their draft regions.
 *
 * dims: the verify call's dims (batch, num_q = T, page_size, max_pages,
 * max_kv_len, kv_seq_stride, kv_rows; the same checks as mla_verify_attn).
 * c_kv bf16 [kv_rows, 512] and k_rope bf16 [kv_rows, 64] are updated in place
 * (16-byte aligned); accepted i32 [B, T], num_accepted i32 [B], new_kv_lens
 * i32 [B] (may alias kv_lens), all 4-byte aligned device memory. Enqueued on
 * `stream`; no workspace. Returns MLA_OK or a negative MLA_ERR_* code. */
int mla_compact_kv(const mla_dims* dims, uint16_t* c_kv, uint16_t* k_rope,
                   const int32_t* page_table, const int32_t* kv_lens, const int32_t* accepted,
                   const int32_t* num_accepted, int32_t* new_kv_lens, void* stream);

/* Per-head projection around absorbed attention: for every token m and head h
 *     y[m, h, :] = x[m, h, :] . w[h]          (w[h] is in_dim x out_dim)
 * in bf16 with fp32 accumulation and a round-to-nearest-even bf16 result.
 * Absorbed MLA ("The Shared Memory Ceiling", section "The Broader Context:
 * Building a Custom sm_120 Verify Kernel": attention over the shared MLA
 * latent) uses it on both sides of mla_verify_attn: the query absorption
 * q_lat = q_nope . W_UK (in_dim 128, out_dim 512) and the per-head output
 * o = out . W_UV (in_dim 512, out_dim 128).
 *
 * x bf16 [tokens, heads, in_dim], w bf16 [heads, in_dim, out_dim], y bf16
 * [tokens, heads, out_dim], row-major, 16-byte aligned device memory, caller
 * owned; y must not overlap x or w. Checks (MLA_ERR_INVALID): tokens >= 1,
 * heads >= 1, in_dim a multiple of 16 in [16, 1024], out_dim a multiple of 32,
 * in_dim * out_dim < 2^30, tokens * heads * max(in_dim, out_dim) < 2^40.
 * Enqueued on `stream`; no workspace. */
int mla_head_project(int32_t tokens, int32_t heads, int32_t in_dim, int32_t out_dim,
                     const uint16_t* x, const uint16_t* w, uint16_t* y, void* stream);

/* Top-k index selection for the sparse path ("The SMEM Ceiling", section "The
 * Problem Space: Sparse Decode on Blackwell": each decode token attends only to
 * the top-k set an index-selection step picks). The scores are inputs.
 *
 * For each row r (a query token) with n = row_lens[r] clamped to [0, row_len]
 * candidates (row_len when row_lens is NULL): positions p < n are ranked by
 * scores[r, p] (IEEE-754 total order of float32: -inf < ... < -0.0 < +0.0 < ...
 * < +inf, every NaN below every number), ties by lower p; the first min(k, n)
 * positions are written to indices[r, :] in ascending order and the rest of the
 * k slots are -1 (which mla_sparse_attn skips).
 *
 * scores fp32 [rows, row_stride] (16-byte aligned, row_stride >= row_len and a
 * multiple of 4: rows are read 16 bytes at a time), row_lens i32 [rows] or
 * NULL, indices i32 [rows, k] (4-byte aligned device memory). Checks
 * (MLA_ERR_INVALID): those, rows >= 1, row_len >= 1, 1 <= k <= 2^20, pointers
 * non-NULL, workspace 16-byte aligned when given.
 *
 * workspace: NULL runs one workgroup per row (no scratch memory). With a
 * device buffer of at least mla_select_topk_workspace_bytes(rows, row_len)
 * bytes, rows are spread over several workgroups when there are too few rows
 * to fill the GPU (three kernel launches; the buffer holds per-piece digit
 * histograms and counts and room for every score as a candidate, about
 * 8 bytes per score, and every call writes what it later reads, so it needs no
 * clearing).
 * A smaller non-NULL buffer than that path needs is MLA_ERR_WORKSPACE. The
 * result is identical either way. Calls sharing one workspace must be ordered
 * on one stream. Enqueued on `stream`. */
int mla_select_topk(int32_t rows, int32_t row_len, int64_t row_stride, int32_t k,
                    const float* scores, const int32_t* row_lens, int32_t* indices,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for mla_select_topk's several-workgroup path on any device
 * (0 when rows are never split: row_len <= 4096 or invalid arguments):
 * rows x (up to 32 pieces x 1,056 + (row_len + 1,024 x pieces) x 8). */
size_t mla_select_topk_workspace_bytes(int32_t rows, int32_t row_len);

/* Static description of an error code (never NULL). */
const char* mla_verify_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* MLA_VERIFY_H */
