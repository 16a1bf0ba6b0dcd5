// MLA tree-verify attention kernels for gfx950 (CDNA4).
//
// What is computed ("The Shared Memory Ceiling", sections "The Broader
// Context" and "Technical Deep Dive: Why Shared Memory Matters"): every query
// row (draft token t, head h) scores the visible keys of one latent cache
// (512 latent + 64 rope dims, shared by all heads), and returns the
// softmax-weighted sum of the 512-wide latent rows plus the log-sum-exp. The
// score row is never stored: an online softmax keeps a running max and sum per
// row and rescales the accumulator when the max grows. Long key ranges are
// split across workgroups and merged by a log-sum-exp combine (the "split
// kernel" of "The SMEM Ceiling", section "The Problem Space").
//
// Design on gfx950 (the pages' sm_120 head-tile of 8 heads is prior art):
//  * A workgroup is 4 waves x 32 query rows = 128 rows that share every KV
//    tile; 2 LDS stages of 64 keys (73,728 B each) fit the 160 KB LDS.
//  * Tiles move HBM -> LDS with 16-byte buffer loads that write LDS directly
//    (buffer_load_dwordx4 ... lds). Buffer range checks zero-fill keys past the
//    end of a sequence, outside the index set, or on an invalid page, so masked
//    value rows are 0 (never stale NaN) in the PV product.
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 with the K tile as the LDS
//    operand and Q held in registers. In the 32x32 accumulator layout each lane
//    then owns one query row (16 keys per block, two lanes per row), so the row
//    max is an in-lane max plus one exchange with lane^32, and the row sum stays
//    per-lane until the end.
//  * The same accumulator registers, rounded to bf16, are directly the B
//    operand of O^T += V^T * P^T (the key order inside each 16-key step is
//    permuted identically on both operands). V^T comes from the row-major tile
//    through ds_read_b64_tr_b16 (transposing LDS read), so K and V share one
//    tile (MLA's value rows are the first 512 dims of its key rows).
//  * The 256 accumulator registers per lane are not rescaled tile by tile (a
//    VALU rescale in the loop pulls them out of the accumulation registers):
//    exponents use a fixed per-row reference, raised by an exact power of two
//    at the end of a tile whose terms sum past 2^32, with a two-pass fallback
//    when a single tile exceeds it by more than 2^96.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"
#include "mla_internal.h"

namespace mlav {


constexpr int kLatBytes = kTile * kDL * 2;    // 65536: latent part of a tile
constexpr int kRopeBytes = kTile * kDR * 2;   // 8192: rope part of a tile
constexpr int kStageBytes = kLatBytes + kRopeBytes;  // 73728
constexpr int kStages = 2;
constexpr int kLdsBytes = kStages * kStageBytes;  // 147456
constexpr int kQLatBytes = kRowsPerWave * kDL * 2;           // 32768: a wave's latent query rows
constexpr int kQWaveBytes = kQLatBytes + kRowsPerWave * kDR * 2;  // 36864: with the rope rows
static_assert(kWaves * kQWaveBytes == kLdsBytes && 2 * kQWaveBytes == kStageBytes,
              "a row block's query rows fill both stages, two waves' rows one stage");
static_assert(kLdsBytes + 16 <= 163840, "two KV stages must fit one gfx950 CU's 160 KB LDS");
constexpr int kLoadsPerStage = kStageBytes / (64 * 16);  // 72 wave-wide 16-byte loads
static_assert(kLoadsPerStage == 72 && kLoadsPerStage % kWaves == 0, "load split");
constexpr unsigned kOobOffset = 0x80000000u;     // an offset every range check rejects
// Exponent reference bounds (log2 units). A tile whose row sum reaches
// 2^kRaiseLog2 raises the row's reference at the tile's end (an exact
// power-of-two rescale); one that reaches 2^kRerunLog2 (a single tile more than
// ~96 log2 units above the reference, where an fp32 term could overflow) makes
// the split run again with the reference at that tile's maximum.
constexpr float kRaiseLog2 = 32.0f;
constexpr float kRerunLog2 = 96.0f;
constexpr float kLn2 = 0.69314718055994530942f;
// LDS fragments in flight ahead of the MFMA that consumes them: one wave per
// SIMD leaves nothing else to cover the LDS latency.
#ifndef MLA_FRAG_AHEAD
#define MLA_FRAG_AHEAD 2
#endif
constexpr int kFragAhead = MLA_FRAG_AHEAD;

// ---------------------------------------------------------------------------
// LDS swizzles. A tile is stored row-major (key-major) with its 16-byte chunks
// permuted inside each key row so that both read patterns are free of bank
// conflicts on the 64 four-byte LDS banks:
//  - S^T operand (16-byte reads, 16 lanes per bank pass): 16 consecutive keys
//    read the same logical chunk, so swz_lat must be a bijection on key mod 16;
//  - V^T operand (transposing 8-byte reads, 32 lanes per bank pass): 4
//    consecutive keys read the same 4 aligned logical chunks, so swz_lat must
//    give the 4 keys of an aligned quad distinct values in bits 2..3.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz_lat(int key) {  // permutes the low 4 chunk bits
  return ((key & 3) << 2) | ((key >> 2) & 3);
}
__device__ __forceinline__ int swz_rope(int key) {  // permutes the 3 chunk bits
  return ((key >> 1) ^ (key << 2)) & 7;
}

// Score MFMAs with VGPR accumulators. Every accumulating MFMA in a function is
// otherwise given AGPR accumulators, and the 256 output accumulators already
// fill the AGPR file; scores are consumed by VALU code, so they belong in VGPRs.
// The hardware resolves back-to-back accumulation into the same registers;
// reading the result with VALU needs the wait states of score_fence().
__device__ __forceinline__ f32x16 mfma32_v_first(bf16x8 a, bf16x8 b) {
  f32x16 d;
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ void mfma32_v_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// Independent-instruction wait states between the last score MFMA and the VALU
// reads and writes of its result (scores are touched by nothing else): 12, the
// count the compiler itself puts between v_mfma_f32_32x32x16_bf16 and a VALU
// read of its result on gfx950.
__device__ __forceinline__ void score_fence(f32x16& s) {
  asm volatile("s_nop 11" : "+v"(s));
}

// Two floats times a scale, each rounded once (to nearest even) to fp16, packed
// low = x0: the low half written by v_fma_mixlo_f16, the high half by
// v_fma_mixhi_f16 into the same register (no separate shift and merge).
__device__ __forceinline__ uint32_t scale_pack_f16x2(float x0, float x1, float s) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %3, 0 op_sel_hi:[0,0,0]\n\t"
      "v_fma_mixhi_f16 %0, %2, %3, 0 op_sel_hi:[0,0,0]"
      : "=&v"(r) : "v"(x0), "v"(x1), "v"(s));
  return r;
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }


// Keys of one query group and how its tiles are split (shared by both kernels).
struct GroupInfo {
  int b;        // sequence
  int kv_len;   // clamped kv_lens[b]
  int n_tiles;  // 64-key tiles covering the group's key list
};

__device__ __forceinline__ int clamped_kv_len(const MainArgs& a, int b) {
  const int kv = a.kv_lens[b];
  return kv < 0 ? 0 : (kv > a.max_kv_len ? a.max_kv_len : kv);
}

__device__ __forceinline__ GroupInfo group_info(const MainArgs& a, int group, bool sparse) {
  GroupInfo g;
  g.b = sparse ? group / a.T : group;
  g.kv_len = clamped_kv_len(a, g.b);
  const int n_keys = sparse ? a.topk : g.kv_len;
  g.n_tiles = (n_keys + kTile - 1) / kTile;
  return g;
}

// ---------------------------------------------------------------------------
// Dense split plan, computed on the device from kv_lens (the host only fixes
// the number of (sequence, split) slots, a.split_slots = P, per row block).
// Every sequence b with t_b tiles gets n_b = max(1, ceil(t_b / C)) consecutive
// slots, where the chunk C is the smallest value >= max(kMinChunkDense, ceil(sum t / P),
// ceil(max t / kMaxSplits)) with sum_b n_b <= P, so a ragged batch spreads its
// tiles evenly over the slots instead of planning every sequence for the
// longest one. Within a sequence the tiles are then spread evenly over its
// slots. Pure integer arithmetic over kv_lens, evaluated identically by every
// wave of both kernels (all lanes of a wave take part; results are uniform).
// ---------------------------------------------------------------------------
// Wave reductions. The result is the same in every lane; readfirstlane tells
// the compiler so, which keeps everything derived from it (split bounds, tile
// loop counters) in scalar registers and the tile loop free of divergence.
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, __shfl_xor(v, o));
  return __builtin_amdgcn_readfirstlane(v);
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int seq_slots(int t, int chunk) { return t > 0 ? (t + chunk - 1) / chunk : 1; }
__device__ __forceinline__ int seq_tiles(const MainArgs& a, int b) {
  return (clamped_kv_len(a, b) + kTile - 1) / kTile;
}

// Tiles of sequence `lane` (lane < num_groups <= 64), or of lane-strided
// sequences when the batch is larger; one read of kv_lens per wave.
struct BatchTiles {
  int t;      // tiles of sequence i0 + lane for the first block (i0 = 0)
  bool small; // num_groups <= 64: t covers the whole batch
};
__device__ __forceinline__ BatchTiles batch_tiles(const MainArgs& a) {
  const int lane = threadIdx.x & 63;
  BatchTiles bt;
  bt.small = a.num_groups <= 64;
  bt.t = lane < a.num_groups ? seq_tiles(a, lane) : 0;
  return bt;
}
// sum over the batch of f(t_b) (f returns 0 for padding lanes' t = -1)
template <typename F>
__device__ __forceinline__ int batch_sum(const MainArgs& a, const BatchTiles& bt, F f) {
  const int lane = threadIdx.x & 63;
  int acc = lane < a.num_groups ? f(bt.t) : 0;
  if (!bt.small) {
    for (int i = 64 + lane; i < a.num_groups; i += 64) acc += f(seq_tiles(a, i));
  }
  return wave_sum_i(acc);
}

__device__ int dense_chunk(const MainArgs& a, const BatchTiles& bt) {
  if (a.fixed_chunk > 0) return a.fixed_chunk;
  const int G = a.num_groups, P = a.split_slots;
  const int tsum = batch_sum(a, bt, [](int t) { return t; });  // the host keeps B x tiles < 2^31
  const int tmax = wave_max_i(bt.small ? bt.t : [&] {
    int m = bt.t;
    for (int i = 64 + (int)(threadIdx.x & 63); i < G; i += 64) m = max(m, seq_tiles(a, i));
    return m;
  }());
  int lo = max(kMinChunkDense, max((tsum + P - 1) / P, (tmax + kMaxSplits - 1) / kMaxSplits));
  // C = ceil(sum t / (P - G)) always fits: sum ceil(t_b / C) <= sum t_b / C + G <= P.
  int hi = P > G ? (tsum + (P - G) - 1) / (P - G) : max(tmax, 1);
  hi = max(hi, lo);
  while (lo < hi) {  // smallest chunk in [lo, hi] whose slots fit
    const int mid = lo + ((hi - lo) >> 1);
    const int need = batch_sum(a, bt, [mid](int t) { return seq_slots(t, mid); });
    if (need <= P) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// The split a dense slot belongs to. group < 0: the slot is unused.
struct DenseSlot {
  int group, split;
  int n_slots;  // slots of the group
};

__device__ DenseSlot dense_slot(const MainArgs& a, const BatchTiles& bt, int chunk, int slot) {
  const int lane = threadIdx.x & 63;
  const int G = a.num_groups;
  DenseSlot r = {-1, 0, 0};
  int base = 0;
  for (int i0 = 0; i0 < G; i0 += 64) {
    const int i = i0 + lane;
    const int t = i0 == 0 ? bt.t : (i < G ? seq_tiles(a, i) : 0);
    const int n = i < G ? seq_slots(t, chunk) : 0;
    int incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    incl += base;
    const int excl = incl - n;
    const uint64_t hit = __ballot(i < G && excl <= slot && slot < incl);
    if (hit != 0ull) {
      const int src = __builtin_ctzll(hit);
      r.group = uniform(__shfl(i, src));
      r.n_slots = uniform(__shfl(n, src));
      r.split = slot - uniform(__shfl(excl, src));
      return r;
    }
    base = uniform(__shfl(incl, 63));
  }
  return r;
}

// Splits holding keys for a dense group of t tiles over n slots: every slot
// gets at least one tile when there are enough, and split s of `active` covers
// tiles [s*t/active, (s+1)*t/active), so lengths differ by at most one tile.
__device__ __forceinline__ int dense_active(int t, int n) { return t > 0 ? min(t, n) : 0; }
__device__ __forceinline__ int dense_tile_bound(int s, int t, int active) {
  return active > 0 ? (int)(((int64_t)s * t) / active) : 0;
}

// ---------------------------------------------------------------------------
// Split kernel: one workgroup = (row block, split, query group).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
mla_split_kernel(MainArgs a) {
  constexpr bool kSparseMode = MODE == kSparse || MODE == kSparsePaged;
  constexpr bool kPagedMode = MODE == kPaged || MODE == kSparsePaged;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLdsBytes + 16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int half = lane >> 5;  // which 16-key half of the 32x32 accumulator a lane holds
  const int l32 = lane & 31;

  // Block -> (row block, split, query group). Sparse: bid = rb*(S*G) + split*G +
  // group, uniform splits. Dense: bid = rb*slots + slot, the slot decoded by the
  // device plan. Workgroups are dealt to the 8 XCDs round-robin, so when the
  // stride (S*G or slots) is a multiple of 8, as in the long single-sequence
  // case, all row blocks of one KV chunk share one XCD's L2. (Padding other
  // strides to a multiple of 8 measured slower for short sequences.)
  const int bid = blockIdx.x;
  int rb, split, group, n_active, t_begin, t_end;
  int64_t rec_slot;  // workspace record of (rb, split, group), before the wave index
  if (kSparseMode) {
    const int sg = a.num_splits * a.num_groups;
    rb = bid / sg;
    const int rem = bid - rb * sg;
    split = rem / a.num_groups;
    group = rem - split * a.num_groups;
    const int chunk = a.chunk_tiles;
    const int n_tiles = group_info(a, group, true).n_tiles;
    n_active = min(a.num_splits, (n_tiles + chunk - 1) / chunk);
    t_begin = split * chunk;
    t_end = min(t_begin + chunk, n_tiles);
    rec_slot = ((int64_t)split * a.num_groups + group) * a.row_blocks + rb;
  } else {
    rb = bid / a.slot_stride;
    const int slot = bid - rb * a.slot_stride;
    if (slot >= a.split_slots) return;
    int n_slots;
    if (a.num_groups == 1) {
      // One sequence: all slots are its splits (no search).
      group = 0;
      split = slot;
      n_slots = a.split_slots;
    } else {
      const BatchTiles bt = batch_tiles(a);
      const DenseSlot ds = dense_slot(a, bt, dense_chunk(a, bt), slot);
      if (ds.group < 0) return;  // slot left over by the plan
      group = ds.group;
      split = ds.split;
      n_slots = ds.n_slots;
    }
    const int n_tiles = group_info(a, group, false).n_tiles;
    n_active = dense_active(n_tiles, n_slots);
    t_begin = dense_tile_bound(split, n_tiles, n_active);
    t_end = split < n_active ? dense_tile_bound(split + 1, n_tiles, n_active) : t_begin;
    if (a.num_groups > 1 && split == 0 && rb == 0 && threadIdx.x == 0 && a.ws_meta != nullptr)
      a.ws_meta[group] = make_int2(slot, n_active);  // the combine's map to this group's records
    rec_slot = (int64_t)slot * a.row_blocks + rb;
  }
  // One split holding all of a group's keys writes out/lse itself.
  const bool direct = a.final_out != 0 || n_active <= 1;

  const GroupInfo gi = group_info(a, group, kSparseMode);
  const int b = gi.b;
  const int kv_len = gi.kv_len;

  const int row0 = rb * kRowsPerBlock + wave * kRowsPerWave;
  const bool wave_active = row0 < a.rows_per_group;
  const int row = row0 + l32;
  const bool row_valid = row < a.rows_per_group;
  const int64_t qrow = (int64_t)group * a.rows_per_group + row;

  if (t_begin >= t_end) {
    // No keys for this group at all: empty softmax (a trailing empty split of a
    // group with keys elsewhere writes nothing; the combine skips it).
    if (direct && split == 0 && row_valid) {
      uint2 z = {0u, 0u};
      for (int d = 4 * half; d < kDL; d += 8)
        *reinterpret_cast<uint2*>(a.out + qrow * kDL + d) = z;
      if (half == 0) a.lse[qrow] = -__builtin_inff();
    }
    return;
  }

  // ---- per-lane LDS read offsets ------------------------------------------
  // The swizzle XORs chunk-index bits that lie below a key row's base offset,
  // so every fragment offset is one per-lane base XOR a compile-time constant.
  // S^T operand (K rows): key = kb*32 + l32, logical 16-byte chunk 2c + half:
  //   offset = (l32*1024 + 16*(half ^ swz(l32))) ^ (32*(c%8)) + 256*(c/8) + kb*32768.
  const int xlat = half ^ swz_lat(l32);
  const int yrope = half ^ swz_rope(l32);
  const unsigned kbaseA = (unsigned)(l32 * 1024 + 16 * xlat);
  // V^T operand through the transposing read: within each 16-lane group G,
  // lane i addresses key (base + i/4) and 4 dims starting at 4*(i%4); the
  // hardware hands lane i the 4 keys of dim i. Two reads (keys +0 and +8) make
  // one 8-key operand: offset = vbase[second] ^ (64*(db%4)) + 256*(db/4) + 16384*kc.
  unsigned vbase[2];
  {
    const int G = lane >> 4, i = lane & 15, h = lane >> 5;
    const int u = 2 * (G & 1) + ((i & 3) >> 1);
#pragma unroll
    for (int second = 0; second < 2; ++second) {
      const int key = 8 * second + 4 * h + (i >> 2);
      vbase[second] = (unsigned)(key * 1024 + 16 * (u ^ swz_lat(key)) + 8 * (i & 1));
    }
  }

  // ---- tile loads ------------------------------------------------------------
  // Wave w issues loads w + 4*i: i < 16 -> one latent key row (key w + 4i, lane =
  // stored chunk), i = 16, 17 -> rope rows of keys 8j .. 8j+7 with j = w, w + 4.
  // Byte offset, within a key row, of the logical chunk stored at slot `lane`:
  auto lat_chunk_off = [&](int key) -> unsigned { return (unsigned)((lane ^ swz_lat(key & 15)) * 16); };
  const unsigned rope_chunk_off =
      (unsigned)(((lane & 7) ^ swz_rope(8 * wave + (lane >> 3))) * 16);  // same for j = w + 4

  const int64_t seq_row0 = kPagedMode ? 0 : (int64_t)b * a.kv_seq_stride;

  // Sparse: lane k holds the physical row of key k of a tile (-1 = absent).
  auto fetch_index = [&](int tile) -> int {
    const int k = tile * kTile + lane;
    return k < a.topk ? a.indices[(int64_t)group * a.topk + k] : -1;
  };
  auto resolve_row = [&](int idx) -> int {
    if (idx < 0 || idx >= kv_len) return -1;
    if (!kPagedMode) return idx;
    const int page = a.page_table[(int64_t)b * a.max_pages + idx / a.page_size];
    if (page < 0) return -1;
    const int64_t r = (int64_t)page * a.page_size + idx % a.page_size;
    return r < a.kv_rows ? (int)r : -1;
  };

  // A tile's 18 loads of this wave (16 latent key rows, 2 x 8 rope rows),
  // prepared once and issued one at a time: spread over the first score chain,
  // they keep the vector-memory issue from stalling the wave. Sparse gathers
  // are non-temporal: a gathered row feeds one workgroup, whereas a dense tile
  // is read by every row block of its chunk through the same L2.
  struct TileLoad {
    __amdgpu_buffer_rsrc_t rl, rr;
    uint8_t* dst;
    int rows;         // sparse: lane k holds key k's physical row (-1 = absent)
    unsigned lane16;  // dense: 16 * lane, an opaque per-tile copy (see score_chain)
  };
  // Dense: returns the number of leading keys of the tile that exist in `nv`.
  // A tile past the split (`tile` >= t_end) loads nothing: its loads read as
  // out of range and only zero-fill the free stage.
  auto prepare_dense = [&](int tile, int stage, int& nv) -> TileLoad {
    const int pos = tile * kTile;
    nv = tile < t_end ? min(kTile, kv_len - pos) : 0;
    int64_t rbase = 0;
    if (nv > 0) {
      if (kPagedMode) {
        const int page = a.page_table[(int64_t)b * a.max_pages + pos / a.page_size];
        rbase = (int64_t)page * a.page_size + pos % a.page_size;
        if (page < 0 || rbase >= a.kv_rows) {
          nv = 0;
          rbase = 0;
        } else if (rbase + nv > a.kv_rows) {
          nv = (int)(a.kv_rows - rbase);
        }
      } else {
        rbase = seq_row0 + pos;
      }
    } else {
      nv = 0;
    }
    TileLoad tl;
    tl.rl = make_rsrc(a.c_kv + rbase * kDL, (uint32_t)nv * 1024u);
    tl.rr = make_rsrc(a.k_rope + rbase * kDR, (uint32_t)nv * 128u);
    tl.dst = smem + stage * kStageBytes;
    tl.rows = 0;
    tl.lane16 = (unsigned)lane * 16u;
    asm volatile("" : "+v"(tl.lane16));
    return tl;
  };
  // Sparse: (the host limits sparse extents to 2^21 rows, so byte offsets stay below 2^31)
  const int64_t sparse_rows = kPagedMode ? a.kv_rows : (int64_t)kv_len;
  auto prepare_sparse = [&](int rows, int stage) -> TileLoad {
    TileLoad tl;
    tl.rl = make_rsrc(a.c_kv + seq_row0 * kDL, (uint32_t)(sparse_rows * 1024));
    tl.rr = make_rsrc(a.k_rope + seq_row0 * kDR, (uint32_t)(sparse_rows * 128));
    tl.dst = smem + stage * kStageBytes;
    tl.rows = rows;
    tl.lane16 = 0;
    return tl;
  };
  auto load_one = [&](const TileLoad& tl, int i) {
    if (i < 16) {
      const int key = wave + 4 * i;
      unsigned off;
      if (kSparseMode) {
        const int r = __builtin_amdgcn_readlane(tl.rows, key);
        off = r >= 0 ? (unsigned)r * 1024u + lat_chunk_off(key) : kOobOffset;
      } else {
        off = (tl.lane16 ^ (unsigned)(16 * swz_lat(key & 15))) + (unsigned)key * 1024u;
      }
      buffer_to_lds<kSparseMode>(tl.rl, tl.dst + key * 1024, off);
    } else {
      const int j = wave + 4 * (i - 16);
      unsigned off;
      if (kSparseMode) {
        const int r = __shfl(tl.rows, 8 * j + (lane >> 3));
        off = r >= 0 ? (unsigned)r * 128u + rope_chunk_off : kOobOffset;
      } else {
        off = (unsigned)j * 1024u + (unsigned)((lane >> 3) * 128) + rope_chunk_off;
      }
      buffer_to_lds<kSparseMode>(tl.rr, tl.dst + kLatBytes + j * 1024, off);
    }
  };
  constexpr int kLoadsPerWave = 18;

  // The first tile of the split (re-issued by a second pass). Dense: issued
  // with the query rows' DMA when they fit in stage 1, else right after the
  // rows are read out of LDS. (Sparse issues it in the pass loop: holding its
  // index state across the query rows costs the gather loop spilled registers.)
  int nv_cur = 0, nv_next = 0;
  uint64_t vm_cur = 0, vm_next = 0;
  int idx_next = -1;
  // Sparse: the first tile's indices, fetched before the query rows' DMA so
  // that their round trip overlaps it (a second pass fetches them again).
  int idx_first = kSparseMode ? fetch_index(t_begin) : -1;
  auto issue_first_tile = [&]() {
    TileLoad tl0;
    nv_next = 0;
    vm_next = 0;
    if (kSparseMode) {
      const int r0 = resolve_row(idx_first);
      vm_cur = __ballot(r0 >= 0);
      tl0 = prepare_sparse(r0, 0);
      idx_next = t_begin + 1 < t_end ? fetch_index(t_begin + 1) : -1;
    } else {
      tl0 = prepare_dense(t_begin, 0, nv_cur);
    }
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; ++i) load_one(tl0, i);
  };
  // ---- query rows: HBM -> LDS by DMA, then into registers ------------------
  // Register q[c] of lane (row l32, half h) holds 16-byte chunk 2c + h of the
  // row's 1,152 bytes (chunks 0..63: latent, 64..71: rope): the B operand of
  // S^T = K Q^T. Loaded straight into that layout, every load instruction
  // touches 32 rows, 32 bytes each, and the wave's 36 loads take twice as long
  // to go through the memory path as the same bytes read a whole 1 KiB row per
  // instruction. So each wave DMAs its 32 rows into LDS, one row (or 8 rope
  // rows) per instruction, and reads its fragments from there. In LDS a latent
  // row r holds chunk k at slot k ^ (r & 15), a rope row r at slot
  // k ^ ((r >> 1) & 7), which makes the 16-byte reads of 16 rows' same chunk
  // conflict-free. Rows past the group's end read as zero (they are never
  // written out). A row block of at most 64 rows (two waves) stages its rows in
  // stage 1 while the first tile streams into stage 0; a larger one needs both
  // stages, so its first tile waits until every wave holds its rows.
  const bool q_in_stage1 = a.rows_per_group - rb * kRowsPerBlock <= 2 * kRowsPerWave;
  uint8_t* const q_lds = smem + (q_in_stage1 ? kStageBytes : 0) + wave * kQWaveBytes;
  if (!kSparseMode && q_in_stage1) issue_first_tile();
  if (wave_active) {
    const int nrows = min(kRowsPerWave, a.rows_per_group - row0);
    const int64_t qbase = (int64_t)group * a.rows_per_group + row0;
    const auto ql = make_rsrc(a.q_lat + qbase * kDL, (uint32_t)nrows * 1024u);
    const auto qr = make_rsrc(a.q_rope + qbase * kDR, (uint32_t)nrows * 128u);
#pragma unroll
    for (int c = 0; c < kRowsPerWave; ++c)
      buffer_to_lds(ql, q_lds + c * 1024, (unsigned)(c * 1024 + 16 * (lane ^ (c & 15))));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 8 * j + (lane >> 3);
      buffer_to_lds(qr, q_lds + kQLatBytes + j * 1024,
                    (unsigned)(r * 128 + 16 * ((lane & 7) ^ ((r >> 1) & 7))));
    }
  }
  bf16x8 q[36];
  auto read_query = [&](bool after_gather) {
    // the rows' DMA landed (after a first gather, whose 18 loads and index
    // prefetch went out later, only the rows' own: those loads may stay in flight)
    if (after_gather) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else __builtin_amdgcn_s_waitcnt(0);
    if (wave_active) {
      // chunk 2c + h of latent row r sits at r*1024 + 16*((2c + h) ^ (r & 15)) =
      // (lb ^ 32*(c % 8)) + 256*(c / 8), lb = r*1024 + 16*(h ^ (r & 15)); rope
      // chunk 2j + h at rb ^ 32j, rb = 32768 + r*128 + 16*(h ^ ((r >> 1) & 7)).
      // Built here from the lane index counted anew (v_mbcnt, in an asm block
      // the compiler cannot move), so the 36 offsets are computed at the reads
      // instead of being hoisted (with their bases, or the lane index) to the
      // prologue and spilled.
      unsigned ln;
      asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
      const unsigned r = ln & 31u, h = ln >> 5;
      const unsigned lb = r * 1024u + 16u * (h ^ (r & 15u));
      const unsigned rbq = (unsigned)kQLatBytes + r * 128u + 16u * (h ^ ((r >> 1) & 7u));
#pragma unroll
      for (int c = 0; c < 36; ++c) {
        const unsigned off = c < 32 ? (lb ^ (unsigned)(32 * (c & 7))) + (unsigned)(256 * (c >> 3))
                                    : rbq ^ (unsigned)(32 * (c - 32));
        q[c] = lds_read16(q_lds, off);
      }
    } else {
#pragma unroll
      for (int c = 0; c < 36; ++c) q[c] = bf16x8{};
    }
  };

  // ---- visibility of the T draft keys for this lane's row (dense) ----------
  uint64_t vis = 0;
  const int prefix = kv_len - a.T;
  if (!kSparseMode && row_valid) {
    const int t = row / a.H;
    if (a.tree_mask != nullptr) {
      const uint8_t* mrow = a.tree_mask + ((int64_t)b * a.T + t) * a.T;
      if ((a.T & 15) == 0 && (reinterpret_cast<uintptr_t>(a.tree_mask) & 15) == 0) {
        // rows are 16-byte aligned: one load per 16 drafts
#pragma unroll
        for (int j0 = 0; j0 < 64; j0 += 16) {
          if (j0 < a.T) {
            const uint4 v = *reinterpret_cast<const uint4*>(mrow + j0);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 16; ++j)
              vis |= (uint64_t)(((w[j >> 2] >> (8 * (j & 3))) & 0xffu) != 0u) << (j0 + j);
          }
        }
      } else {
        // 16 independent byte loads per chunk, one wait per chunk
#pragma unroll
        for (int j0 = 0; j0 < 64; j0 += 16) {
          if (j0 < a.T) {
            uint32_t m[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) m[j] = (j0 + j < a.T) ? mrow[j0 + j] : 0u;
#pragma unroll
            for (int j = 0; j < 16; ++j) vis |= (uint64_t)(m[j] != 0u) << (j0 + j);
          }
        }
      }
    } else {
      vis = (t >= 63) ? ~0ull : ((2ull << t) - 1ull);  // chain: drafts 0..t
    }
  }


  // Sparse calls with the rows in stage 1 read them once the first gather is
  // out (in the pass loop); the others now.
  const bool q_after_gather = kSparseMode && q_in_stage1;
  if (!q_after_gather) {
    read_query(false);
    if (!q_in_stage1) {
      __builtin_amdgcn_s_waitcnt(0);  // this wave's reads of both stages are done
      __syncthreads();                // ... and every other wave's
      if (!kSparseMode) issue_first_tile();
    }
  }

  // ---- softmax state ------------------------------------------------------------
  // Exponents are taken against a per-row reference m_ref (log2 units), not a
  // running max: set at the row max of the first half-tile with a visible key,
  // it stays put tile after tile while the accumulators stay in place. A tile
  // whose row sum reaches 2^32 (a score more than ~32 log2 units above m_ref)
  // raises m_ref at the tile's end by the whole number k = ceil(log2 sum), and
  // O and the row sums, that tile's terms included, are scaled by 2^-k: exact
  // in fp32, so the result equals the one the higher reference would have
  // given throughout. Terms stay below 2^96 inside a tile (fp32 safe); a tile
  // beyond that (a jump of more than ~96 log2 units) sends the split to a
  // second pass with the reference at the largest score seen.
  f32x16 o[16];
  float m_ref = -__builtin_inff();   // log2 domain; equal in both lanes of a row
  float m_hi = -__builtin_inff();    // largest score of half-tiles that overflowed
  float l_run = 0.f;                 // this lane's share of the row sum (fp32 terms: the lse)
  float lq_run = 0.f;                // the same sum over the bf16-rounded terms fed to PV
  int* restart_flag = reinterpret_cast<int*>(smem + kLdsBytes);
  const float c2 = a.scale_log2;
  const bf16x2 ones2 = {(__bf16)1.0f, (__bf16)1.0f};

  // Visibility of the tile's 64 keys for this lane's row (bit = key), and of the
  // lane's 16 keys of half `kb` (bit r <-> accumulator register r, which holds
  // key 32kb + 8(r/4) + 4*half + r%4).
  auto tile_visibility = [&](int pos0, int nv, uint64_t vm) -> uint64_t {
    if (kSparseMode) return vm;
    const uint64_t valid = nv >= 64 ? ~0ull : ((1ull << nv) - 1ull);
    const int d = prefix - pos0;  // tile-relative position of draft 0
    const uint64_t pre = d <= 0 ? 0ull : (d >= 64 ? ~0ull : ((1ull << d) - 1ull));
    const uint64_t drafts = d >= 64 ? 0ull : (d >= 0 ? (vis << d) : (d <= -64 ? 0ull : (vis >> -d)));
    return valid & (pre | drafts);
  };
  auto half_bits = [&](uint64_t tv, int kb) -> uint32_t {
    const uint32_t w = (uint32_t)(tv >> (32 * kb + 4 * half));
    return (w & 0xFu) | ((w >> 4) & 0xF0u) | ((w >> 8) & 0xF00u) | ((w >> 12) & 0xF000u);
  };
  // Row max (log2 units) of a half's raw scores (masked ones are -inf), both lanes of the row.
  auto half_row_max = [&](const f32x16& s) -> float {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx *= c2;
    return fmaxf(mx, __shfl_xor(mx, 32));
  };
  // Score chain of half `kb` (keys 32kb .. 32kb+31) with a VALU slice `work(c)`
  // placed after each of its 36 MFMAs; K fragments are read one step ahead.
  auto score_chain = [&](const uint8_t* sb, int kb, auto&& work) -> f32x16 {
    // opaque copy: keeps the compiler from hoisting the 8 XORed offsets into registers
    unsigned kbase = kbaseA;
    asm volatile("" : "+v"(kbase));
    auto k_off = [&](int c) -> unsigned {
      return c < 32 ? (kbase ^ (unsigned)(32 * (c & 7))) + (unsigned)((c >> 3) * 256 + kb * 32 * 1024)
                    : (unsigned)(kLatBytes + (l32 + 32 * kb) * 128 + (((2 * (c - 32)) ^ yrope) * 16));
    };
    f32x16 acc;
    bf16x8 kf[kFragAhead];
#pragma unroll
    for (int j = 0; j < kFragAhead; ++j) kf[j] = lds_read16(sb, k_off(j));
#pragma unroll
    for (int c = 0; c < 36; ++c) {
      if (c == 0) acc = mfma32_v_first(kf[0], q[0]);
      else mfma32_v_acc(acc, kf[c % kFragAhead], q[c]);
      if (c + kFragAhead < 36) kf[c % kFragAhead] = lds_read16(sb, k_off(c + kFragAhead));
      work(c);
      __builtin_amdgcn_sched_barrier(0);
    }
    score_fence(acc);
    return acc;
  };
  // One slice of the softmax of a half, placed after one MFMA. Each slot holds
  // independent operations on different terms (scale term k, exp2 of term
  // k-1, add term k-2 to the sum; later, pack pair j to bf16 and add pair j-1
  // to the rounded sum), so no slot waits on a transcendental or conversion
  // result. Every result is tied to its slot by an empty asm: without the tie
  // the compiler sinks the whole softmax of S_a past the masking branches into
  // the PV block, where it runs with no MFMA to overlap.
  auto pin = [](auto& x) { asm volatile("" : "+v"(x)); };
  uint32_t packed_prev = 0;  // the halves' softmaxes run one after the other, never interleaved
  auto softmax_step = [&](int k, f32x16& s, float m_use, float& psum, float& qsum,
                          bf16x8* pk) {
    if (k < 16) {
      float x = __builtin_fmaf(s[k], c2, -m_use);
      pin(x);
      s[k] = x;
    }
    if (k >= 1 && k <= 16) {
      float p = fast_exp2(s[k - 1]);
      pin(p);
      s[k - 1] = p;
    }
    if (k >= 2 && k <= 17) {
      psum += s[k - 2];
      pin(psum);
    }
    if (k >= 18 && k < 26) {  // the pair packed in the previous slot
      qsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed_prev), ones2, qsum, false);
      pin(qsum);
    }
    if (k >= 17 && k < 25) {
      const int j = k - 17;
      uint32_t u = pack_bf16x2(s[2 * j], s[2 * j + 1]);
      pin(u);
      u32x4 w = __builtin_bit_cast(u32x4, pk[j >> 2]);
      w[j & 3] = u;
      pk[j >> 2] = __builtin_bit_cast(bf16x8, w);
      packed_prev = u;
    }
  };
  auto init_reference = [&](const f32x16& s) {
    if (__ballot(m_ref == -__builtin_inff()) != 0ull) {
      const float mx = half_row_max(s);
      m_ref = m_ref == -__builtin_inff() ? mx : m_ref;
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) o[d] = f32x16{};
    l_run = 0.f;
    lq_run = 0.f;
    bool overflow = false;

    if (kSparseMode && pass > 0) idx_first = fetch_index(t_begin);
    if (kSparseMode || pass > 0) issue_first_tile();  // stage 0 is free: a pass ends on a barrier
    if (q_after_gather && pass == 0) read_query(true);
    if (threadIdx.x == 0) *restart_flag = 0;

    for (int tile = t_begin; tile < t_end; ++tile) {
      const int stage = (tile - t_begin) & 1;
      // The next tile's loads (past the split's end: none that touch memory).
      // Dense: their descriptors depend only on the tile index, so they are built
      // before the wait, off the path from the barrier to the first MFMA.
      TileLoad nl;
      if (!kSparseMode) nl = prepare_dense(tile + 1, stage ^ 1, nv_next);
      __builtin_amdgcn_s_waitcnt(0);  // this wave's loads (tile data, prefetched indices) landed
      __syncthreads();                // ... and every other wave's; previous stage is free
      if (kSparseMode) {
        const int r1 = tile + 1 < t_end ? resolve_row(idx_next) : -1;
        vm_next = __ballot(r1 >= 0);
        nl = prepare_sparse(r1, stage ^ 1);
        if (tile + 2 < t_end) idx_next = fetch_index(tile + 2);
      }
      if (!wave_active) {
#pragma unroll
        for (int i = 0; i < kLoadsPerWave; ++i) load_one(nl, i);
      }

      if (wave_active) {
        const uint8_t* sb = smem + stage * kStageBytes;
        const int pos0 = tile * kTile;
        // Tiles holding absent or invisible keys (sequence tail, draft keys,
        // sparse gaps) set those raw scores to -inf (scale > 0 keeps them -inf).
        const bool masked = kSparseMode ? (vm_cur != ~0ull)
                                        : (nv_cur < kTile || pos0 + kTile > prefix);
        auto apply_mask = [&](f32x16& sc, int kb) {
          if (masked) {
            const uint32_t bits = half_bits(tile_visibility(pos0, nv_cur, vm_cur), kb);
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = ((bits >> r) & 1u) ? sc[r] : -__builtin_inff();
          }
        };
        float psa = 0.f, qsa = 0.f, psb = 0.f, qsb = 0.f;
        bf16x8 pk[4];

        // One stream of 136 LDS operand fragments per tile: 36 K fragments of
        // keys 0..31 (S_a), 36 of keys 32..63 (S_b), then 64 V^T fragments (PV,
        // step = 16-key chunk kc x 32-dim block db). Each is read kFragAhead
        // steps before its MFMA, across the chain boundaries too, so no chain
        // starts on an LDS round trip. The VALU work is written between the
        // MFMAs: the next tile's loads in S_a, S_a's softmax in S_b, S_b's in PV.
        unsigned kbase = kbaseA, vb0 = vbase[0], vb1 = vbase[1];
        asm volatile("" : "+v"(vb0), "+v"(vb1));  // see score_chain
        // Dense: the 8 XOR variants of the K base are hoisted into registers, so
        // K fragment reads need no address arithmetic; the sparse modes keep them
        // opaque (hoisting costs them spills).
        if constexpr (kSparseMode) asm volatile("" : "+v"(kbase));
        auto frag = [&](int f) -> bf16x8 {
          if (f < 72) {
            const int kb = f / 36, c = f % 36;
            const unsigned off =
                c < 32 ? (kbase ^ (unsigned)(32 * (c & 7))) + (unsigned)((c >> 3) * 256 + kb * 32 * 1024)
                       : (unsigned)(kLatBytes + (l32 + 32 * kb) * 128 + (((2 * (c - 32)) ^ yrope) * 16));
            return lds_read16(sb, off);
          }
          const int step = f - 72, kc = step >> 4, db = step & 15;
          const unsigned hi = (unsigned)((db >> 2) * 256 + kc * 16384);
          const bf16x4 v0 = lds_read_tr(sb, (vb0 ^ (unsigned)(64 * (db & 3))) + hi);
          const bf16x4 v1 = lds_read_tr(sb, (vb1 ^ (unsigned)(64 * (db & 3))) + hi);
          return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
        };
        bf16x8 ring[kFragAhead];
#pragma unroll
        for (int j = 0; j < kFragAhead; ++j) ring[j] = frag(j);
        // Dense: both reads go out before the first MFMA (left alone, the scheduler
        // issues the second after it, exposing a second LDS round trip per tile).
        // The sparse modes keep the scheduler's order: the pin costs them spills.
        if constexpr (!kSparseMode) __builtin_amdgcn_sched_barrier(0);
        // S_a: scores of keys 0..31
        f32x16 sa;
#pragma unroll
        for (int f = 0; f < 36; ++f) {
          if (f == 0) sa = mfma32_v_first(ring[0], q[0]);
          else mfma32_v_acc(sa, ring[f % kFragAhead], q[f]);
          ring[f % kFragAhead] = frag(f + kFragAhead);
          if ((f & 1) == 0 && (f >> 1) < kLoadsPerWave) load_one(nl, f >> 1);
          __builtin_amdgcn_sched_barrier(0);
        }
        score_fence(sa);
        apply_mask(sa, 0);
        init_reference(sa);
        const float mu_a = m_ref == -__builtin_inff() ? 0.f : m_ref;
        // S_b: scores of keys 32..63, S_a's softmax on the VALU
        f32x16 sbk;
#pragma unroll
        for (int f = 36; f < 72; ++f) {
          if (f == 36) sbk = mfma32_v_first(ring[f % kFragAhead], q[0]);
          else mfma32_v_acc(sbk, ring[f % kFragAhead], q[f - 36]);
          ring[f % kFragAhead] = frag(f + kFragAhead);
          softmax_step(f - 36, sa, mu_a, psa, qsa, pk);
          __builtin_amdgcn_sched_barrier(0);
        }
        score_fence(sbk);
        apply_mask(sbk, 1);
        init_reference(sbk);
        const float mu_b = m_ref == -__builtin_inff() ? 0.f : m_ref;
        // PV: O^T += V^T P^T, S_b's softmax on the VALU
#pragma unroll
        for (int f = 72; f < 136; ++f) {
          const int step = f - 72;
          o[step & 15] = mfma32(ring[f % kFragAhead], pk[step >> 4], o[step & 15]);
          if (f + kFragAhead < 136) ring[f % kFragAhead] = frag(f + kFragAhead);
          if (step < 32) softmax_step(step, sbk, mu_b, psb, qsb, pk + 2);
          __builtin_amdgcn_sched_barrier(0);
        }
        l_run += psa + psb;
        lq_run += qsa + qsb;

        // -- rare: the tile's row sum reached 2^kRaiseLog2: raise the reference --
        const float tsum = psa + psb;
        if (__ballot(!(tsum < __builtin_ldexpf(1.0f, (int)kRaiseLog2))) != 0ull) {
          const float row_sum = tsum + __shfl_xor(tsum, 32);
          // k = ceil(log2(row sum)) whole powers of two (0 for rows that stay)
          const int k = row_sum >= __builtin_ldexpf(1.0f, (int)kRaiseLog2) && row_sum < __builtin_inff()
                            ? __builtin_amdgcn_frexp_expf(row_sum) : 0;
          const float f = __builtin_ldexpf(1.0f, -k);
          // register by register in place (a plain vector multiply makes the
          // compiler move the whole accumulator file out of the AGPRs, and spill);
          // first the wait states between the tile's last MFMA and AGPR reads of
          // its result, which the compiler cannot see inside the asm
          asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
          for (int d = 0; d < 16; ++d) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
              float x = o[d][e];
              float tmp;
              asm volatile(
                  "v_accvgpr_read_b32 %1, %0\n\t"
                  "v_mul_f32 %1, %1, %2\n\t"
                  "v_accvgpr_write_b32 %0, %1"
                  : "+a"(x), "=&v"(tmp)
                  : "v"(f));
              o[d][e] = x;
            }
          }
          l_run *= f;
          lq_run *= f;
          m_ref += (float)k;
        }

        // -- rarer: a tile jumped past 2^kRerunLog2; find its largest scores --------
        const float rerun_at = __builtin_ldexpf(1.0f, (int)kRerunLog2);
        const bool ovf = !(psa < rerun_at) || !(psb < rerun_at);
        if (__ballot(ovf) != 0ull) {
          f32x16 ra = score_chain(sb, 0, [](int) {});
          apply_mask(ra, 0);
          m_hi = fmaxf(m_hi, half_row_max(ra));
          f32x16 rb = score_chain(sb, 1, [](int) {});
          apply_mask(rb, 1);
          m_hi = fmaxf(m_hi, half_row_max(rb));
          overflow = true;
        }
      }
      nv_cur = nv_next;
      vm_cur = vm_next;
    }

    // Run the split again only if some row of the workgroup overflowed.
    if (overflow) *restart_flag = 1;
    __syncthreads();
    const bool again = pass == 0 && *restart_flag != 0;
    __syncthreads();
    if (!again) break;
    m_ref = fmaxf(m_ref, m_hi);
  }

  if (!wave_active) return;

  // ---- epilogue ------------------------------------------------------------------
  const float l_row = l_run + __shfl_xor(l_run, 32);
  const float lq_row = lq_run + __shfl_xor(lq_run, 32);
  const bool live = l_row > 0.f;
  const float inv = live && lq_row > 0.f ? 1.0f / lq_row : 0.f;
  const float lse2 = live ? m_ref + fast_log2(l_row) : -__builtin_inff();
  if (direct) {
    if (row_valid) {
      uint16_t* dst = a.out + qrow * kDL;
#pragma unroll
      for (int db = 0; db < 16; ++db) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int d = db * 32 + 8 * qq + 4 * half;
          uint2 pkd;
          pkd.x = pack_bf16x2(o[db][4 * qq + 0] * inv, o[db][4 * qq + 1] * inv);
          pkd.y = pack_bf16x2(o[db][4 * qq + 2] * inv, o[db][4 * qq + 3] * inv);
          *reinterpret_cast<uint2*>(dst + d) = pkd;
        }
      }
      if (half == 0) a.lse[qrow] = live ? lse2 * kLn2 : -__builtin_inff();
    }
  } else {
    const int64_t rec = rec_slot * kWaves + wave;
    // fp16 with a per-row power-of-two scale keeps 11 significant bits of the
    // normalised partial (|o| <= the largest value-row entry) at half the bytes.
    // The partials are written through the caches (sc0 sc1 stores): every
    // workgroup writes its 128 KB at the same moment and only the combine, a
    // later kernel, reads them, so they should neither take L2 lines nor be
    // left dirty there for the kernel's end.
    float amax = 0.f;
#pragma unroll
    for (int db = 0; db < 16; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[db][r]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32)) * inv;
    // scale = 2^(e-15) with amax < 2^e, so |o / scale| < 2^15 fits fp16
    const float scale = amax > 0.f ? __builtin_ldexpf(1.0f, __builtin_amdgcn_frexp_expf(amax) - 15) : 1.0f;
    const float inv_s = inv / scale;
    const __amdgpu_buffer_rsrc_t prs = make_rsrc(a.ws_o + rec * kRecElems, (uint32_t)(kRecElems * 2));
#pragma unroll
    for (int db = 0; db < 16; ++db) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const u32x2 pkd = {scale_pack_f16x2(o[db][4 * qq + 0], o[db][4 * qq + 1], inv_s),
                           scale_pack_f16x2(o[db][4 * qq + 2], o[db][4 * qq + 3], inv_s)};
        buffer_store_b64_wt(pkd, prs, (unsigned)(((db * 4 + qq) * 64 + lane) * 8));
      }
    }
    if (half == 0) {
      float* st = a.ws_lse + rec * (kRecRowStats * kRowsPerWave) + l32;
      st[0] = lse2;
      st[kRowsPerWave] = live && lq_row > 0.f ? m_ref + fast_log2(lq_row) : -__builtin_inff();
      st[2 * kRowsPerWave] = scale;
    }
  }
}

// ---------------------------------------------------------------------------
// Combine kernel: lse = log2 sum_s 2^{lse_s}; out = sum_s w_s o_s with
// w_s = 2^{lq_s} / sum_s' 2^{lq_s'}, where lq_s is split s's log2-sum of the
// rounded terms its partial was normalised by (an exact convex combination of
// the accumulated terms) and lse_s the same from fp32 terms.
// Block = one 32-dim block of one wave record (32 rows x 32 dims). Each thread
// first issues the loads of up to 32 splits' partials, the block turns the
// (row, split) statistics into unnormalised weights in LDS meanwhile, and the
// row's 1 / sum of weights scales the accumulated output once.
// ---------------------------------------------------------------------------
static_assert(16 * 256 * 4 == kRecElems, "16 combine blocks of 256 threads x 4 dims cover one wave record");

// The combine of one block; KBATCH (8, 16, 24, 32) is the number of splits whose
// loads are issued together, chosen from the planned count n_plan so that a
// block with few splits issues no loads it does not use. The loads are clamped
// to the planned splits (whose records exist) and issued before the actual
// count n_active <= n_plan, which depends on kv_lens, is used: the kv_lens
// round trip overlaps the workspace loads. A block whose group ended up with
// one split (written out by the split kernel itself) returns after the loads.
template <int KBATCH>
__device__ __forceinline__ bool combine_rows(const MainArgs& a, float (*wts)[kMaxSplits + 1],
                                             float (*red)[8][kRowsPerWave], float* row_lse,
                                             float* row_inv, int rb, int group, int wave, int db,
                                             int n_plan, int n_active, int64_t rec0, int64_t rec_stride,
                                             bool go) {
  constexpr int kBatch = KBATCH;
  const int t = threadIdx.x;
  const int64_t st_step = rec_stride * (kRecRowStats * kRowsPerWave);

  // Loads are issued statistics first, then the first kBatch splits' partials
  // (4 dims of one row per thread): loads complete in issue order, so the
  // weights are formed while the partials stream in (with at most kBatch
  // splits there is no other round trip).
  const int lane = t & 63, qq = t >> 6, half = lane >> 5, l32 = lane & 31;
  const int r = t & 31, sl = t >> 5;  // phase 1: 8 split lanes per row
  const float* st = a.ws_lse + rec0 * (kRecRowStats * kRowsPerWave) + r;
  // The first kBatch splits' statistics stay in registers (one load each).
  // Every load is issued unconditionally (past the last split it re-reads that
  // split, and the value is not used): straight-line loads let the compiler
  // wait for the statistics alone before phase 1 while the partials are still
  // in flight, where branches around each load made it wait for nearly all.
  constexpr int kHeld = kBatch / 8;
  float h_le[kHeld], h_lq[kHeld], h_sc[kHeld];
#pragma unroll
  for (int i = 0; i < kHeld; ++i) {
    const int s = sl + 8 * i;
    const int sc = min(s, n_plan - 1);
    const float le = st[sc * st_step], lq = st[sc * st_step + kRowsPerWave];
    const float sf = st[sc * st_step + 2 * kRowsPerWave];
    const bool v = s < n_active;
    h_le[i] = v ? le : -__builtin_inff();
    h_lq[i] = v ? lq : -__builtin_inff();
    h_sc[i] = v ? sf : 0.f;
  }
  // The partials are read once: non-temporal loads keep them out of the caches.
  const uint16_t* o_p = a.ws_o + rec0 * kRecElems + ((db * 4 + qq) * 64 + lane) * 4;
  const int64_t o_step = rec_stride * kRecElems;
  auto load_partial = [&](int s) -> uint2 {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(o_p + s * o_step));
    return uint2{v.x, v.y};
  };
  uint2 raw[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) raw[j] = load_partial(min(j, n_plan - 1));
  if (!go || n_active < 1) return false;  // (block-uniform)

  // ---- phase 1: per-row maxima, sums and weights (thread = row x split lane) ----
  {
    float mx = -__builtin_inff(), mxq = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
      mx = fmaxf(mx, h_le[i]);
      mxq = fmaxf(mxq, h_lq[i]);
    }
    for (int s = sl + kBatch; s < n_active; s += 8) {
      mx = fmaxf(mx, st[s * st_step]);
      mxq = fmaxf(mxq, st[s * st_step + kRowsPerWave]);
    }
    red[0][sl][r] = mx;
    red[1][sl][r] = mxq;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mx = fmaxf(mx, red[0][j][r]);
      mxq = fmaxf(mxq, red[1][j][r]);
    }
    __syncthreads();
    float es = 0.f, ws = 0.f;
#pragma unroll
    for (int i = 0; i < kHeld; ++i) {
      const int s = sl + 8 * i;
      if (s < n_active) {
        const float w = h_lq[i] == -__builtin_inff() ? 0.f : fast_exp2(h_lq[i] - mxq);
        es += h_le[i] == -__builtin_inff() ? 0.f : fast_exp2(h_le[i] - mx);
        ws += w;
        wts[r][s] = w * h_sc[i];
      }
    }
    for (int s = sl + kBatch; s < n_active; s += 8) {
      const float le = st[s * st_step], lq = st[s * st_step + kRowsPerWave];
      const float w = lq == -__builtin_inff() ? 0.f : fast_exp2(lq - mxq);
      es += le == -__builtin_inff() ? 0.f : fast_exp2(le - mx);
      ws += w;
      wts[r][s] = w * st[s * st_step + 2 * kRowsPerWave];
    }
    red[0][sl][r] = es;
    red[1][sl][r] = ws;
    __syncthreads();
    es = 0.f;
    ws = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      es += red[0][j][r];
      ws += red[1][j][r];
    }
    if (sl == 0) row_inv[r] = ws > 0.f ? 1.0f / ws : 0.f;
    if (sl == 0)
      row_lse[r] = (mx != -__builtin_inff() && es > 0.f) ? (mx + fast_log2(es)) * kLn2 : -__builtin_inff();
    __syncthreads();
  }

  // ---- phase 2: out = sum_s w_s o_s for 4 dims per thread -------------------------
  const int row = rb * kRowsPerBlock + wave * kRowsPerWave + l32;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < n_active; s0 += kBatch) {
    if (s0 > 0) {
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        raw[j] = s0 + j < n_active ? load_partial(s0 + j) : uint2{0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < n_active) {
        const float w = wts[l32][s0 + j];
        acc[0] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].x & 0xffffu));
        acc[1] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].x >> 16));
        acc[2] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].y & 0xffffu));
        acc[3] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].y >> 16));
      }
    }
  }
  if (row >= a.rows_per_group) return true;
  const float inv = row_inv[l32];
  acc[0] *= inv;
  acc[1] *= inv;
  acc[2] *= inv;
  acc[3] *= inv;
  const int64_t qrow = (int64_t)group * a.rows_per_group + row;
  const int d = db * 32 + 8 * qq + 4 * half;
  uint2 pkd;
  pkd.x = pack_bf16x2(acc[0], acc[1]);
  pkd.y = pack_bf16x2(acc[2], acc[3]);
  *reinterpret_cast<uint2*>(a.out + qrow * kDL + d) = pkd;
  if (db == 0 && qq == 0 && half == 0) a.lse[qrow] = row_lse[l32];
  return true;
}

// The splits planned for a group (their records exist) and those holding keys,
// and where its records of one (row block, wave) start and step (shared by the
// combine kernels). Sparse calls and single sequences know their records
// without reading memory; only the count holding keys of a single sequence
// depends on kv_lens. Several sequences read their record map first.
template <bool kSparseMode>
__device__ __forceinline__ void group_records(const MainArgs& a, int group, int rb, int wave,
                                              int& n_plan, int& n_active, int64_t& rec0,
                                              int64_t& rec_stride) {
  if (kSparseMode) {
    const int n_tiles = (a.topk + kTile - 1) / kTile;
    n_active = min(a.num_splits, (n_tiles + a.chunk_tiles - 1) / a.chunk_tiles);
    n_plan = n_active;
    rec0 = ((int64_t)group * a.row_blocks + rb) * kWaves + wave;
    rec_stride = (int64_t)a.num_groups * a.row_blocks * kWaves;
  } else if (a.num_groups == 1) {
    n_plan = a.split_slots;
    n_active = dense_active(group_info(a, group, false).n_tiles, a.split_slots);
    rec0 = (int64_t)rb * kWaves + wave;
    rec_stride = (int64_t)a.row_blocks * kWaves;
  } else {
    const int2 m = a.ws_meta[group];  // written by the split kernel
    n_plan = n_active = m.y;
    rec0 = ((int64_t)m.x * a.row_blocks + rb) * kWaves + wave;
    rec_stride = (int64_t)a.row_blocks * kWaves;
  }
}

// Combine for groups of more than 32 splits (sparse calls and single
// sequences, whose split count is planned on the host), in one launch: block =
// (wave record, 4-dim group g4 = 2 g + h, g = 4 db + qq), i.e. 32 rows x 4
// dims, the 256 contiguous bytes of every split's record that hold them; 512
// threads = 16 split groups x 32 rows. Each thread issues the loads of its
// splits' partials (sg, sg + 16, ...; at most KPT) and statistics before
// anything else, phase 1 turns the statistics into weights in LDS meanwhile,
// each split group accumulates its splits, and the 16 sums meet in LDS: one
// memory round trip in all. (A T=1 decode over a 65,536-key prefix, 205
// splits: 8-dim blocks of 8 split groups took 7.8 us, these 6.5; two launches
// with two round trips each took the call to 39.5 us against 37.6.)
constexpr int kWideThreads = 512;
constexpr int kWideGroups = kWideThreads / 32;  // split groups of 32 rows
template <int KPT>
__device__ __forceinline__ void combine_wide(const MainArgs& a, float (*wts)[kMaxSplits + 1],
                                             float (*red)[16][kRowsPerWave], f32x4 (*gsum)[32],
                                             float* row_lse, float* row_inv, int g4, int rb, int group,
                                             int wave, int n_plan, int n_active, int64_t rec0,
                                             int64_t rec_stride) {
  const int t = threadIdx.x;
  const int sg = t >> 5, l32 = t & 31;
  const int g = g4 >> 1, half = g4 & 1;
  const uint16_t* o_p = a.ws_o + rec0 * kRecElems + (g * 64 + half * 32 + l32) * 4;
  const int64_t o_step = rec_stride * kRecElems;
  uint2 raw[KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    raw[j] = *reinterpret_cast<const uint2*>(o_p + min(sg + kWideGroups * j, n_plan - 1) * o_step);
  // the same splits' statistics, read once (loading them before the partials
  // measured slower)
  const int r = l32, sl = sg;
  const int64_t st_step = rec_stride * (kRecRowStats * kRowsPerWave);
  const float* st = a.ws_lse + rec0 * (kRecRowStats * kRowsPerWave) + r;
  constexpr int KST = KPT;
  float h_le[KST], h_lq[KST], h_sc[KST];
#pragma unroll
  for (int i = 0; i < KST; ++i) {
    const int sc = min(sl + 16 * i, n_plan - 1);
    h_le[i] = st[sc * st_step];
    h_lq[i] = st[sc * st_step + kRowsPerWave];
    h_sc[i] = st[sc * st_step + 2 * kRowsPerWave];
  }
  if (n_active <= 1) return;  // (block-uniform) the split kernel wrote out/lse itself

  // ---- phase 1: per-row maxima, sums and weights ---------------------------------
  float mx = -__builtin_inff(), mxq = -__builtin_inff();
#pragma unroll
  for (int i = 0; i < KST; ++i) {
    if (sl + 16 * i < n_active) {
      mx = fmaxf(mx, h_le[i]);
      mxq = fmaxf(mxq, h_lq[i]);
    }
  }
  red[0][sl][r] = mx;
  red[1][sl][r] = mxq;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    mx = fmaxf(mx, red[0][j][r]);
    mxq = fmaxf(mxq, red[1][j][r]);
  }
  __syncthreads();
  float es = 0.f, ws = 0.f;
#pragma unroll
  for (int i = 0; i < KST; ++i) {
    const int s = sl + 16 * i;
    if (s < n_active) {
      const float w = h_lq[i] == -__builtin_inff() ? 0.f : fast_exp2(h_lq[i] - mxq);
      es += h_le[i] == -__builtin_inff() ? 0.f : fast_exp2(h_le[i] - mx);
      ws += w;
      wts[r][s] = w * h_sc[i];
    }
  }
  red[0][sl][r] = es;
  red[1][sl][r] = ws;
  __syncthreads();
  if (sl == 0) {
    es = 0.f;
    ws = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      es += red[0][j][r];
      ws += red[1][j][r];
    }
    row_inv[r] = ws > 0.f ? 1.0f / ws : 0.f;
    row_lse[r] = (mx != -__builtin_inff() && es > 0.f) ? (mx + fast_log2(es)) * kLn2 : -__builtin_inff();
  }

  // ---- phase 2: this split group's weighted sum of 4 dims of one row -------------
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int s = sg + kWideGroups * j;
    if (s < n_active) {
      const float w = wts[l32][s];
      acc[0] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].x & 0xffffu));
      acc[1] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].x >> 16));
      acc[2] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].y & 0xffffu));
      acc[3] += w * (float)__builtin_bit_cast(_Float16, (uint16_t)(raw[j].y >> 16));
    }
  }
  if (sg > 0) gsum[sg - 1][l32] = acc;
  __syncthreads();
  if (sg > 0) return;
#pragma unroll
  for (int j = 0; j < kWideGroups - 1; ++j) acc += gsum[j][l32];
  const int row = rb * kRowsPerBlock + wave * kRowsPerWave + l32;
  if (row >= a.rows_per_group) return;
  const float inv = row_inv[l32];
  const int64_t qrow = (int64_t)group * a.rows_per_group + row;
  const int d = (g >> 2) * 32 + 8 * (g & 3) + 4 * half;
  uint2 pkd;
  pkd.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pkd.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<uint2*>(a.out + qrow * kDL + d) = pkd;
  if (g4 == 0) a.lse[qrow] = row_lse[l32];
}

template <int MODE>
__global__ void __launch_bounds__(kWideThreads) mla_combine_wide_kernel(MainArgs a) {
  constexpr bool kSparseMode = MODE == kSparse || MODE == kSparsePaged;
  __shared__ float wts[kRowsPerWave][kMaxSplits + 1];  // unnormalised weight x fp16 scale
  __shared__ float red[2][16][kRowsPerWave];
  __shared__ f32x4 gsum[kWideGroups - 1][32];
  __shared__ float row_lse[kRowsPerWave];
  __shared__ float row_inv[kRowsPerWave];
  const int bid = blockIdx.x;
  const int g4 = bid & 127;
  const int wrec = bid >> 7;
  const int wave = wrec & 3;
  const int rbg = wrec >> 2;
  const int rb = rbg % a.row_blocks;
  const int group = rbg / a.row_blocks;
  if (rb * kRowsPerBlock + wave * kRowsPerWave >= a.rows_per_group) return;  // padding wave record
  int n_plan, n_active;
  int64_t rec0, rec_stride;
  group_records<kSparseMode>(a, group, rb, wave, n_plan, n_active, rec0, rec_stride);
  static_assert(kWideGroups * 16 >= kMaxSplits, "one batch of loads covers every split");
  if (n_plan <= kWideGroups * 4)
    combine_wide<4>(a, wts, red, gsum, row_lse, row_inv, g4, rb, group, wave, n_plan, n_active, rec0, rec_stride);
  else if (n_plan <= kWideGroups * 8)
    combine_wide<8>(a, wts, red, gsum, row_lse, row_inv, g4, rb, group, wave, n_plan, n_active, rec0, rec_stride);
  else
    combine_wide<16>(a, wts, red, gsum, row_lse, row_inv, g4, rb, group, wave, n_plan, n_active, rec0, rec_stride);
}

template <int MODE>
__global__ void __launch_bounds__(256) mla_combine_kernel(MainArgs a) {
  constexpr bool kSparseMode = MODE == kSparse || MODE == kSparsePaged;
  __shared__ float wts[kRowsPerWave][kMaxSplits + 1];  // unnormalised weight x fp16 scale
  __shared__ float red[3][8][kRowsPerWave];
  __shared__ float row_lse[kRowsPerWave];
  __shared__ float row_inv[kRowsPerWave];  // 1 / sum of the unnormalised weights

  const int bid = blockIdx.x;
  const int db = bid & 15;
  const int wrec = bid >> 4;
  const int wave = wrec & 3;
  const int rbg = wrec >> 2;
  const int rb = rbg % a.row_blocks;
  const int group = rbg / a.row_blocks;
  const int t = threadIdx.x;
  if (rb * kRowsPerBlock + wave * kRowsPerWave >= a.rows_per_group) return;  // padding wave record

  int n_plan, n_active;
  int64_t rec0, rec_stride;  // record of split 0 of this (group, rb, wave); step per split
  group_records<kSparseMode>(a, group, rb, wave, n_plan, n_active, rec0, rec_stride);
  // (n_active <= 1: the split kernel wrote this group's out/lse itself)
  if (n_plan <= 8)
    combine_rows<8>(a, wts, red, row_lse, row_inv, rb, group, wave, db, n_plan, n_active, rec0, rec_stride,
                    n_active > 1);
  else if (n_plan <= 16)
    combine_rows<16>(a, wts, red, row_lse, row_inv, rb, group, wave, db, n_plan, n_active, rec0, rec_stride,
                     n_active > 1);
  else if (n_plan <= 24)
    combine_rows<24>(a, wts, red, row_lse, row_inv, rb, group, wave, db, n_plan, n_active, rec0, rec_stride,
                     n_active > 1);
  else
    combine_rows<32>(a, wts, red, row_lse, row_inv, rb, group, wave, db, n_plan, n_active, rec0, rec_stride,
                     n_active > 1);
}

// ---------------------------------------------------------------------------
template <int MODE>
static hipError_t launch_split(const MainArgs& a, hipStream_t s) {
  constexpr bool kSparseMode = MODE == kSparse || MODE == kSparsePaged;
  const unsigned grid = kSparseMode
                            ? (unsigned)a.row_blocks * (unsigned)a.num_splits * (unsigned)a.num_groups
                            : (unsigned)a.row_blocks * (unsigned)a.slot_stride;
  hipLaunchKernelGGL(mla_split_kernel<MODE>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

template <int MODE>
static hipError_t launch_combine(const MainArgs& a, hipStream_t s) {
  const unsigned grid = (unsigned)a.num_groups * (unsigned)a.row_blocks * kWaves * 16u;
  if (a.wide_combine) {
    hipLaunchKernelGGL(mla_combine_wide_kernel<MODE>, dim3(grid * 8u), dim3(kWideThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(mla_combine_kernel<MODE>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_split_kernel(const MainArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case kContig: return launch_split<kContig>(a, s);
    case kPaged: return launch_split<kPaged>(a, s);
    case kSparse: return launch_split<kSparse>(a, s);
    case kSparsePaged: return launch_split<kSparsePaged>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_combine_kernel(const MainArgs& a, int mode, hipStream_t s) {
  switch (mode) {
    case kContig: return launch_combine<kContig>(a, s);
    case kPaged: return launch_combine<kPaged>(a, s);
    case kSparse: return launch_combine<kSparse>(a, s);
    case kSparsePaged: return launch_combine<kSparsePaged>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace mlav
