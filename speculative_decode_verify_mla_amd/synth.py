"""Seeded synthetic inputs for MLA tree-verify attention.

This module draws inputs only: latent queries and cache rows, draft trees and
their visibility masks, ragged prefix lengths, page tables and sparse index
sets. It holds no attention arithmetic (no scores, no softmax, no weighted
sums), so both the fp64 oracle's tests and the HIP path's tests and benchmark
can take their inputs from here without sharing any of the method's steps.

Shapes follow the pages' MLA geometry: a 512-wide latent (``c_kv``) plus a
64-wide rotary part (``k_rope``) per cached token, shared by every head
("The Shared Memory Ceiling", section "The Broader Context", and section
"The Guard" for the Dl/Dr widths). Values are float32 N(0, 1) rounded to
bfloat16 with round-to-nearest-even; the oracle reads back those exact bf16
values.

Draw order for one workload (seed fixed per workload): structure first
(prefix lengths, tree parents, page permutation, sparse indices), then
``q_lat``, ``q_rope``, ``c_kv``, ``k_rope``.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Union

import numpy as np

DL = 512  # latent width shared by all heads
DR = 64  # rotary width
DK = DL + DR  # key width of the score contraction
PAGE = 64  # tokens per page in the paged workload

# fp32 scale used by every workload: 1/sqrt(128 + 64), the pre-absorption
# head width of an MLA head (nope + rope).
SCALE = float(np.float32(1.0 / math.sqrt(192.0)))


# ---------------------------------------------------------------------------
# bfloat16 encoding (input preparation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 1 << 16) -> np.ndarray:
    """N(0,1) float32 draws rounded to bf16 bits, drawn in row chunks (bounded memory)."""
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0 or shape[0] == 0:
        return np.zeros(shape, dtype=np.uint16)
    out = np.empty(shape, dtype=np.uint16)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = f32_to_bf16_bits(
            rng.standard_normal((r1 - r0,) + shape[1:], dtype=np.float32))
    return out


# ---------------------------------------------------------------------------
# Draft-tree structure
# ---------------------------------------------------------------------------
def random_tree_parents(rng: np.random.Generator, T: int) -> np.ndarray:
    """parent[0] = -1; parent[i] uniform in [-1, i-1]. -1 hangs the node off the prefix."""
    parents = np.full(T, -1, dtype=np.int32)
    for i in range(1, T):
        parents[i] = rng.integers(-1, i)
    return parents


def chain_parents(T: int) -> np.ndarray:
    return np.arange(-1, T - 1, dtype=np.int32)


def tree_visibility(parents: Sequence[int]) -> np.ndarray:
    """u8 [T, T]: entry [i, j] = 1 iff draft j is draft i or one of its ancestors."""
    T = len(parents)
    vis = np.zeros((T, T), dtype=np.uint8)
    for i in range(T):
        j = i
        while j >= 0:
            vis[i, j] = 1
            j = int(parents[j])
    return vis


# ---------------------------------------------------------------------------
# Workload description and generation
# ---------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic verify (or sparse decode) call."""

    name: str
    B: int
    T: int
    H: int
    layout: str  # "contig" | "paged" | "sparse"
    prefix: Union[int, Sequence[int], tuple] = 128  # int, per-sequence list, or ("loguniform", lo, hi)
    tree: str = "random"  # "random" | "chain"
    page_size: int = PAGE
    cache_len: int = 0  # sparse: cache rows per sequence
    topk: int = 0  # sparse: indices per query
    pass_null_mask: bool = False  # chain trees: hand NULL to the kernel (chain is the default)
    paged_sparse: bool = False  # sparse over a paged cache


@dataclasses.dataclass
class Workload:
    spec: Spec
    seed: int
    B: int
    T: int
    H: int
    layout: str
    q_lat: np.ndarray  # u16 [B, T, H, 512]
    q_rope: np.ndarray  # u16 [B, T, H, 64]
    c_kv: np.ndarray  # u16 [rows_materialised, 512]
    k_rope: np.ndarray  # u16 [rows_materialised, 64]
    kv_lens: np.ndarray  # i32 [B]
    kv_rows: int  # physical rows of the cache on the device
    kv_seq_stride: int  # contiguous / sparse: rows between sequences
    max_kv_len: int
    scale: float
    parents: Optional[np.ndarray] = None  # i32 [B, T]
    tree_mask: Optional[np.ndarray] = None  # u8 [B, T, T]
    page_table: Optional[np.ndarray] = None  # i32 [B, max_pages]
    page_size: int = 0
    indices: Optional[np.ndarray] = None  # i32 [B, T, K]
    topk: int = 0
    # Sparse workloads materialise only the cache rows some index selects:
    # row_ids[i] is the physical row that c_kv[i] / k_rope[i] hold. Every other
    # physical row is never read by the method; devices fill it with NaN.
    row_ids: Optional[np.ndarray] = None  # i64 [rows_materialised] or None (= arange)
    poison_rows: Optional[np.ndarray] = None  # physical rows that hold NaN (paged tail slots)

    @property
    def mask_for_kernel(self) -> Optional[np.ndarray]:
        if self.spec.pass_null_mask:
            return None
        return self.tree_mask

    def dense_rows(self):
        """(c_kv, k_rope) as full [kv_rows, ...] u16 arrays (only for materialised-dense layouts)."""
        if self.row_ids is None:
            return self.c_kv, self.k_rope
        c = np.full((self.kv_rows, DL), 0x7FC0, dtype=np.uint16)
        k = np.full((self.kv_rows, DR), 0x7FC0, dtype=np.uint16)
        c[self.row_ids] = self.c_kv
        k[self.row_ids] = self.k_rope
        return c, k


def _prefix_lengths(rng: np.random.Generator, spec: Spec) -> np.ndarray:
    p = spec.prefix
    if isinstance(p, tuple) and len(p) == 3 and p[0] == "loguniform":
        lo, hi = float(p[1]), float(p[2])
        u = rng.uniform(math.log(lo), math.log(hi), size=spec.B)
        return np.maximum(np.floor(np.exp(u)), lo).astype(np.int64)
    if isinstance(p, (list, tuple, np.ndarray)):
        arr = np.asarray(p, dtype=np.int64)
        assert arr.shape == (spec.B,)
        return arr
    return np.full(spec.B, int(p), dtype=np.int64)


def generate(spec: Spec, seed: int, poison: bool = False) -> Workload:
    """Draw one workload. ``poison`` puts NaN in cache rows the method must never read."""
    rng = np.random.default_rng(seed)
    B, T, H = spec.B, spec.T, spec.H
    assert 1 <= T <= 64 and B >= 1 and H >= 1

    if spec.layout == "sparse":
        return _generate_sparse(rng, spec, seed, poison)

    # -- structure -----------------------------------------------------------
    prefix = _prefix_lengths(rng, spec)
    kv_lens = (prefix + T).astype(np.int32)
    if spec.tree == "chain":
        parents = np.stack([chain_parents(T) for _ in range(B)])
    else:
        parents = np.stack([random_tree_parents(rng, T) for _ in range(B)])
    tree_mask = np.stack([tree_visibility(parents[b]) for b in range(B)]).astype(np.uint8)

    page_table = None
    page_size = 0
    poison_rows = None
    if spec.layout == "paged":
        page_size = spec.page_size
        n_pages = [(int(n) + page_size - 1) // page_size for n in kv_lens]
        pool = int(sum(n_pages))
        perm = rng.permutation(pool).astype(np.int32)
        max_pages = max(n_pages)
        page_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        tails = []
        for b in range(B):
            page_table[b, : n_pages[b]] = perm[off: off + n_pages[b]]
            off += n_pages[b]
            last = int(page_table[b, n_pages[b] - 1])
            used = int(kv_lens[b]) - (n_pages[b] - 1) * page_size
            tails.extend(range(last * page_size + used, (last + 1) * page_size))
        kv_rows = pool * page_size
        kv_seq_stride = 0
        poison_rows = np.asarray(tails, dtype=np.int64)
    else:
        kv_seq_stride = int(kv_lens.max())
        kv_rows = B * kv_seq_stride
        # rows past a sequence's length (ragged batches) are never read
        tails = [b * kv_seq_stride + r for b in range(B) for r in range(int(kv_lens[b]), kv_seq_stride)]
        poison_rows = np.asarray(tails, dtype=np.int64)

    # -- values --------------------------------------------------------------
    q_lat = normal_bf16(rng, (B, T, H, DL))
    q_rope = normal_bf16(rng, (B, T, H, DR))
    c_kv = normal_bf16(rng, (kv_rows, DL))
    k_rope = normal_bf16(rng, (kv_rows, DR))
    if poison and poison_rows.size:
        c_kv[poison_rows] = 0x7FC0
        k_rope[poison_rows] = 0x7FC0

    return Workload(
        spec=spec, seed=seed, B=B, T=T, H=H, layout=spec.layout,
        q_lat=q_lat, q_rope=q_rope, c_kv=c_kv, k_rope=k_rope,
        kv_lens=kv_lens, kv_rows=kv_rows, kv_seq_stride=kv_seq_stride,
        max_kv_len=int(kv_lens.max()), scale=SCALE,
        parents=parents.astype(np.int32), tree_mask=tree_mask,
        page_table=page_table, page_size=page_size,
        poison_rows=poison_rows if poison else None,
    )


def _generate_sparse(rng: np.random.Generator, spec: Spec, seed: int, poison: bool) -> Workload:
    B, T, H, K, L = spec.B, spec.T, spec.H, spec.topk, spec.cache_len
    assert 1 <= K <= L
    # -- structure: per-(b, t) sorted unique indices in [0, L) ----------------
    indices = np.empty((B, T, K), dtype=np.int32)
    for b in range(B):
        for t in range(T):
            indices[b, t] = np.sort(rng.choice(L, size=K, replace=False)).astype(np.int32)
    kv_lens = np.full(B, L, dtype=np.int32)
    page_table = None
    page_size = 0
    if spec.paged_sparse:
        page_size = spec.page_size
        n_pages = (L + page_size - 1) // page_size
        perm = rng.permutation(B * n_pages).astype(np.int32)
        page_table = perm.reshape(B, n_pages)
        kv_rows = B * n_pages * page_size
        kv_seq_stride = 0

        def phys(b, p):
            return page_table[b, p // page_size].astype(np.int64) * page_size + p % page_size
    else:
        kv_seq_stride = L
        kv_rows = B * L

        def phys(b, p):
            return b * L + p.astype(np.int64)

    # rows some index selects, per sequence, in logical order
    row_ids = []
    for b in range(B):
        sel = np.unique(indices[b].reshape(-1))
        row_ids.append(phys(b, sel))
    row_ids = np.concatenate(row_ids).astype(np.int64)

    # -- values --------------------------------------------------------------
    q_lat = normal_bf16(rng, (B, T, H, DL))
    q_rope = normal_bf16(rng, (B, T, H, DR))
    c_kv = normal_bf16(rng, (row_ids.size, DL))
    k_rope = normal_bf16(rng, (row_ids.size, DR))
    return Workload(
        spec=spec, seed=seed, B=B, T=T, H=H, layout="sparse",
        q_lat=q_lat, q_rope=q_rope, c_kv=c_kv, k_rope=k_rope,
        kv_lens=kv_lens, kv_rows=kv_rows, kv_seq_stride=kv_seq_stride,
        max_kv_len=L, scale=SCALE, indices=indices, topk=K,
        page_table=page_table, page_size=page_size, row_ids=row_ids,
    )


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------
CONFIGS = {
    # tiny chain verify: one CPU-seconds instance
    1: Spec("tiny_chain_h16_l128_t4", B=1, T=4, H=16, layout="contig", prefix=128,
            tree="chain", pass_null_mask=True),
    # Kimi-K2-like verify: 64 heads, 4k prefix, 16-node random tree
    2: Spec("kimi_h64_l4096_t16", B=1, T=16, H=64, layout="contig", prefix=4096),
    # long-prefix verify past any full-score-row kernel's limit
    3: Spec("long_h64_l65536_t16", B=1, T=16, H=64, layout="contig", prefix=65536),
    # batched paged verify, ragged log-uniform prefixes
    4: Spec("paged_b8_h64_t8_loguniform", B=8, T=8, H=64, layout="paged",
            prefix=("loguniform", 1024, 32768)),
    # sparse top-k decode over a 131072-token cache
    5: Spec("sparse_b32_h64_k2048_l131072", B=32, T=1, H=64, layout="sparse",
            cache_len=131072, topk=2048),
    # diagnostic (not one of the five): the long-prefix shape with a single query
    # token, a plain decode step over the 64k latent prefix, bound by reading the cache
    6: Spec("decode_t1_h64_l65536", B=1, T=1, H=64, layout="contig", prefix=65536),
}


def config(i: int, poison: bool = False) -> Workload:
    """Workload ``i`` (1..6), seeded with its own number."""
    return generate(CONFIGS[i], seed=i, poison=poison)


def plant_late_spikes(w: Workload, split_bounds, nats: float = 40.0) -> Workload:
    """Give every query row one key per key range that scores about ``nats``
    above the rest, placed in the last 64-key tile of each range of
    ``split_bounds`` (tile boundaries [t0 = 0 < t1 < ... < tn]): rope dim 0 of
    every query is set to 1 and rope dim 0 of the chosen prefix keys to
    nats / scale (rounded to bf16). Inputs only; a single contiguous sequence."""
    assert w.layout == "contig" and w.B == 1
    w.q_rope[..., 0] = f32_to_bf16_bits(np.ones(w.q_rope[..., 0].shape, np.float32))
    prefix = int(w.kv_lens[0]) - w.T
    big = f32_to_bf16_bits(np.array([nats / w.scale], np.float32))[0]
    keys = []
    for t0, t_end in zip(split_bounds[:-1], split_bounds[1:]):
        # 5 keys into the range's last tile, or its last prefix key when that
        # tile holds draft keys only
        p = min((int(t_end) - 1) * 64 + 5, prefix - 1)
        if int(t0) * 64 <= p < prefix:
            w.k_rope[p, 0] = big
            keys.append(p)
    return w, keys
