"""The oracle: masked softmax attention over an MLA latent cache, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, for sequence b, draft token t and head h
("The Shared Memory Ceiling", section "Technical Deep Dive: Why Shared Memory
Matters": score the query against every visible key, normalise, take the
weighted sum of values; "The Broader Context" for the shared 512-wide MLA
latent):

    visible set V(b, t):
        dense : every prefix position p < P_b = kv_len_b - T, plus draft
                position P_b + j for each draft j that tree_mask[b, t, j]
                marks (a NULL mask means a chain: j <= t)
        sparse: the positions indices[b, t, :] (entries outside [0, kv_len_b)
                select nothing)
    s_p  = scale * (q_lat[b,t,h] . c_kv[row(p)] + q_rope[b,t,h] . k_rope[row(p)])
    m    = max_p s_p,  l = sum_p exp(s_p - m)
    lse  = m + ln l                                (natural log)
    out  = sum_p exp(s_p - m) * c_kv[row(p)] / l   (values are the latent rows)

An empty visible set gives out = 0 and lse = -inf. A key whose physical row
lies outside the cache's [0, kv_rows) (a page-table entry that is negative or
points past the pool) is absent: it leaves the visible set, when kv_rows is
given (the pages say nothing about invalid pages; this is the plain reading of
a row that does not exist).

``attend`` is that definition with one matrix product per side. The same
result, reached through per-tile running max/sum updates ("Technical Deep
Dive", the online-softmax paragraph) or through per-chunk partial results
merged by their log-sum-exp (the split kernel of "The SMEM Ceiling", section
"The Problem Space"), is given by ``attend_streaming`` and ``attend_chunked``;
tests pin both to ``attend``.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

DL = 512
DR = 64


def attend(q_lat: np.ndarray, q_rope: np.ndarray, k_lat: np.ndarray, k_rope: np.ndarray,
           scale: float):
    """One query group against one key set.

    q_lat [H, 512], q_rope [H, 64], k_lat [n, 512], k_rope [n, 64] (float64).
    Returns out [H, 512], lse [H].
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    H = q_lat.shape[0]
    n = k_lat.shape[0]
    if n == 0:
        return np.zeros((H, DL)), np.full(H, -np.inf)
    k_lat = np.asarray(k_lat, dtype=np.float64)
    k_rope = np.asarray(k_rope, dtype=np.float64)
    s = float(scale) * (q_lat @ k_lat.T + q_rope @ k_rope.T)  # [H, n]
    m = s.max(axis=1, keepdims=True)
    w = np.exp(s - m)
    l = w.sum(axis=1)
    out = (w @ k_lat) / l[:, None]
    lse = m[:, 0] + np.log(l)
    return out, lse


def attend_streaming(q_lat, q_rope, k_lat, k_rope, scale: float, tile: int):
    """Same result as ``attend``, visiting the keys tile by tile.

    Keeps a running max m and sum l per head and an unnormalised accumulator;
    when a tile raises the max, the earlier sum and accumulator are scaled by
    exp(m_old - m_new) before the tile's terms are added.
    """
    q_lat = np.asarray(q_lat, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    H = q_lat.shape[0]
    m = np.full(H, -np.inf)
    l = np.zeros(H)
    acc = np.zeros((H, DL))
    for t0 in range(0, k_lat.shape[0], tile):
        kl = np.asarray(k_lat[t0:t0 + tile], dtype=np.float64)
        kr = np.asarray(k_rope[t0:t0 + tile], dtype=np.float64)
        s = float(scale) * (q_lat @ kl.T + q_rope @ kr.T)
        m_new = np.maximum(m, s.max(axis=1))
        alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        p = np.exp(s - m_new[:, None])
        l = alpha * l + p.sum(axis=1)
        acc = alpha[:, None] * acc + p @ kl
        m = m_new
    if not np.isfinite(m).all():
        return np.zeros((H, DL)), np.full(H, -np.inf)
    return acc / l[:, None], m + np.log(l)


def attend_chunked(q_lat, q_rope, k_lat, k_rope, scale: float, bounds):
    """Same result as ``attend``, through split partials and a log-sum-exp merge.

    ``bounds`` lists chunk boundaries [0 = b0 <= b1 <= ... <= bn = n]. Each
    chunk yields (o_s, lse_s) by ``attend``; then
        lse = ln sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) * o_s,
    where an empty chunk (lse_s = -inf) carries weight zero.
    """
    H = np.asarray(q_lat).shape[0]
    parts = []
    for a, b in zip(bounds[:-1], bounds[1:]):
        parts.append(attend(q_lat, q_rope, k_lat[a:b], k_rope[a:b], scale))
    lses = np.stack([p[1] for p in parts])  # [S, H]
    mx = lses.max(axis=0)
    out = np.zeros((H, DL))
    lse = np.full(H, -np.inf)
    live = np.isfinite(mx)
    if live.any():
        w = np.where(np.isneginf(lses[:, live]), 0.0, np.exp(lses[:, live] - mx[live]))
        tot = w.sum(axis=0)
        lse[live] = mx[live] + np.log(tot)
        for s, (o_s, _) in enumerate(parts):
            out[live] += (w[s] / tot)[:, None] * o_s[live]
    return out, lse


def dense_visible_positions(kv_len: int, T: int, t: int, mask_row: Optional[np.ndarray]):
    """Logical key positions token t sees: the prefix plus its marked drafts.

    Draft j sits at position kv_len - T + j. ``mask_row`` is tree_mask[b, t, :]
    (nonzero = visible); None means a chain (drafts 0..t).
    """
    prefix = kv_len - T
    pos = list(range(max(prefix, 0)))
    for j in range(T):
        seen = (j <= t) if mask_row is None else bool(mask_row[j])
        p = prefix + j
        if seen and 0 <= p < kv_len:
            pos.append(p)
    return np.asarray(pos, dtype=np.int64)


class _Rows:
    """Physical-row lookup for caches given in full or as a materialised subset."""

    def __init__(self, c_kv, k_rope, row_ids=None):
        self.c_kv = c_kv
        self.k_rope = k_rope
        if row_ids is None:
            self.order = None
        else:
            row_ids = np.asarray(row_ids, dtype=np.int64)
            self.order = np.argsort(row_ids, kind="stable")
            self.sorted_ids = row_ids[self.order]

    def get(self, phys: np.ndarray):
        phys = np.asarray(phys, dtype=np.int64)
        if self.order is None:
            idx = phys
        else:
            pos = np.searchsorted(self.sorted_ids, phys)
            if phys.size and (np.any(pos >= self.sorted_ids.size)
                              or np.any(self.sorted_ids[np.minimum(pos, self.sorted_ids.size - 1)] != phys)):
                raise KeyError("cache row not materialised")
            idx = self.order[pos]
        return (np.asarray(self.c_kv[idx], dtype=np.float64),
                np.asarray(self.k_rope[idx], dtype=np.float64))


def _physical_rows(b: int, pos: np.ndarray, kv_seq_stride: int, page_table, page_size: int):
    pos = np.asarray(pos, dtype=np.int64)
    if page_table is None:
        return b * int(kv_seq_stride) + pos
    pages = np.asarray(page_table[b], dtype=np.int64)[pos // page_size]
    return pages * page_size + pos % page_size


def _present(rows: np.ndarray, kv_rows):
    """Mask of the physical rows that exist (all of them when kv_rows is None)."""
    if kv_rows is None:
        return np.ones(rows.shape, dtype=bool)
    return (rows >= 0) & (rows < int(kv_rows))


def verify_dense(q_lat, q_rope, c_kv, k_rope, kv_lens, tree_mask, scale: float, *,
                 kv_seq_stride: int = 0, page_table=None, page_size: int = 0, row_ids=None,
                 kv_rows=None):
    """Tree-verify attention for a batch of sequences.

    q_lat [B,T,H,512], q_rope [B,T,H,64] (float64); c_kv [rows,512], k_rope [rows,64];
    kv_lens [B] = prefix + T; tree_mask [B,T,T] or None (chain).
    Contiguous caches place sequence b at rows b*kv_seq_stride + p; paged caches
    place logical position p at page_table[b][p // page_size] * page_size + p % page_size.
    With kv_rows given, keys whose row falls outside [0, kv_rows) are absent.
    Returns out [B,T,H,512], lse [B,T,H].
    """
    B, T, H, _ = q_lat.shape
    rows = _Rows(c_kv, k_rope, row_ids)
    out = np.zeros((B, T, H, DL))
    lse = np.zeros((B, T, H))
    for b in range(B):
        for t in range(T):
            mrow = None if tree_mask is None else tree_mask[b, t]
            pos = dense_visible_positions(int(kv_lens[b]), T, t, mrow)
            phys = _physical_rows(b, pos, kv_seq_stride, page_table, page_size)
            kl, kr = rows.get(phys[_present(phys, kv_rows)])
            out[b, t], lse[b, t] = attend(q_lat[b, t], q_rope[b, t], kl, kr, scale)
    return out, lse


def verify_sparse(q_lat, q_rope, c_kv, k_rope, kv_lens, indices, scale: float, *,
                  kv_seq_stride: int = 0, page_table=None, page_size: int = 0, row_ids=None,
                  kv_rows=None):
    """Sparse top-k attention: query (b, t) sees the positions indices[b, t, :].

    Index entries outside [0, kv_lens[b]) select nothing. All heads of a token
    share its index set. Returns out [B,T,H,512], lse [B,T,H].
    """
    B, T, H, _ = q_lat.shape
    rows = _Rows(c_kv, k_rope, row_ids)
    out = np.zeros((B, T, H, DL))
    lse = np.zeros((B, T, H))
    for b in range(B):
        for t in range(T):
            idx = np.asarray(indices[b, t], dtype=np.int64)
            idx = idx[(idx >= 0) & (idx < int(kv_lens[b]))]
            phys = _physical_rows(b, idx, kv_seq_stride, page_table, page_size)
            kl, kr = rows.get(phys[_present(phys, kv_rows)])
            out[b, t], lse[b, t] = attend(q_lat[b, t], q_rope[b, t], kl, kr, scale)
    return out, lse
